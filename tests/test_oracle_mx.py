"""Pins for the oracle's MXFP8 format and GEMM (CPU only).

"Low-precision LLM inference", §10: the OCP MX specification makes a block of
elements and its shared scale one data format.  The oracle follows OCP MX
v1.0 for MXFP8: 32 consecutive elements share an E8M0 scale 2^(E - 127) with
E = floor(log2 amax) - 8 + 127 (8 = largest E4M3 exponent), and the elements
are saturating RNE E4M3 casts of v / 2^(E - 127).  Pinned against an
independent numpy/torch reading of that rule (frexp for the exponent, torch's
E4M3 cast after clamping to +-448), closed forms, the element error bound,
and the GEMM against numpy and against the (separately pinned) FP8 W8A8
oracle at unit scales.
"""
import numpy as np
import torch

from bit_gemm_w4_amd import synth


def _np_mx(x):
    R, C = x.shape
    xb = x.reshape(R, C // 32, 32).astype(np.float32)
    amax = np.abs(xb).max(axis=2)
    _, ex = np.frexp(amax)                        # amax = f * 2^ex, f in [0.5, 1)
    e = np.where(amax > 0, np.clip(ex - 1 - 8 + 127, 0, 254), 127).astype(np.int64)
    scaled = (xb.astype(np.float64) * np.exp2(127 - e)[:, :, None]).astype(np.float32)
    clamped = torch.from_numpy(np.clip(scaled, -448.0, 448.0))
    q = clamped.to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(R, C)
    return q, e.astype(np.uint8)


def test_mxfp8_quant_vs_independent_reading(orc):
    w, x = synth.layer(64, 16, 1024, "f32", seed=60, x_outlier_cols=8)
    x[3, :32] = 0.0                                # an all-zero block
    x[4, 64:96] *= 1e-30                           # tiny values: exponent clamp region
    x[5, 96:128] = 448.0 * 2.0 ** np.arange(-16, 16)[:32]
    q, e = orc.quant_mxfp8(x)
    qn, en = _np_mx(x)
    assert np.array_equal(e, en)
    assert np.array_equal(q, qn)
    assert e[3, 0] == 127 and not q[3, :32].any()


def test_mxfp8_closed_forms_and_bound(orc):
    x = np.zeros((3, 64), np.float32)
    x[0, :32] = 448.0                              # amax 448: scale 1, codes exact
    x[1, :32] = 1.0                                # amax 1: scale 2^-8, elements 256
    x[2, :32] = np.linspace(-1.0, 1.0, 32)
    q, e = orc.quant_mxfp8(x)
    assert e[0, 0] == 127 and e[1, 0] == 119 and e[0, 1] == 127
    dec = orc.e4m3_decode(q) * np.exp2(np.repeat(e.astype(np.int64), 32, axis=1) - 127)
    assert np.array_equal(dec[0, :32], x[0, :32]) and np.array_equal(dec[1, :32], x[1, :32])
    # error bound: relative 2^-4 for elements in E4M3's normal range below the
    # saturation point; elements that scale past 448 (only a block's largest
    # can, since it maps into [256, 512)) come back as +-448 X
    rng = np.random.default_rng(61)
    v = (rng.standard_normal((32, 256)) * np.exp(rng.uniform(-20, 20, (32, 1)))).astype(np.float32)
    q, e = orc.quant_mxfp8(v)
    X = np.exp2(np.repeat(e.astype(np.int64), 32, axis=1) - 127)
    dec = orc.e4m3_decode(q) * X
    r = np.abs(v) / X
    normal = (r >= 2.0 ** -6) & (r < 448.0)
    assert np.all(np.abs(dec - v)[normal] <= 2.0 ** -4 * np.abs(v)[normal])
    sat = r >= 464.0
    assert sat.any() and np.array_equal(dec[sat], np.sign(v[sat]) * 448.0 * X[sat])
    top = np.abs(v).reshape(32, 8, 32).max(axis=2) / np.exp2(e.astype(np.int64) - 127)
    assert np.all((top >= 256) & (top < 512))


def test_mxfp8_gemm_vs_numpy_and_fp8_oracle(orc):
    M, N, K = 33, 48, 256
    w, x = synth.layer(M, N, K, "f32", seed=62, x_outlier_cols=8)
    a, ea = orc.quant_mxfp8(x)
    q, ew = orc.quant_mxfp8(w)
    y = orc.gemm_mxfp8(a, ea, q, ew)
    def deq(c, e):
        return orc.e4m3_decode(c) * np.exp2(np.repeat(e.astype(np.int64), 32, axis=1) - 127)
    ref = deq(a, ea) @ deq(q, ew).T
    assert orc.rel_l2(y, ref) <= 1e-14
    # all scales 1: the FP8 W8A8 GEMM with unit per-tensor scales, bit for bit
    ones = np.full((M, K // 32), 127, np.uint8)
    onesw = np.full((N, K // 32), 127, np.uint8)
    unit = np.ones(2, np.float32)
    assert np.array_equal(orc.gemm_mxfp8(a, ones, q, onesw), orc.gemm_w8a8(a, unit, 0, q, unit, 0, True))
