"""Pins for the oracle's MXFP8 and MXFP4 formats and GEMMs (CPU only).

"Low-precision LLM inference", §10: the OCP MX specification makes a block of
elements and its shared scale one data format.  The oracle follows OCP MX
v1.0 for MXFP8: 32 consecutive elements share an E8M0 scale 2^(E - 127) with
E = floor(log2 amax) - 8 + 127 (8 = largest E4M3 exponent), and the elements
are saturating RNE E4M3 casts of v / 2^(E - 127).  Pinned against an
independent numpy/torch reading of that rule (frexp for the exponent, torch's
E4M3 cast after clamping to +-448), closed forms, the element error bound,
and the GEMM against numpy and against the (separately pinned) FP8 W8A8
oracle at unit scales.

MXFP4 (same section: E2M1 = 1 sign, 2 exponent, 1 mantissa bit, and MXFP4
as the OCP MX block format of it): the same rule with 2 (the largest E2M1
exponent) in place of 8 and saturating RNE E2M1 elements.  Pinned by the
E2M1 value table of the format definition, a brute-force nearest-value
search with ties to the even mantissa, an independent numpy reading of the
block rule, closed forms, and the GEMM against numpy and against the MXFP8
oracle (every E2M1 value is an E4M3 value, so the two GEMMs must agree bit
for bit on the same scales).
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


# ---- MXFP4 ----

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])     # magnitudes of codes 0..7


def _nearest_e2m1(r):
    """Code of the E2M1 value nearest to r (binary64), ties to the even
    mantissa bit, magnitudes above 6 saturating: a brute-force search."""
    r = np.asarray(r, np.float64)
    a = np.minimum(np.abs(r), 6.0)
    d = np.abs(a[..., None] - E2M1)                               # distance to every magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    even = cand & ((np.arange(8) & 1) == 0)
    pick = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    return (pick | np.where(np.signbit(r), 8, 0)).astype(np.uint8)


def test_e2m1_value_table_and_round_trip(orc):
    codes = np.arange(16, dtype=np.uint8)
    v = orc.e2m1_decode(codes)
    assert np.array_equal(np.abs(v[:8]), E2M1) and np.array_equal(v[8:], -E2M1)
    assert np.signbit(v[8])                                      # code 8 is -0
    assert np.array_equal(orc.e2m1_encode(v.astype(np.float32)), codes)


def test_e2m1_encode_brute_force(orc):
    grid = np.arange(-8 * 256, 8 * 256 + 1, dtype=np.float64) / 256.0   # every tie point lies on it
    rng = np.random.default_rng(63)
    extra = rng.standard_normal(20000) * np.exp(rng.uniform(-6, 4, 20000))
    for v in (grid, extra):
        v32 = v.astype(np.float32)
        assert np.array_equal(orc.e2m1_encode(v32), _nearest_e2m1(v32.astype(np.float64)))
    # the ties, one by one: to the even mantissa (codes 0, 2, 2, 4, 4, 6, 6)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    assert list(orc.e2m1_encode(ties)) == [0, 2, 2, 4, 4, 6, 6]
    assert list(orc.e2m1_encode(-ties)) == [8, 10, 10, 12, 12, 14, 14]
    assert list(orc.e2m1_encode(np.array([6.0, 7.0, 1e30, np.inf], np.float32))) == [7, 7, 7, 7]


def _np_mx4(x):
    R, C = x.shape
    xb = x.reshape(R, C // 32, 32).astype(np.float32)
    amax = np.abs(xb).max(axis=2)
    _, ex = np.frexp(amax)
    e = np.where(amax > 0, np.clip(ex - 1 - 2 + 127, 0, 254), 127).astype(np.int64)
    scaled = (xb.astype(np.float64) * np.exp2(127 - e)[:, :, None]).astype(np.float32)
    codes = _nearest_e2m1(scaled.astype(np.float64)).reshape(R, C)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return q, e.astype(np.uint8)


def test_mxfp4_quant_vs_independent_reading(orc):
    w, x = synth.layer(64, 16, 1024, "f32", seed=64, x_outlier_cols=8)
    x[3, :32] = 0.0                                # an all-zero block
    x[4, 64:96] *= 1e-30                           # tiny values: exponent clamp region
    x[5, 96:128] = 6.0 * 2.0 ** np.arange(-16, 16)[:32]
    x[6, 128:160] = -x[6, 128:160]
    q, e = orc.quant_mxfp4(x)
    qn, en = _np_mx4(x)
    assert q.shape == (64, 512) and e.shape == (64, 32)
    assert np.array_equal(e, en)
    assert np.array_equal(q, qn)
    assert e[3, 0] == 127 and not q[3, :16].any()


def test_mxfp4_closed_forms(orc):
    x = np.zeros((4, 64), np.float32)
    x[0, :32] = 6.0                                # amax 6: scale 1, every element code 7
    x[1, :32] = 1.0                                # amax 2^0: scale 2^-2, elements 4.0 (code 6)
    x[2, :32] = np.linspace(-1.0, 1.0, 32)
    x[3, :32] = 2.0 ** 20 * 5.0                    # a block of ties at 5 X: to 4 X
    q, e = orc.quant_mxfp4(x)
    assert e[0, 0] == 127 and e[1, 0] == 125 and e[0, 1] == 127 and e[3, 0] == 127 + 20
    assert np.all(q[0, :16] == 0x77) and np.all(q[1, :16] == 0x66) and np.all(q[3, :16] == 0x66)
    assert not q[0, 16:].any()
    # a block's largest magnitude always scales into [4, 8); elements are
    # within half a quantum of v / X below 6, and saturate to 6 above it
    rng = np.random.default_rng(65)
    v = (rng.standard_normal((32, 256)) * np.exp(rng.uniform(-20, 20, (32, 1)))).astype(np.float32)
    q, e = orc.quant_mxfp4(v)
    codes = np.empty((32, 256), np.uint8)
    codes[:, 0::2], codes[:, 1::2] = q & 15, q >> 4
    X = np.exp2(np.repeat(e.astype(np.int64), 32, axis=1) - 127)
    r = np.abs(v) / X
    dec = orc.e2m1_decode(codes)
    quantum = np.where(r < 2, 0.5, np.where(r < 4, 1.0, 2.0))
    ok = r <= 6.0
    assert np.all(np.abs(np.abs(dec) - r)[ok] <= quantum[ok] / 2)
    assert np.all(np.abs(dec[~ok]) == 6.0)
    top = r.reshape(32, 8, 32).max(axis=2)
    assert np.all((top >= 4) & (top < 8))


def test_mxfp4_gemm_vs_numpy_and_mxfp8_oracle(orc):
    M, N, K = 33, 48, 256
    w, x = synth.layer(M, N, K, "f32", seed=66, x_outlier_cols=8)
    a, ea = orc.quant_mxfp4(x)
    q, ew = orc.quant_mxfp4(w)
    assert a.shape == (M, K // 2) and q.shape == (N, K // 2)
    y = orc.gemm_mxfp4(a, ea, q, ew)

    def codes(p):
        c = np.empty((p.shape[0], p.shape[1] * 2), np.uint8)
        c[:, 0::2], c[:, 1::2] = p & 15, p >> 4
        return c

    def deq(p, e):
        return orc.e2m1_decode(codes(p)) * np.exp2(np.repeat(e.astype(np.int64), 32, axis=1) - 127)

    ref = deq(a, ea) @ deq(q, ew).T
    assert orc.rel_l2(y, ref) <= 1e-14
    # every E2M1 value is an E4M3 value: the same blocks as MXFP8 elements
    a8 = orc.e4m3_encode(orc.e2m1_decode(codes(a)).astype(np.float32))
    q8 = orc.e4m3_encode(orc.e2m1_decode(codes(q)).astype(np.float32))
    assert np.array_equal(orc.gemm_mxfp8(a8, ea, q8, ew), y)
    # and quantising the dequantised MXFP4 values again gives them back
    a2, ea2 = orc.quant_mxfp4(deq(a, ea).astype(np.float32))
    nz = ea != 127
    assert np.array_equal(a2, a) and np.array_equal(ea2[nz], ea[nz])


def test_mx_infinite_block(orc):
    """floor(log2 inf) is infinite, so a block holding an infinity takes the
    top of the clamp, E = 254: the infinity saturates and the finite
    elements scale to (signed) zero."""
    x = np.zeros((2, 64), np.float32)
    x[0, :32] = np.linspace(-3.0, 3.0, 32)
    x[0, 5] = np.inf
    x[1, 40] = -np.inf
    x[1, 41] = 1e30
    q8, e8 = orc.quant_mxfp8(x)
    q4, e4 = orc.quant_mxfp4(x)
    assert e8[0, 0] == 254 and e4[0, 0] == 254 and e8[1, 1] == 254 and e4[1, 1] == 254
    assert e8[0, 1] == 127 and e4[1, 0] == 127
    assert q8[0, 5] == 0x7E and q8[1, 40] == 0xFE
    c4 = np.empty((2, 64), np.uint8)
    c4[:, 0::2], c4[:, 1::2] = q4 & 15, q4 >> 4
    assert c4[0, 5] == 7 and c4[1, 40] == 15
    others = np.ones(32, bool)
    others[5] = False
    assert np.all(orc.e4m3_decode(q8[0, :32])[others] == 0) and np.all(orc.e2m1_decode(c4[0, :32])[others] == 0)
