"""Pins for the oracle's GEMMs (CPU only).

The GEMMs are plain definitions (Y = X W^T on the dequantized operands, in
binary64 / exact integers).  They are pinned against numpy's matmul on operands
that the test dequantizes itself, against exact rational / big-integer brute
force on tiny shapes, and against special cases whose result is known in
closed form (one-hot inputs select a weight row, all-ones inputs give column
sums, unit scales give integer results).

Sources: "Quantization throughput by method" (hrletsgo.me), W4A16 section
(INT4 weights dequantized into a 16-bit GEMM) and W8A8/FP8 section (native
INT8/FP8 GEMM); "Low-precision LLM inference", §22 (INT32 / FP32 accumulators)
and §8 "Block scaling".
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from bit_gemm_w4_amd import synth
from pins import np_unpack_w4


def _np_dequant(qweight, s16, zeros, K, G=128):
    N = qweight.shape[0] * 16
    u, s, z = np_unpack_w4(qweight, s16, zeros, N, K)
    sv = s.view(np.float16).astype(np.float64)
    return np.repeat(sv, G, axis=1) * (u.astype(np.float64) - np.repeat(z.astype(np.float64), G, axis=1))


def _np_acts(bits, dtype):
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("x_dtype,asym", [("f16", False), ("bf16", True), ("bf16", False)])
def test_w4a16_vs_numpy(orc, x_dtype, asym):
    M, N, K = 5, 96, 768
    w, x = synth.layer(M, N, K, x_dtype, seed=21, w_outlier_frac=0.01)
    qweight, s16, zeros = orc.w4_pack(w, 128, asym)
    y = orc.gemm_w4a16(x, x_dtype, qweight, s16, zeros)
    ref = _np_acts(x, x_dtype) @ _np_dequant(qweight, s16, zeros, K).T
    assert orc.rel_l2(y, ref) <= 1e-13
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_w4a16_special_cases(orc):
    N, K = 32, 256
    w = synth.weights(N, K, seed=22)
    qweight, s16, zeros = orc.w4_pack(w, 128, True)
    what = _np_dequant(qweight, s16, zeros, K)
    # one-hot activations select one column of W^, i.e. weight [:, k]
    ks = [0, 1, 127, 128, 255]
    x = np.zeros((len(ks), K), np.float16)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    y = orc.gemm_w4a16(x.view(np.uint16), "f16", qweight, s16, zeros)
    assert np.array_equal(y, what[:, ks].T)
    # all-ones activations give the row sums of W^
    ones = np.ones((1, K), np.float16).view(np.uint16)
    y = orc.gemm_w4a16(ones, "f16", qweight, s16, zeros)
    assert np.allclose(y[0], what.sum(axis=1), rtol=1e-14, atol=1e-15)


def test_w4a16_exact_rational_tiny(orc):
    M, N, K = 2, 16, 256
    w, x = synth.layer(M, N, K, "bf16", seed=23)
    qweight, s16, zeros = orc.w4_pack(w, 128, True)
    y = orc.gemm_w4a16(x, "bf16", qweight, s16, zeros)
    what = _np_dequant(qweight, s16, zeros, K)
    xv = _np_acts(x, "bf16")
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(xv[m, k])) * Fraction(float(what[n, k])) for k in range(K))
            assert abs(Fraction(float(y[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 40) + Fraction(1, 2 ** 60)


def test_i8_acc_big_int_brute_force(orc):
    rng = np.random.default_rng(24)
    M, N, K = 3, 5, 128
    a = rng.integers(-128, 128, size=(M, K), dtype=np.int64).astype(np.int8)
    w = rng.integers(-128, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    a[0, :] = -128
    w[0, :] = -128
    acc = orc.gemm_i8_acc(a, w)
    for m in range(M):
        for n in range(N):
            assert int(acc[m, n]) == sum(int(a[m, k]) * int(w[n, k]) for k in range(K))


def test_i8_acc_vs_numpy_and_overflow(orc):
    rng = np.random.default_rng(25)
    a = rng.integers(-127, 128, size=(33, 1024)).astype(np.int8)
    w = rng.integers(-127, 128, size=(48, 1024)).astype(np.int8)
    acc = orc.gemm_i8_acc(a, w)
    assert np.array_equal(acc, a.astype(np.int64) @ w.astype(np.int64).T)
    # |acc| <= 14336 * 127 * 127 < 2^31 fits; a longer K of saturated codes does not
    big = np.full((1, 140032), 127, np.int8)
    with pytest.raises(OverflowError):
        orc.gemm_i8_acc(big, big)
    ok = np.full((1, 14336), -128, np.int8)
    assert int(orc.gemm_i8_acc(ok, ok)[0, 0]) == 14336 * 128 * 128


def _np_w8a8(a, a_s, a_gran, w, w_s, w_gran, fp8):
    def deq(q, s, gran):
        R, C = q.shape
        v = (torch.from_numpy(q).view(torch.float8_e4m3fn).double().numpy() if fp8
             else q.astype(np.float64))
        if gran == 0:
            return v * float(s[0])
        if gran == 1:
            return v * s.astype(np.float64)[:, None]
        if gran == 2:
            return v * np.repeat(s.astype(np.float64), 128, axis=1)
        return v * np.repeat(np.repeat(s.astype(np.float64), 128, axis=0), 128, axis=1)
    return deq(a, a_s, a_gran) @ deq(w, w_s, w_gran).T


@pytest.mark.parametrize("fp8,a_gran,w_gran", [
    (False, 1, 1), (False, 0, 0), (False, 0, 1), (True, 0, 0), (True, 1, 1), (True, 2, 3)])
def test_w8a8_vs_numpy(orc, fp8, a_gran, w_gran):
    M, N, K = 130, 256, 384
    w, x = synth.layer(M, N, K, "f32", seed=26, x_outlier_cols=8)
    quant = orc.act_quant_fp8 if fp8 else orc.act_quant_int8
    a, a_s = quant(x, a_gran)
    wq, w_s = quant(w, w_gran)
    y = orc.gemm_w8a8(a, a_s, a_gran, wq, w_s, w_gran, fp8)
    ref = _np_w8a8(a, a_s, a_gran, wq, w_s, w_gran, fp8)
    assert orc.rel_l2(y, ref) <= 1e-13
    if not fp8 and a_gran == 1 and w_gran == 1:
        # per-row x per-channel: y = acc * s_a[m] * s_w[n] with the exact INT32 accumulator
        acc = orc.gemm_i8_acc(a, wq).astype(np.float64)
        ref2 = acc * a_s.astype(np.float64)[:, None] * w_s.astype(np.float64)[None, :]
        assert orc.rel_l2(y, ref2) <= 1e-13


def test_w8a8_unit_scales_integer_exact(orc):
    """With every scale 1 the FP8 GEMM is an exact sum of products of E4M3 values."""
    rng = np.random.default_rng(27)
    a = rng.integers(0, 256, size=(4, 256), dtype=np.int64).astype(np.uint8)
    w = rng.integers(0, 256, size=(8, 256), dtype=np.int64).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0                      # no NaN codes
    w[(w & 0x7F) == 0x7F] = 0
    ones = np.ones(2, np.float32)
    y = orc.gemm_w8a8(a, ones, 0, w, ones, 0, True)
    av = orc.e4m3_decode(a)
    wv = orc.e4m3_decode(w)
    for m in range(4):
        for n in range(8):
            exact = sum(Fraction(float(av[m, k])) * Fraction(float(wv[n, k])) for k in range(256))
            assert Fraction(float(y[m, n])) == exact      # all partial sums exact in binary64


# ------------------------------------------------------------------- W4A8 ----
# "Low-precision LLM inference", §1 (W4A8: INT4 weights, INT8 activations,
# INT32/FP32 accumulation) and §14 (per-token activation scales).

def _w4a8_inputs(M, N, K, seed, asym):
    w, x = synth.layer(M, N, K, "f32", seed=seed, w_outlier_frac=0.01, x_outlier_cols=8)
    return w, x


@pytest.mark.parametrize("a_gran,asym", [(1, True), (1, False), (0, True)])
def test_w4a8_vs_numpy(orc, a_gran, asym):
    M, N, K = 37, 80, 768
    w, x = _w4a8_inputs(M, N, K, 28, asym)
    qweight, s16, zeros = orc.w4_pack(w, 128, asym)
    a, a_s = orc.act_quant_int8(x, a_gran)
    y = orc.gemm_w4a8(a, a_s, a_gran, qweight, s16, zeros)
    sa = np.full(M, float(a_s[0])) if a_gran == 0 else a_s.astype(np.float64)
    ref = (a.astype(np.float64) * sa[:, None]) @ _np_dequant(qweight, s16, zeros, K).T
    assert orc.rel_l2(y, ref) <= 1e-13
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_w4a8_unit_scales_integer_exact(orc):
    """Unit scales: Y is the exact integer sum_k a (u - z), i.e. the INT8 GEMM of
    the activation codes against the signed codes u - z."""
    rng = np.random.default_rng(29)
    M, N, K = 9, 32, 512
    u = rng.integers(0, 16, size=(N, K), dtype=np.int64).astype(np.uint8)
    z = rng.integers(0, 16, size=(N, K // 128), dtype=np.int64).astype(np.uint8)
    s16 = np.full((N, K // 128), 0x3C00, np.uint16)                     # FP16 1.0
    qweight, scales, zeros = orc.w4_pack_codes(u, s16, z, True)
    a = rng.integers(-128, 128, size=(M, K), dtype=np.int64).astype(np.int8)
    a[0, :] = -128
    y = orc.gemm_w4a8(a, np.ones(M, np.float32), 1, qweight, scales, zeros)
    signed = (u.astype(np.int64) - np.repeat(z.astype(np.int64), 128, axis=1)).astype(np.int8)
    acc = orc.gemm_i8_acc(a, signed)
    assert np.array_equal(y, acc.astype(np.float64))


def test_w4a8_matches_w4a16_on_representable_activations(orc):
    """With power-of-two activation scales every a * s_a is a BF16 value, and the
    W4A8 layer must equal the W4A16 layer on those activations bit for bit."""
    rng = np.random.default_rng(30)
    M, N, K = 6, 48, 512
    w = synth.weights(N, K, seed=31, outlier_frac=0.01)
    qweight, s16, zeros = orc.w4_pack(w, 128, True)
    a = rng.integers(-127, 128, size=(M, K), dtype=np.int64).astype(np.int8)
    a_s = (2.0 ** rng.integers(-12, 3, size=M)).astype(np.float32)
    y = orc.gemm_w4a8(a, a_s, 1, qweight, s16, zeros)
    xv = torch.from_numpy(a.astype(np.float32) * a_s[:, None]).to(torch.bfloat16)
    assert torch.equal(xv.float(), torch.from_numpy(a.astype(np.float32) * a_s[:, None]))   # exact
    x_bits = xv.view(torch.int16).numpy().view(np.uint16)
    y16 = orc.gemm_w4a16(x_bits, "bf16", qweight, s16, zeros)
    assert np.array_equal(y, y16)


def test_w4a8_exact_rational_tiny(orc):
    M, N, K = 2, 16, 256
    w, x = _w4a8_inputs(M, N, K, 32, True)
    qweight, s16, zeros = orc.w4_pack(w, 128, True)
    a, a_s = orc.act_quant_int8(x, 1)
    y = orc.gemm_w4a8(a, a_s, 1, qweight, s16, zeros)
    what = _np_dequant(qweight, s16, zeros, K)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(int(a[m, k])) * Fraction(float(a_s[m])) * Fraction(float(what[n, k]))
                        for k in range(K))
            assert abs(Fraction(float(y[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 40) + Fraction(1, 2 ** 60)
