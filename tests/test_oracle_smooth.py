"""Pins for the oracle's SmoothQuant fold (CPU only).

"Low-precision LLM inference", §15: Y = X W^T = (X S^-1)(W S)^T with a
diagonal S over the input channels, chosen from calibration statistics and a
smoothing strength and folded into the static weights.  The page gives no
formula for S; the oracle takes the SmoothQuant rule s_j = amax_x[j]^alpha /
amax_w[j]^(1-alpha) (1 where a column maximum is 0).  Pinned against numpy,
closed forms (alpha = 1, 0, 1/2 on powers of four), the balance property of
alpha = 1/2 (both smoothed column maxima equal sqrt(amax_x amax_w)), the
exactness of the fold for power-of-two factors, and the method's purpose:
the fold lowers the INT8 W8A8 error on activations with outlier channels.
"""
import numpy as np
import pytest

from bit_gemm_w4_amd import synth


def test_col_amax_vs_numpy(orc):
    rng = np.random.default_rng(40)
    x = rng.standard_normal((37, 300)).astype(np.float32)
    x[:, 5] = 0.0
    x[3, 7] = -1e30
    x[:, 9] = -0.0
    assert np.array_equal(orc.col_amax(x), np.abs(x).max(axis=0))


def test_smooth_scales_closed_forms(orc):
    ax = np.array([4.0, 16.0, 0.25, 0.0, 3.0, 7.5], np.float32)
    aw = np.array([1.0, 0.0625, 4.0, 2.0, 0.0, 0.5], np.float32)
    # alpha = 1/2 on powers of four: sqrt is exact
    s = orc.smooth_scales(ax, aw, 0.5)
    assert s[0] == 2.0 and s[1] == 16.0 and s[2] == 0.25
    assert s[3] == 1.0 and s[4] == 1.0                     # a zero column maximum
    # alpha = 1: s = amax_x; alpha = 0: s = 1 / amax_w
    s1 = orc.smooth_scales(ax, aw, 1.0)
    assert s1[0] == 4.0 and s1[5] == np.float32(7.5)
    s0 = orc.smooth_scales(ax, aw, 0.0)
    assert s0[2] == 0.25 and s0[5] == 2.0


def test_smooth_scales_balance(orc):
    """alpha = 1/2: max |x_j / s_j| and max |w_j s_j| both equal sqrt(amax_x amax_w)."""
    rng = np.random.default_rng(41)
    ax = np.exp(rng.uniform(-8, 8, 512)).astype(np.float32)
    aw = np.exp(rng.uniform(-8, 2, 512)).astype(np.float32)
    s = orc.smooth_scales(ax, aw, 0.5).astype(np.float64)
    g = np.sqrt(ax.astype(np.float64) * aw.astype(np.float64))
    assert np.allclose(ax / s, g, rtol=2e-7) and np.allclose(aw * s, g, rtol=2e-7)


def test_col_mul_vs_numpy(orc):
    rng = np.random.default_rng(42)
    x = rng.standard_normal((20, 256)).astype(np.float32)
    m = rng.uniform(0.01, 100.0, 256).astype(np.float32)
    assert np.array_equal(orc.col_mul(x, m), x * m[None, :])   # IEEE binary32 products


def test_fold_is_exact_for_power_of_two_factors(orc):
    rng = np.random.default_rng(43)
    w = rng.standard_normal((48, 256)).astype(np.float32)
    x = rng.standard_normal((9, 256)).astype(np.float32)
    s = (2.0 ** rng.integers(-6, 7, 256)).astype(np.float32)
    xs = orc.col_mul(x, (1.0 / s).astype(np.float32)).astype(np.float64)
    ws = orc.col_mul(w, s).astype(np.float64)
    assert np.array_equal(xs * ws[0][None, :], x.astype(np.float64) * w[0].astype(np.float64)[None, :])
    assert np.allclose(xs @ ws.T, x.astype(np.float64) @ w.astype(np.float64).T, rtol=0, atol=1e-12)


def test_fold_lowers_int8_error_on_outlier_channels(orc):
    """8 activation channels x50 (the INT8 prefill recipe): per-token INT8
    activations lose the small channels to the outliers' scale; the fold moves
    that range into the weights and the W8A8 error drops."""
    M, N, K = 64, 128, 512
    w, x = synth.layer(M, N, K, "f32", seed=44, x_outlier_cols=8)
    exact = x.astype(np.float64) @ w.astype(np.float64).T

    def w8a8_err(xq_in, wq_in):
        a, sa = orc.act_quant_int8(xq_in, 1)
        q, sq = orc.act_quant_int8(wq_in, 1)
        return orc.rel_l2(orc.gemm_w8a8(a, sa, 1, q, sq, 1, False), exact)

    base = w8a8_err(x, w)
    s = orc.smooth_scales(orc.col_amax(x), orc.col_amax(w), 0.5)
    smooth = w8a8_err(orc.col_mul(x, (1.0 / s).astype(np.float32)), orc.col_mul(w, s))
    assert smooth < 0.5 * base, (base, smooth)
