"""Pins for the oracle's LLM.int8() outlier side path (CPU only).

"Low-precision LLM inference", §16 (Mixed-precision Outlier Path): outlier
feature channels take a higher-precision path, the rest the INT8 GEMM, and
the partial outputs are summed.  The oracle reads an outlier channel as an
input column whose largest magnitude reaches tau, quantizes the other
columns per token (outlier columns zeroed), and adds the unquantized
activations of the outlier columns times the dequantized INT8 weight
columns.  Pinned by brute-force detection (numpy), the two limits (no
outliers: the separately pinned W8A8 oracle; every channel an outlier: a
plain numpy product), the decomposition against numpy, a hand-worked tiny
case, and the accuracy claim of the section on synthetic outlier channels.
"""
import numpy as np

from bit_gemm_w4_amd import synth


def _w8(orc, w):
    return orc.act_quant_int8(w, orc.GRAN_ROW)          # per-output-channel INT8 weight


def test_outlier_channels_brute_force(orc):
    w, x = synth.layer(48, 16, 512, "f32", seed=90, x_outlier_cols=8)
    x[:, 7] = 0.0
    x[5, 7] = -6.0                                       # exactly tau: an outlier (>=)
    x[:, 9] = np.clip(x[:, 9], -5.0, 5.0)
    x[3, 9] = np.nextafter(np.float32(6.0), np.float32(0.0))   # just below tau: not one
    for tau in (6.0, 3.0, 1e9, 0.0):
        idx = orc.outlier_channels(x, tau)
        ref = np.flatnonzero(np.abs(x).max(axis=0) >= np.float32(tau)).astype(np.int32)
        assert idx.dtype == np.int32 and np.array_equal(idx, ref)
    idx = orc.outlier_channels(x, 6.0)
    assert 7 in idx and 9 not in idx and len(idx) == 9
    assert len(orc.outlier_channels(x, 0.0)) == 512


def test_no_outliers_is_plain_w8a8(orc):
    w, x = synth.layer(40, 48, 384, "f32", seed=91, x_outlier_cols=8)
    q, sw = _w8(orc, w)
    idx = orc.outlier_channels(x, np.inf)
    assert idx.size == 0
    a, sa = orc.act_quant_int8_outlier(x, idx)
    a0, sa0 = orc.act_quant_int8(x, orc.GRAN_ROW)
    assert np.array_equal(a, a0) and np.array_equal(sa, sa0)
    y = orc.gemm_w8a8_outlier(a, sa, q, sw, x, idx)
    assert orc.rel_l2(y, orc.gemm_w8a8(a0, sa0, orc.GRAN_ROW, q, sw, orc.GRAN_ROW, False)) <= 1e-14


def test_all_outliers_is_the_side_path(orc):
    w, x = synth.layer(24, 32, 256, "f32", seed=92)
    q, sw = _w8(orc, w)
    idx = orc.outlier_channels(x, 0.0)
    a, sa = orc.act_quant_int8_outlier(x, idx)
    assert not a.any() and np.all(sa == 1.0)             # an all-zero row gets scale 1
    y = orc.gemm_w8a8_outlier(a, sa, q, sw, x, idx)
    ref = x.astype(np.float64) @ (q.astype(np.float64) * sw.astype(np.float64)[:, None]).T
    assert orc.rel_l2(y, ref) <= 1e-14


def test_decomposition_against_numpy(orc):
    w, x = synth.layer(33, 40, 640, "f32", seed=93, x_outlier_cols=8)
    q, sw = _w8(orc, w)
    idx = orc.outlier_channels(x, 6.0)
    assert len(idx) == 8
    a, sa = orc.act_quant_int8_outlier(x, idx)
    assert not a[:, idx].any()
    common = np.setdiff1d(np.arange(640), idx)
    a_ref, sa_ref = orc.act_quant_int8(np.ascontiguousarray(x[:, common]), orc.GRAN_ROW)
    assert np.array_equal(a[:, common], a_ref) and np.array_equal(sa, sa_ref)
    y = orc.gemm_w8a8_outlier(a, sa, q, sw, x, idx)
    f = np.float64
    ref = (a.astype(f) @ q.astype(f).T) * sa.astype(f)[:, None] * sw.astype(f)[None, :]
    ref += x[:, idx].astype(f) @ (q[:, idx].astype(f) * sw.astype(f)[:, None]).T
    assert orc.rel_l2(y, ref) <= 1e-14


def test_tiny_hand_worked(orc):
    x = np.array([[0.9, -2.0, 100.0, 0.25]], np.float32)
    idx = orc.outlier_channels(x, 6.0)
    assert list(idx) == [2]
    a, sa = orc.act_quant_int8_outlier(x, idx)
    s = np.float32(2.0) / np.float32(127.0)             # amax of the common columns / 127
    assert sa[0] == s and list(a[0]) == [57, -127, 0, 16]
    q = np.array([[127, -64, 5, 2]], np.int8)
    sw = np.array([0.5], np.float32)
    y = orc.gemm_w8a8_outlier(a, sa, q, sw, x, idx)
    # 57*127 + (-127)(-64) + 16*2 = 15399 from INT8; 100 * (0.5 * 5) from the side path
    assert y[0, 0] == float(s) * 0.5 * 15399 + 250.0


def test_side_path_restores_accuracy(orc):
    """Per-token INT8 of activations with 8 channels x50: the side path removes
    most of the activation error (the weight's own INT8 error remains)."""
    w, x = synth.layer(128, 128, 1024, "f32", seed=94, x_outlier_cols=8)
    q, sw = _w8(orc, w)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    a0, sa0 = orc.act_quant_int8(x, orc.GRAN_ROW)
    plain = orc.gemm_w8a8(a0, sa0, orc.GRAN_ROW, q, sw, orc.GRAN_ROW, False)
    idx = orc.outlier_channels(x, 6.0)
    a, sa = orc.act_quant_int8_outlier(x, idx)
    side = orc.gemm_w8a8_outlier(a, sa, q, sw, x, idx)
    e_plain, e_side = orc.rel_l2(plain, exact), orc.rel_l2(side, exact)
    w_only = orc.rel_l2(x.astype(np.float64) @ (q.astype(np.float64) * sw.astype(np.float64)[:, None]).T, exact)
    assert e_side < 0.35 * e_plain
    assert e_side < 3.0 * w_only
