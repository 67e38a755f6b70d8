"""Pins for the oracle's quantizers and packer (CPU only).

What the pages fix and these tests check, without re-deriving the oracle's
own arithmetic:

* "Low-precision LLM inference", §2 eq. (1)-(2): the code is the rounded
  x/s (+z) clamped to the code range and x^ = s(q - z); hence every element
  inside the range is reproduced within s/2, and the code is the nearest one;
* §3 eq. (3): symmetric s = max|x|/qmax, so the largest magnitude lands on
  code +-qmax;
* §4: one scale per tensor / row / 1x128 group / 128x128 block;
* §5 eq. (4)-(5): 4 + 16/128 = 4.125 bits per weight with FP16 scales;
* §8 "Block scaling": scale = amax / max representable FP8 (448 for E4M3).
"""
from fractions import Fraction

import numpy as np
import pytest

from bit_gemm_w4_amd import synth
from pins import _e4m3_brute_force, np_unpack_w4


def _unpack(orc_pack, N, K):
    qweight, scales, zeros = orc_pack
    return np_unpack_w4(qweight, scales, zeros, N, K)


def _adversarial_weights(N=64, K=512, seed=3):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[0, :128] = 0.0                                   # all-zero group
    w[1, :128] = 0.013                                 # constant positive group
    w[2, :128] = -0.013                                # constant negative group
    w[3, :128] = np.linspace(-1, 1, 128, dtype=np.float32)
    w[4, 128:256] = np.float32(7.0) * np.arange(-64, 64, dtype=np.float32) / 64  # many .5 ties
    w[5, :] *= 1e-30                                   # scales below FP16 normal range
    w[6, :128] = 1e-9                                  # scale underflows FP16 -> clamped
    w[7, ::37] *= 20.0                                 # outlier input channels
    w[8, :128] = np.linspace(0.5, 1.0, 128, dtype=np.float32)    # all-positive group
    w[9, :128] = np.linspace(-1.0, -0.25, 128, dtype=np.float32)  # all-negative group
    return w


@pytest.mark.parametrize("asym", [False, True])
def test_w4_codes_nearest_and_roundtrip(orc, asym):
    w = np.concatenate([_adversarial_weights(), synth.weights(64, 512, seed=5, outlier_frac=0.01)])
    N, K, G = w.shape[0], w.shape[1], 128
    u, s16, z = _unpack(orc.w4_pack(w, G, asym), N, K)
    u = u.astype(np.int64)
    z = z.astype(np.int64)
    s = s16.view(np.float16).astype(np.float64)
    assert np.all(s > 0) and np.all(np.isfinite(s))
    zk = np.repeat(z, G, axis=1)
    sk = np.repeat(s, G, axis=1)
    wd = w.astype(np.float64)
    what = sk * (u - zk)
    err = np.abs(wd - what)
    # nearest code among 0..15 (exact distances in binary64, which hold them exactly)
    cand = sk[..., None] * (np.arange(16)[None, None, :] - zk[..., None])
    best = np.abs(wd[..., None] - cand).min(axis=2)
    # allowed slack: the binary32 division x/s may turn a near-tie into a tie
    assert np.all(err <= best + 2.0 ** -22 * sk + 1e-45)
    inside = (wd / sk + zk >= -0.5) & (wd / sk + zk <= 15.5)
    assert np.all(err[inside] <= sk[inside] / 2 * (1 + 2.0 ** -20))
    if not asym:
        assert u.min() >= 1 and u.max() <= 15                     # code -8 never produced
        assert np.all(err <= sk / 2 * (1 + 2.0 ** -20))           # nothing is clamped
    else:
        # the group range [min(0,w), max(0,w)] spans the 16 codes, so even the
        # clamped extremes stay within one step of the weight
        assert np.all(err <= sk * (1 + 2.0 ** -10))


def test_w4_round_half_to_even(orc):
    """Reading of round(): ties go to the even integer.  A group with amax
    0.875 gets the exact FP16 scale 0.125; elements at odd multiples of 0.0625
    sit exactly halfway between two codes."""
    w = np.zeros((16, 256), np.float32)
    vals = [0.875, 0.0625, 0.1875, 0.3125, 0.4375, 0.5625, 0.6875, 0.8125,
            -0.0625, -0.1875, -0.3125, -0.4375, -0.5625, -0.6875, -0.8125]
    w[0, :len(vals)] = vals
    qweight, s16, _ = orc.w4_pack(w, 128, False)
    assert s16[0, 0, 0] == np.float16(0.125).view(np.uint16)
    u, _, _ = np_unpack_w4(qweight, s16, None, 16, 256)
    codes = [int(c) - 8 for c in u[0, :len(vals)]]
    #        7, 0.5->0, 1.5->2, 2.5->2, 3.5->4, 4.5->4, 5.5->6, 6.5->6, and the negatives
    assert codes == [7, 0, 2, 2, 4, 4, 6, 6, 0, -2, -2, -4, -4, -6, -6]


def test_w4_symmetric_scale_and_extreme_code(orc):
    w = synth.weights(32, 1024, seed=7)
    u_all, s16, _ = _unpack(orc.w4_pack(w, 128, False), 32, 1024)
    s = s16.view(np.float16).astype(np.float64)
    amax = np.abs(w.astype(np.float64)).reshape(32, 8, 128).max(axis=2)
    # s16 is the FP16 value nearest to amax/7 (exact rational comparison on a sample)
    f16 = np.arange(31744, dtype=np.uint16).view(np.float16).astype(np.float64)  # all finite +ve
    for n in range(0, 32, 5):
        for g in range(8):
            target = Fraction(float(amax[n, g])) / 7
            d = abs(Fraction(float(s[n, g])) - target)
            i = np.searchsorted(f16, float(target))
            neigh = [Fraction(float(f16[j])) for j in (i - 1, i, i + 1) if 0 <= j < len(f16)]
            assert d <= min(abs(v - target) for v in neigh)
    u = u_all.astype(np.int64).reshape(32, 8, 128)
    arg = np.abs(w).reshape(32, 8, 128).argmax(axis=2)
    sign = np.sign(np.take_along_axis(w.reshape(32, 8, 128), arg[..., None], 2)[..., 0])
    extreme = np.take_along_axis(u, arg[..., None], 2)[..., 0] - 8
    assert np.array_equal(extreme, (7 * sign).astype(np.int64))


def test_w4_symmetric_idempotent(orc):
    w = synth.weights(16, 512, seed=9, outlier_frac=0.01)
    qweight, s16, _ = orc.w4_pack(w, 128, False)
    what = orc.w4_dequant(qweight, s16, None, 16, 512)
    assert np.array_equal(what.astype(np.float32).astype(np.float64), what)   # exact in binary32
    q2, s2, _ = orc.w4_pack(what.astype(np.float32), 128, False)
    assert np.array_equal(q2, qweight) and np.array_equal(s2, s16)


def test_w4_asym_zero_exact_and_range(orc):
    w = _adversarial_weights()
    N, K = w.shape
    u, _, z = _unpack(orc.w4_pack(w, 128, True), N, K)
    assert u.max() <= 15 and z.max() <= 15
    # a zero weight is represented exactly: its code equals the zero-point
    zk = np.repeat(z, 128, axis=1)
    assert np.array_equal(u[w == 0], zk[w == 0])
    # the group minimum (range widened to include 0) lands on code 0
    for n in range(N):
        for g in range(K // 128):
            grp = w[n, g * 128:(g + 1) * 128]
            if grp.min() < 0:
                assert u[n, g * 128 + int(np.argmin(grp))] == 0


def test_w4_all_zero_group(orc):
    w = np.zeros((16, 256), np.float32)
    for asym in (False, True):
        qweight, s16, zeros = orc.w4_pack(w, 128, asym)
        assert np.all(s16 == 0x3C00)                                  # scale 1.0
        what = orc.w4_dequant(qweight, s16, zeros, 16, 256)
        assert np.all(what == 0.0)


def layout_position(n, k, K):
    """(flat word index, nibble) of weight (n, k) as the packed-format spec states it."""
    t, r, g, c = n // 16, n % 16, k // 128, k % 128
    slot, word, i = 16 * (c // 32) + r, (c % 32) // 8, k % 8
    nibble = i // 2 if i % 2 == 0 else 4 + i // 2
    return ((t * (K // 128) + g) * 64 + slot) * 4 + word, nibble


def test_w4_pack_one_hot(orc):
    """Setting one weight changes exactly one nibble of one word, at the
    position the tiled layout specifies, and nothing else."""
    N, K = 32, 256
    base = np.zeros((N, K), np.float32)
    q0 = orc.w4_pack(base, 128, False)[0].reshape(-1)
    for n, k in [(0, 0), (1, 7), (2, 8), (3, 255), (2, 130), (1, 3), (0, 4), (17, 33), (31, 100), (16, 127)]:
        w = base.copy()
        w[n, k] = 0.5
        q = orc.w4_pack(w, 128, False)[0].reshape(-1)
        widx, nib = layout_position(n, k, K)
        assert np.flatnonzero(q != q0).tolist() == [widx]
        changed = int(q[widx]) ^ int(q0[widx])
        assert changed != 0 and changed & ~(0xF << (4 * nib)) == 0
        assert (int(q[widx]) >> (4 * nib)) & 0xF == 15                 # +7 + 8


def test_w4_scale_zero_layout(orc):
    """Scale of (n, g) at [n/16][g][n%16]; zero-point byte at [n/16][g/2][n%16]."""
    N, K = 32, 512
    w = np.zeros((N, K), np.float32)
    w[19, 256:384] = np.linspace(-0.05, 0.1, 128)   # group 2 of row 19: z = 5
    w[19, 384:512] = np.linspace(-0.1, 0.05, 128)   # group 3: z = 10
    _, scales, zeros = orc.w4_pack(w, 128, True)
    assert scales.shape == (2, 4, 16) and zeros.shape == (2, 2, 16)
    assert zeros[1, 1, 3] == 0xA5
    assert np.count_nonzero(scales != 0x3C00) == 2
    assert scales[1, 2, 3] != 0x3C00 and scales[1, 3, 3] != 0x3C00


def test_w4_zero_nibble_order(orc):
    """zero-point byte: low nibble = group 2h, high nibble = group 2h+1."""
    N, K = 16, 512
    w = np.zeros((N, K), np.float32)
    w[0, 0:128] = np.linspace(-0.1, 0.0, 128)        # z = 15 (all <= 0)
    w[0, 128:256] = np.linspace(0.0, 0.1, 128)       # z = 0  (all >= 0)
    w[0, 256:384] = np.linspace(-0.05, 0.1, 128)     # z = 5
    w[0, 384:512] = np.linspace(-0.1, 0.05, 128)     # z = 10
    _, _, zeros = orc.w4_pack(w, 128, True)
    assert zeros[0, :, 0].tolist() == [0x0F, 0xA5]
    assert np.all(zeros[0, :, 1:] == 0)                # other rows: all-zero groups, z = 0


@pytest.mark.parametrize("asym,bits", [(False, 4.125), (True, 4.15625)])
def test_effective_bits(orc, asym, bits):
    """Section 5 of the low-precision page: b + m/G = 4 + 16/128 = 4.125 bits per
    weight (with 4-bit zero-points: + 4/128 = 4.15625)."""
    N, K = 256, 4096
    qweight, s16, zeros = orc.w4_pack(synth.weights(N, K, seed=1), 128, asym)
    nbytes = qweight.nbytes + s16.nbytes + (0 if zeros is None else zeros.nbytes)
    assert nbytes * 8 == bits * N * K


# ------------------------------------------------------ W8A8 quantizers ----

def _unit_view(x: np.ndarray, gran: int):
    """Reshape so that axis -1 enumerates the elements of each scale unit."""
    R, C = x.shape
    if gran == 0:
        return x.reshape(1, R * C)
    if gran == 1:
        return x.reshape(R, C)
    if gran == 2:
        return x.reshape(R * (C // 128), 128)
    return x.reshape(R // 128, 128, C // 128, 128).transpose(0, 2, 1, 3).reshape(-1, 128 * 128)


def _acts(R, C, seed):
    x = synth.activations(R, C, "f32", seed=seed, n_outlier_cols=8)
    x[0, :128] = 0.0
    if R > 1:
        x[1] = 0.0                                       # an all-zero row
    return x


@pytest.mark.parametrize("gran", [0, 1, 2, 3])
def test_int8_quant_properties(orc, gran):
    x = _acts(256, 512, seed=11)
    q, s = orc.act_quant_int8(x, gran)
    xs = _unit_view(x.astype(np.float64), gran)
    qs = _unit_view(q.astype(np.float64), gran)
    svec = (s[:1] if gran == 0 else s.reshape(-1)).astype(np.float64)
    amax = np.abs(xs).max(axis=1)
    if gran == 0:
        assert s[1] == amax[0]                            # the tensor amax is reported
    zero = amax == 0
    assert np.all(svec[zero] == 1.0) and np.all(qs[zero] == 0)
    nz = ~zero
    # s is the binary32 value nearest amax/127: |s*127 - amax| <= half an ulp of s times 127
    ulp = np.spacing(svec[nz].astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(svec[nz] - amax[nz] / 127) <= ulp / 2)
    # the amax element lands on +-127, every element is within s/2 (no clamping occurs)
    assert np.all(np.abs(qs[nz]).max(axis=1) == 127)
    err = np.abs(xs - svec[:, None] * qs)
    assert np.all(err[nz] <= svec[nz, None] / 2 * (1 + 2.0 ** -20))
    assert q.min() >= -127


@pytest.mark.parametrize("gran", [0, 1, 2, 3])
def test_fp8_quant_properties(orc, gran):
    x = _acts(256, 512, seed=12)
    q, s = orc.act_quant_fp8(x, gran)
    xs = _unit_view(x.astype(np.float64), gran)
    qs = _unit_view(q, gran)
    svec = (s[:1] if gran == 0 else s.reshape(-1)).astype(np.float64)
    amax = np.abs(xs).max(axis=1)
    zero = amax == 0
    assert np.all(svec[zero] == 1.0) and np.all((qs[zero] & 0x7F) == 0)
    nz = ~zero
    ulp = np.spacing(svec[nz].astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(svec[nz] - amax[nz] / 448) <= ulp / 2)
    # amax element -> code of magnitude 448 (0x7E); every code is the nearest
    # E4M3 value of x/s (checked against a brute-force search of the table)
    mag = qs & 0x7F
    assert np.all(mag[nz].max(axis=1) == 0x7E)
    dec = orc.e4m3_decode(qs)
    assert not np.isnan(dec).any()
    ratio = (xs.astype(np.float32) / svec.astype(np.float32)[:, None]).astype(np.float32)
    assert np.array_equal(qs[nz], _e4m3_brute_force(ratio[nz]))


def test_quant_scale_layouts(orc):
    """Scale tensor shapes per granularity (section 4 of the low-precision page)."""
    x = _acts(256, 384, seed=13)
    for gran, shape in [(0, (2,)), (1, (256,)), (2, (256, 3)), (3, (2, 3))]:
        _, s = orc.act_quant_int8(x, gran)
        assert s.shape == shape
        _, s = orc.act_quant_fp8(x, gran)
        assert s.shape == shape
    # 1x128 group scale (r, g) covers exactly x[r, 128g:128g+128]
    _, s = orc.act_quant_fp8(x, 2)
    assert s[5, 2] == np.float32(np.abs(x[5, 256:384]).max()) / np.float32(448)
    _, s = orc.act_quant_fp8(x, 3)
    assert s[1, 0] == np.float32(np.abs(x[128:256, 0:128]).max()) / np.float32(448)


def test_quant_underflowing_scale(orc):
    """Reading for a unit whose amax/qmax underflows binary32 to zero: like an
    all-zero unit it gets scale 1 (all codes 0), so no division by zero occurs."""
    x = np.zeros((2, 128), np.float32)
    x[0, 3] = np.float32(1e-44)                   # subnormal; 1e-44/127 == 0
    x[1, 3] = np.float32(1e-40)                   # subnormal; scale stays subnormal, > 0
    q, s = orc.act_quant_int8(x, 1)
    assert s[0] == 1.0 and np.all(q[0] == 0)
    assert 0 < s[1] < 1e-38 and q[1, 3] == 127
    q, s = orc.act_quant_fp8(x, 1)
    assert s[0] == 1.0 and np.all((q[0] & 0x7F) == 0)
    assert q[1, 3] == 0x7E
