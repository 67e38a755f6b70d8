"""Pins for the oracle's number-format codecs (CPU only).

The oracle encodes FP16 scales and FP8 E4M3 codes from the format definitions
("Low-precision LLM inference", §5: FP16 group scales; §7: E4M3 = 1 sign, 4
exponent, 3 mantissa bits, variant to be pinned -- here OCP E4M3FN).  These
tests pin those codecs against independent routines: numpy's and torch's casts
(library routines the oracle does not call) and a brute-force nearest search
over the decoded code table.
"""
import numpy as np
import pytest
import torch

from pins import _e4m3_brute_force, _e4m3_finite_table


def _all_f16_values():
    return np.arange(65536, dtype=np.uint16).view(np.float16)


def test_f16_decode_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = orc.f16_bits_to_f32(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_decode_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = orc.bf16_bits_to_f32(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _f16_rounding_cases():
    """Every finite FP16 value, every midpoint between neighbours (ties), the
    fp32 values one and two ulps either side of each midpoint, values near the
    overflow threshold, and 4M random binary32 bit patterns."""
    v = _all_f16_values().astype(np.float64)
    v = np.unique(v[np.isfinite(v)])
    mids = ((v[1:] + v[:-1]) / 2).astype(np.float32)      # exact in binary32
    assert np.array_equal(mids.astype(np.float64), (v[1:] + v[:-1]) / 2)
    cases = [v.astype(np.float32), mids]
    for d in (1, 2):
        up = mids.copy()
        dn = mids.copy()
        for _ in range(d):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(-np.inf))
        cases += [up, dn]
    cases.append(np.array([65504, 65519.996, 65520, 65536, 1e10, np.inf, -np.inf, 2.0 ** -25,
                           2.0 ** -24 * 1.5, 2.0 ** -26], np.float32))
    rng = np.random.default_rng(0)
    cases.append(rng.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint32).view(np.float32))
    return np.concatenate(cases)


def test_f16_encode_vs_numpy(orc):
    x = _f16_rounding_cases()
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16)
    got = orc.f32_to_f16_bits(x)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got.view(np.float16)), nan)
    assert np.array_equal(got[~nan], ref[~nan].view(np.uint16))


# ------------------------------------------------------------------ E4M3 ----

def test_e4m3_decode_table(orc):
    codes = np.arange(256, dtype=np.uint8)
    got = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # closed forms of the E4M3FN variant
    assert np.flatnonzero(nan).tolist() == [0x7F, 0xFF]
    assert np.nanmax(got) == 448.0 and np.nanmin(got) == -448.0
    assert got[1] == 2.0 ** -9 and got[8] == 2.0 ** -6          # min subnormal, min normal
    assert not np.isinf(got).any()


def _e4m3_rounding_cases():
    vals, _ = _e4m3_finite_table()
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    cases = [vals.astype(np.float32), mids]
    for d in (1, 2, 3):
        up, dn = mids.copy(), mids.copy()
        for _ in range(d):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(-np.inf))
        cases += [up, dn]
    cases.append(np.array([447.99997, 448, 448.00003, 463.99997, 464, 464.00003, 480, 1e30,
                           np.inf, np.nan, 2.0 ** -10, 2.0 ** -10 * 1.0000001, 2.0 ** -11,
                           1e-45, 0.0], np.float32))
    rng = np.random.default_rng(1)
    cases.append(rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint32).view(np.float32))
    cases.append((rng.standard_normal(1 << 20) * 100).astype(np.float32))
    x = np.concatenate(cases)
    return np.concatenate([x, -x])


def test_e4m3_encode_vs_brute_force(orc):
    x = _e4m3_rounding_cases()
    got = orc.e4m3_encode(x)
    ref = _e4m3_brute_force(x)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, (x[bad[:8]], got[bad[:8]], ref[bad[:8]])


@pytest.mark.slow
def test_e4m3_encode_exhaustive_vs_torch(orc):
    """All 2^32 binary32 bit patterns against torch's float8_e4m3fn cast.
    torch rounds to nearest even but does not saturate (>= 464 -> NaN), so its
    input is clamped to +-448 first; NaN passes through the clamp."""
    chunk = 1 << 26
    for start in range(0, 1 << 32, chunk):
        bits = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32)
        x = bits.view(np.float32)
        got = orc.e4m3_encode(x)
        ref = torch.from_numpy(x).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        if not np.array_equal(got, ref):
            bad = np.flatnonzero(got != ref)[:8]
            raise AssertionError((start, x[bad], got[bad], ref[bad]))
