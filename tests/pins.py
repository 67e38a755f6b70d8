"""Independent reference routines used by the oracle pins (brute force)."""
import numpy as np


def _e4m3_finite_table():
    """Sorted distinct finite non-negative E4M3 magnitudes and their codes."""
    vals, codes = [], []
    for c in range(0x7F):                                         # 0x00..0x7E
        e, m = c >> 3, c & 7
        v = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        vals.append(v)
        codes.append(c)
    return np.array(vals), np.array(codes, np.uint8)


def _e4m3_brute_force(x: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3 magnitude by searching the table, ties to the even
    code, saturation at 448, NaN -> 0x7F|sign.  Independent of the oracle's
    binade arithmetic."""
    vals, codes = _e4m3_finite_table()
    xd = x.astype(np.float64)
    a = np.abs(xd)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    dlo = np.abs(a - vals[lo])
    dhi = np.abs(vals[hi] - a)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[hi] % 2 == 0))
    out = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    out = np.where(a >= 448.0, np.uint8(0x7E), out)
    sign = np.signbit(x).astype(np.uint8) << 7
    out = out | sign
    out = np.where(np.isnan(x), np.uint8(0x7F) | sign, out)
    return out.astype(np.uint8)
