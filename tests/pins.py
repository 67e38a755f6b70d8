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


# nibble slot of k = 8j + i inside its word: even i in the low half-word, odd i in the high
NIBBLE_OF = np.array([0, 4, 1, 5, 2, 6, 3, 7], dtype=np.uint32)


def np_unpack_w4(qweight, scales, zeros, N, K):
    """Independent numpy reading of the tiled INT4 layout: qweight
    [N/16][K/128][64 slots][4 words], slot = 16*(c//32) + n%16 for c = k%128,
    word = (c%32)//8; scales [N/16][K/128][16]; zeros [N/16][K/256][16]
    (low nibble even group).  Returns codes u [N][K], scales [N][K/128] (uint16
    bits), zero-points [N][K/128] (8 when zeros is None)."""
    T, G = N // 16, K // 128
    w = np.asarray(qweight, np.uint32).reshape(T, G, 4, 16, 4)          # t g q r kk
    nib = (w[..., None] >> (4 * NIBBLE_OF)) & 0xF                        # t g q r kk i
    u = nib.transpose(0, 3, 1, 2, 4, 5).reshape(N, K).astype(np.uint8)   # (t r)(g q kk i)
    s = np.asarray(scales, np.uint16).reshape(T, G, 16).transpose(0, 2, 1).reshape(N, G)
    if zeros is None:
        z = np.full((N, G), 8, np.uint8)
    else:
        zz = np.asarray(zeros, np.uint8).reshape(T, G // 2, 16)
        z = np.stack([zz & 0xF, zz >> 4], axis=3).transpose(0, 2, 1, 3).reshape(N, G)
    return u, s, z
