"""Plain CPU oracle for the W4A16 / W8A8 quantized linear layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``.  The product package never imports
it, and it never imports the product package: the two share no code.

The arithmetic lives in ``bg_oracle.c`` (plain loops, binary32 where the method
fixes binary32, binary64 / int64 for the GEMMs); this module only compiles it
with gcc, loads it with ctypes and marshals numpy arrays.  Every function
names the passage of the pages it follows in the C source:

* [LPI] "Low-precision LLM inference: FP8/INT8/INT4/FP4 kernels and
  calibration (8/10)", blog.ruahverce.com -- §1 notation table and precision
  manifest (W4A8), §2 eq. (1)-(2), §3 eq. (3), §10 MX block formats, §15
  SmoothQuant fold,
  §4 granularity, §5 effective bits, §7 FP8 formats, §8 FP8 scale recipes,
  §22 accumulator precision.
* [AIB] "Quantization throughput by method: why W4A16 is overtaken by W8A8 as
  batch grows", hrletsgo.me -- the W4A16 and W8A8/FP8 sections.

Parity pins for every function live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bg_oracle.c")
# BG_ORACLE_LIB: an already built copy of bg_oracle.c to load instead (the
# sanitizer test builds one with -fsanitize=address,undefined)
_LIB_OVERRIDE = os.environ.get("BG_ORACLE_LIB")
_LIB = _LIB_OVERRIDE or os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

GRAN_TENSOR, GRAN_ROW, GRAN_ROW_G128, GRAN_BLOCK128 = 0, 1, 2, 3
GRAN_NAMES = {"tensor": GRAN_TENSOR, "row": GRAN_ROW, "row_g128": GRAN_ROW_G128,
              "block128": GRAN_BLOCK128}

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared", "-Wall"]


def build(force: bool = False) -> str:
    """Compile bg_oracle.c into liboracle.so with gcc (no GPU involved)."""
    if _LIB_OVERRIDE:
        return _LIB
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            I = ctypes.c_int
            sig = {
                "orc_f32_to_f16_n": [P, I64, P],
                "orc_f16_to_f32_n": [P, I64, P],
                "orc_bf16_to_f32_n": [P, I64, P],
                "orc_e4m3_encode_n": [P, I64, P],
                "orc_e4m3_decode_n": [P, I64, P],
                "orc_w4_quantize": [P, I64, I64, I, I, P, P, P],
                "orc_w4_pack": [P, P, P, I64, I64, I, P, P, P],
                "orc_w4_unpack": [P, P, P, I64, I64, P, P, P],
                "orc_w4_dequant": [P, P, P, I64, I64, I, P],
                "orc_gemm_w4a16": [P, I, I64, I64, P, P, P, I64, I, P],
                "orc_quant_int8": [P, I64, I64, I, P, P],
                "orc_quant_fp8": [P, I64, I64, I, P, P],
                "orc_gemm_i8_acc": [P, P, I64, I64, I64, P],
                "orc_gemm_w8a8": [P, P, I, P, P, I, I, I64, I64, I64, P],
                "orc_gemm_w4a8": [P, P, I, I64, I64, P, P, P, I64, I, P],
                "orc_col_amax": [P, I64, I64, P],
                "orc_smooth_scales": [P, P, I64, ctypes.c_double, P],
                "orc_col_mul": [P, I64, I64, P, P],
                "orc_quant_mxfp8": [P, I64, I64, P, P],
                "orc_gemm_mxfp8": [P, P, P, P, I64, I64, I64, P],
                "orc_quant_mxfp4": [P, I64, I64, P, P],
                "orc_outlier_channels": [P, I64, I64, ctypes.c_float, P],
                "orc_gemm_w8a8_outlier": [P, P, P, P, P, P, I64, I64, I64, I64, P],
                "orc_gemm_mxfp4": [P, P, P, P, I64, I64, I64, P],
                "orc_e2m1_encode_n": [P, I64, P],
                "orc_e2m1_decode_n": [P, I64, P],
                "orc_num_threads": [],
            }
            for name, argtypes in sig.items():
                fn = getattr(lib, name)
                fn.argtypes = argtypes
                fn.restype = (ctypes.c_int if name in ("orc_gemm_i8_acc", "orc_num_threads")
                              else ctypes.c_int64 if name == "orc_outlier_channels" else None)
            _lib = lib
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- codecs ----

def f32_to_f16_bits(x) -> np.ndarray:
    """binary32 -> binary16 bits, round to nearest even (IEEE 754)."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().orc_f32_to_f16_n(_p(x), x.size, _p(out))
    return out


def f16_bits_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    _load().orc_f16_to_f32_n(_p(h), h.size, _p(out))
    return out


def bf16_bits_to_f32(b) -> np.ndarray:
    b = _c(b, np.uint16)
    out = np.empty(b.shape, np.float32)
    _load().orc_bf16_to_f32_n(_p(b), b.size, _p(out))
    return out


def bits_to_f32(bits, dtype: str) -> np.ndarray:
    """Exact binary32 value of FP16 ('f16') or BF16 ('bf16') bit patterns."""
    if dtype == "f16":
        return f16_bits_to_f32(bits)
    if dtype == "bf16":
        return bf16_bits_to_f32(bits)
    raise ValueError(dtype)


def e4m3_encode(x) -> np.ndarray:
    """Saturating RNE cast of binary32 values to OCP E4M3 bytes."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    _load().orc_e4m3_encode_n(_p(x), x.size, _p(out))
    return out


def e4m3_decode(c) -> np.ndarray:
    c = _c(c, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().orc_e4m3_decode_n(_p(c), c.size, _p(out))
    return out


# ------------------------------------------------------------------ W4 ----

def w4_quantize(w, group: int = 128, asymmetric: bool = False):
    """Codes u [N][K] (0..15), FP16 scale bits [N][K/G], zero-points [N][K/G]."""
    w = _c(w, np.float32)
    N, K = w.shape
    assert K % group == 0 and (not asymmetric or K % (2 * group) == 0)
    u = np.empty((N, K), np.uint8)
    s = np.empty((N, K // group), np.uint16)
    z = np.empty((N, K // group), np.uint8)
    _load().orc_w4_quantize(_p(w), N, K, group, int(bool(asymmetric)), _p(u), _p(s), _p(z))
    return u, s, z


def w4_pack_codes(u, s16, z, asymmetric: bool = False):
    """Lay codes u [N][K], scale bits [N][K/128], zero-points [N][K/128] out in
    the tiled packed format -> (qweight u32 [N/16][K/128][64][4],
    scales u16 [N/16][K/128][16], zeros u8 [N/16][K/256][16] or None)."""
    u = _c(u, np.uint8)
    s16 = _c(s16, np.uint16)
    z = _c(z, np.uint8)
    N, K = u.shape
    assert N % 16 == 0 and K % 256 == 0
    qweight = np.empty((N // 16, K // 128, 64, 4), np.uint32)
    scales = np.empty((N // 16, K // 128, 16), np.uint16)
    zeros = np.empty((N // 16, K // 256, 16), np.uint8) if asymmetric else None
    _load().orc_w4_pack(_p(u), _p(s16), _p(z), N, K, int(bool(asymmetric)), _p(qweight), _p(scales), _p(zeros))
    return qweight, scales, zeros


def w4_pack(w, group: int = 128, asymmetric: bool = False):
    """Quantize + pack W [N][K] -> (qweight, scales, zeros) in the tiled format
    (zeros None when symmetric)."""
    u, s, z = w4_quantize(w, group, asymmetric)
    return w4_pack_codes(u, s, z, asymmetric)


def w4_unpack(qweight, scales, zeros, N: int, K: int):
    """Tiled packed format -> (codes u [N][K], scale bits [N][K/128], zero-points [N][K/128])."""
    qweight = _c(qweight, np.uint32)
    scales = _c(scales, np.uint16)
    zeros = None if zeros is None else _c(zeros, np.uint8)
    u = np.empty((N, K), np.uint8)
    s = np.empty((N, K // 128), np.uint16)
    z = np.empty((N, K // 128), np.uint8)
    _load().orc_w4_unpack(_p(qweight), _p(scales), _p(zeros), N, K, _p(u), _p(s), _p(z))
    return u, s, z


def w4_dequant(qweight, scales, zeros, N: int, K: int, group: int = 128) -> np.ndarray:
    qweight = _c(qweight, np.uint32)
    scales = _c(scales, np.uint16)
    zeros = None if zeros is None else _c(zeros, np.uint8)
    out = np.empty((N, K), np.float64)
    _load().orc_w4_dequant(_p(qweight), _p(scales), _p(zeros), N, K, group, _p(out))
    return out


def gemm_w4a16(x_bits, x_dtype: str, qweight, scales, zeros, group: int = 128) -> np.ndarray:
    """Y = X W^T in binary64 on the exact activation values and dequantized weights."""
    x_bits = _c(x_bits, np.uint16)
    qweight = _c(qweight, np.uint32)
    scales = _c(scales, np.uint16)
    zeros = None if zeros is None else _c(zeros, np.uint8)
    M, K = x_bits.shape
    N = qweight.shape[0] * 16
    assert qweight.shape[1] * 128 == K
    y = np.empty((M, N), np.float64)
    _load().orc_gemm_w4a16(_p(x_bits), int(x_dtype == "bf16"), M, K, _p(qweight), _p(scales),
                           _p(zeros), N, group, _p(y))
    return y


# ----------------------------------------------------------------- W8A8 ----

def scale_shape(gran: int, R: int, C: int):
    return {GRAN_TENSOR: (2,), GRAN_ROW: (R,), GRAN_ROW_G128: (R, C // 128),
            GRAN_BLOCK128: (R // 128, C // 128)}[gran]


def act_quant_int8(x, gran: int):
    """Dynamic INT8 quantization of binary32 values x [R][C] -> (q int8, scales f32)."""
    x = _c(x, np.float32)
    R, C = x.shape
    q = np.empty((R, C), np.int8)
    s = np.empty(scale_shape(gran, R, C), np.float32)
    _load().orc_quant_int8(_p(x), R, C, gran, _p(q), _p(s))
    return q, s


def act_quant_fp8(x, gran: int):
    """Dynamic E4M3 quantization of binary32 values x [R][C] -> (q uint8, scales f32)."""
    x = _c(x, np.float32)
    R, C = x.shape
    q = np.empty((R, C), np.uint8)
    s = np.empty(scale_shape(gran, R, C), np.float32)
    _load().orc_quant_fp8(_p(x), R, C, gran, _p(q), _p(s))
    return q, s


def gemm_i8_acc(a, w) -> np.ndarray:
    """Exact INT32 accumulators acc[m,n] = sum_k a[m,k] w[n,k]; raises on overflow."""
    a = _c(a, np.int8)
    w = _c(w, np.int8)
    M, K = a.shape
    N = w.shape[0]
    acc = np.empty((M, N), np.int32)
    if _load().orc_gemm_i8_acc(_p(a), _p(w), M, N, K, _p(acc)):
        raise OverflowError("INT32 accumulator overflow")
    return acc


def gemm_w8a8(a, a_scales, a_gran: int, w, w_scales, w_gran: int, fp8: bool) -> np.ndarray:
    """Exact dequantized W8A8 GEMM in binary64: Y = (A*s_a)(W*s_w)^T."""
    a = _c(a, np.uint8 if fp8 else np.int8)
    w = _c(w, np.uint8 if fp8 else np.int8)
    a_scales = _c(a_scales, np.float32)
    w_scales = _c(w_scales, np.float32)
    M, K = a.shape
    N = w.shape[0]
    y = np.empty((M, N), np.float64)
    _load().orc_gemm_w8a8(_p(a), _p(a_scales), a_gran, _p(w), _p(w_scales), w_gran,
                          int(bool(fp8)), M, N, K, _p(y))
    return y


def gemm_w4a8(a, a_scales, a_gran: int, qweight, scales, zeros, group: int = 128) -> np.ndarray:
    """W4A8: Y = (A*s_a) W^T in binary64, A the INT8 activation codes with per-row
    (or per-tensor) scales, W^ the dequantized packed INT4 weights."""
    assert a_gran in (GRAN_TENSOR, GRAN_ROW)
    a = _c(a, np.int8)
    a_scales = _c(a_scales, np.float32)
    qweight = _c(qweight, np.uint32)
    scales = _c(scales, np.uint16)
    zeros = None if zeros is None else _c(zeros, np.uint8)
    M, K = a.shape
    N = qweight.shape[0] * 16
    assert qweight.shape[1] * 128 == K
    y = np.empty((M, N), np.float64)
    _load().orc_gemm_w4a8(_p(a), _p(a_scales), a_gran, M, K, _p(qweight), _p(scales), _p(zeros), N, group, _p(y))
    return y


# ------------------------------------------------------------ SmoothQuant ----

def col_amax(x) -> np.ndarray:
    """max_r |x[r, j]| of a binary32 matrix [R][C]."""
    x = _c(x, np.float32)
    R, C = x.shape
    out = np.empty(C, np.float32)
    _load().orc_col_amax(_p(x), R, C, _p(out))
    return out


def smooth_scales(amax_x, amax_w, alpha: float = 0.5) -> np.ndarray:
    """Per-input-channel smoothing factors s_j = amax_x^alpha / amax_w^(1-alpha)
    (binary64, rounded once to binary32; 1 where a maximum is 0)."""
    amax_x = _c(amax_x, np.float32)
    amax_w = _c(amax_w, np.float32)
    s = np.empty(amax_x.shape, np.float32)
    _load().orc_smooth_scales(_p(amax_x), _p(amax_w), amax_x.size, float(alpha), _p(s))
    return s


def col_mul(x, m) -> np.ndarray:
    """x[r][j] * m[j] in binary32 (one rounding per element)."""
    x = _c(x, np.float32)
    m = _c(m, np.float32)
    R, C = x.shape
    out = np.empty((R, C), np.float32)
    _load().orc_col_mul(_p(x), R, C, _p(m), _p(out))
    return out


# ------------------------------------------------------ LLM.int8() outliers ----

def outlier_channels(x, tau: float) -> np.ndarray:
    """Increasing int32 indices j with max_r |x[r, j]| >= tau (binary32 x)."""
    x = _c(x, np.float32)
    R, C = x.shape
    idx = np.empty(C, np.int32)
    n = _load().orc_outlier_channels(_p(x), R, C, float(tau), _p(idx))
    return idx[:n].copy()


def act_quant_int8_outlier(x, idx):
    """Per-token INT8 of x with the columns idx set to zero: the column
    multiplier with factors 0 on idx and 1 elsewhere, then per-token INT8."""
    x = _c(x, np.float32)
    mask = np.ones(x.shape[1], np.float32)
    mask[np.asarray(idx, np.int64)] = 0.0
    return act_quant_int8(col_mul(x, mask), GRAN_ROW)


def gemm_w8a8_outlier(a, a_scales, w, w_scales, x, idx) -> np.ndarray:
    """INT8 part plus the side path over the outlier columns, binary64
    (per-token a_scales [M], per-channel w_scales [N])."""
    a = _c(a, np.int8)
    w = _c(w, np.int8)
    a_scales = _c(a_scales, np.float32)
    w_scales = _c(w_scales, np.float32)
    x = _c(x, np.float32)
    idx = _c(idx, np.int32)
    M, K = a.shape
    N = w.shape[0]
    y = np.empty((M, N), np.float64)
    _load().orc_gemm_w8a8_outlier(_p(a), _p(a_scales), _p(w), _p(w_scales), _p(x), _p(idx), idx.size, M, N, K,
                                  _p(y))
    return y


# ---------------------------------------------------------------- MXFP8 ----

def quant_mxfp8(x):
    """MXFP8 of binary32 x [R][C] (C % 32 == 0) -> (E4M3 bytes [R][C], E8M0
    scale bytes [R][C/32])."""
    x = _c(x, np.float32)
    R, C = x.shape
    assert C % 32 == 0
    q = np.empty((R, C), np.uint8)
    e = np.empty((R, C // 32), np.uint8)
    _load().orc_quant_mxfp8(_p(x), R, C, _p(q), _p(e))
    return q, e


def gemm_mxfp8(a, ea, w, ew) -> np.ndarray:
    """Exact MXFP8 GEMM in binary64: Y = (A X_a)(W X_w)^T."""
    a, ea, w, ew = (_c(t, np.uint8) for t in (a, ea, w, ew))
    M, K = a.shape
    N = w.shape[0]
    y = np.empty((M, N), np.float64)
    _load().orc_gemm_mxfp8(_p(a), _p(ea), _p(w), _p(ew), M, N, K, _p(y))
    return y


def e2m1_encode(x) -> np.ndarray:
    """Saturating RNE E2M1 codes (0..15) of binary32 values."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    _load().orc_e2m1_encode_n(_p(x), x.size, _p(out))
    return out


def e2m1_decode(c) -> np.ndarray:
    """Values of E2M1 codes (the low nibble of each byte) in binary64."""
    c = _c(c, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().orc_e2m1_decode_n(_p(c), c.size, _p(out))
    return out


def quant_mxfp4(x):
    """MXFP4 of binary32 x [R][C] (C % 32 == 0) -> (packed E2M1 bytes
    [R][C/2], element 2i in the low nibble; E8M0 scale bytes [R][C/32])."""
    x = _c(x, np.float32)
    R, C = x.shape
    assert C % 32 == 0
    q = np.empty((R, C // 2), np.uint8)
    e = np.empty((R, C // 32), np.uint8)
    _load().orc_quant_mxfp4(_p(x), R, C, _p(q), _p(e))
    return q, e


def gemm_mxfp4(a, ea, w, ew) -> np.ndarray:
    """Exact MXFP4 GEMM in binary64: Y = (A X_a)(W X_w)^T, A and W packed
    [rows][K/2]."""
    a, ea, w, ew = (_c(t, np.uint8) for t in (a, ea, w, ew))
    M, K = a.shape[0], a.shape[1] * 2
    N = w.shape[0]
    y = np.empty((M, N), np.float64)
    _load().orc_gemm_mxfp4(_p(a), _p(ea), _p(w), _p(ew), M, N, K, _p(y))
    return y


def num_threads() -> int:
    """Threads the oracle's OpenMP loops run on."""
    return int(_load().orc_num_threads())


def rel_l2(y, ref) -> float:
    """||y - ref||_2 / ||ref||_2 in binary64."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((y - ref).ravel())
    return float(num / den) if den > 0 else float(num)
