"""Thin Python binding of ``libbitgemm.so`` (the C ABI in ``include/bitgemm.h``).

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI.  Torch tensors supply device memory and the current HIP stream; the
functions here check dtypes/devices, allocate outputs with torch, pass raw
pointers and raise :class:`BitGemmError` on a non-zero status.  There is no
CPU fallback: if the library is missing, :func:`lib` raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("BG_LIB_PATH") or os.path.join(_PKG, "libbitgemm.so")

# enums of include/bitgemm.h
F32, F16, BF16, I8, FP8_E4M3, I32 = 0, 1, 2, 3, 4, 5
GRAN_TENSOR, GRAN_ROW, GRAN_ROW_G128, GRAN_BLOCK128 = 0, 1, 2, 3
ALGO_AUTO, ALGO_GEMV, ALGO_SKINNY, ALGO_TILED, ALGO_SPLITK, ALGO_MID = 0, 1, 2, 3, 4, 5
PACK_FORMAT_VERSION = 1

EXPORTS = (
    "w4_pack", "gemm_w4a16", "gemm_w4a16_ex", "gemm_w4a16_ws", "gemm_w4a16_noalloc", "gemm_w4a16_workspace_bytes", "act_quant_int8", "act_quant_fp8",
    "act_quant_int8_smooth", "act_quant_fp8_smooth", "act_quant_mxfp8", "gemm_mxfp8", "act_quant_mxfp4", "gemm_mxfp4", "act_quant_int8_outlier", "act_quant_outlier_workspace_bytes",
    "gemm_w8a8_outlier", "gemm_w8a8",
    "gemm_w8a8_ex", "gemm_w8a8_ws", "gemm_w8a8_workspace_bytes", "gemm_w4a8", "gemm_w4a8_ws", "gemm_w4a8_workspace_bytes",
    "gemm_w4a16_algo", "gemm_w8a8_algo",
    "bg_status_string", "bg_last_error",
    "bg_pack_format_version", "bg_last_kernel",
)

_TORCH_DT = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}


class BitGemmError(RuntimeError):
    def __init__(self, status: int, fn: str):
        L = lib()
        self.status = status
        msg = L.bg_last_error().decode() or L.bg_status_string(status).decode()
        super().__init__(f"{fn}: status {status} ({L.bg_status_string(status).decode()}): {msg}")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libbitgemm.so (built in-tree by ``bit_gemm_w4_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_gemm_w4_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        sig = {
            "w4_pack": [P, I, I64, I64, I, I, P, P, P, P],
            "gemm_w4a16": [P, I, I64, I64, P, P, P, I64, I, P, P],
            "gemm_w4a16_ex": [P, I, I64, I64, P, P, P, I64, I, P, I, P],
            "gemm_w4a16_ws": [P, I, I64, I64, P, P, P, I64, I, P, P, I64, I, P],
            "gemm_w4a16_noalloc": [P, I, I64, I64, P, P, P, I64, I, P, P],
            "gemm_w4a16_workspace_bytes": [I64, I64, I64, I],
            "act_quant_int8": [P, I, I64, I64, I, P, P, P],
            "act_quant_fp8": [P, I, I64, I64, I, P, P, P],
            "act_quant_int8_smooth": [P, I, I64, I64, I, P, P, P, P],
            "act_quant_fp8_smooth": [P, I, I64, I64, I, P, P, P, P],
            "act_quant_mxfp8": [P, I, I64, I64, P, P, P],
            "gemm_mxfp8": [P, P, P, P, I64, I64, I64, P, I, P],
            "act_quant_mxfp4": [P, I, I64, I64, P, P, P],
            "gemm_mxfp4": [P, P, P, P, I64, I64, I64, P, I, P],
            "act_quant_int8_outlier": [P, I, I64, I64, ctypes.c_float, P, P, P, P, P, I64, P],
            "gemm_w8a8_outlier": [P, P, P, P, I, P, I, P, P, I64, I64, I64, P, I, P],
            "act_quant_outlier_workspace_bytes": [I64, I64],
            "gemm_w8a8": [P, P, I, P, P, I, I, I64, I64, I64, P, I, P],
            "gemm_w8a8_ex": [P, P, I, P, P, I, I, I64, I64, I64, P, I, I, P],
            "gemm_w8a8_ws": [P, P, I, P, P, I, I, I64, I64, I64, P, I, P, I64, I, P],
            "gemm_w8a8_workspace_bytes": [I64, I64, I64, I, I, I],
            "gemm_w4a8": [P, P, I, I64, I64, P, P, P, I64, I, P, I, P],
            "gemm_w4a8_ws": [P, P, I, I64, I64, P, P, P, I64, I, P, I, P, I64, P],
            "gemm_w4a8_workspace_bytes": [I64, I64, I64],
            "gemm_w4a16_algo": [I64, I64, I64, I],
            "gemm_w8a8_algo": [I64, I64, I64, I],
            "bg_status_string": [I],
            "bg_last_error": [],
            "bg_pack_format_version": [],
            "bg_last_kernel": [],
        }
        for name, argtypes in sig.items():
            fn = getattr(L, name)
            fn.argtypes = argtypes
            fn.restype = (ctypes.c_char_p if name in ("bg_status_string", "bg_last_error", "bg_last_kernel")
                          else ctypes.c_int64 if name.endswith("_workspace_bytes") else ctypes.c_int)
        _lib = L
    return _lib


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("bitgemm operands must be device tensors")
    if not t.is_contiguous():
        raise ValueError("bitgemm operands must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, fn: str):
    if status != 0:
        raise BitGemmError(status, fn)


def last_kernel() -> str:
    """Kernel instance enqueued by the last successful call on this thread."""
    return lib().bg_last_kernel().decode()


# --------------------------------------------------------------------- W4 ----

@dataclass
class PackedW4:
    """INT4 weights in the tiled w4_pack layout (BG_PACK_FORMAT_VERSION 1):
    one 1 KB tile per (16 output channels, 128-wide group)."""
    qweight: torch.Tensor        # int32 [N/16][K/128][64][4]
    scales: torch.Tensor         # float16 [N/16][K/128][16]
    zeros: torch.Tensor | None   # uint8 [N/16][K/256][16] (two 4-bit zero-points) or None
    N: int
    K: int
    group: int = 128

    @property
    def nbytes(self) -> int:
        z = 0 if self.zeros is None else self.zeros.numel()
        return self.qweight.numel() * 4 + self.scales.numel() * 2 + z


def w4_pack(w: torch.Tensor, group: int = 128, asymmetric: bool = False, stream=None) -> PackedW4:
    N, K = w.shape
    dt = _TORCH_DT.get(w.dtype)
    if dt is None:
        raise ValueError(f"w4_pack: unsupported dtype {w.dtype}")
    if N % 16 or K % 256 or group != 128:
        raise ValueError(f"w4_pack: need N % 16 == 0, K % 256 == 0, group == 128 (N={N}, K={K}, group={group})")
    qweight = torch.empty((N // 16, K // 128, 64, 4), dtype=torch.int32, device=w.device)
    scales = torch.empty((N // 16, K // 128, 16), dtype=torch.float16, device=w.device)
    zeros = torch.empty((N // 16, K // 256, 16), dtype=torch.uint8, device=w.device) if asymmetric else None
    _check(lib().w4_pack(_ptr(w), dt, N, K, group, int(asymmetric), _ptr(qweight), _ptr(scales), _ptr(zeros),
                         _stream(stream)), "w4_pack")
    return PackedW4(qweight, scales, zeros, N, K, group)


_workspaces: dict = {}
_retired: list = []


def workspace(nbytes: int, device) -> torch.Tensor:
    """A device workspace of at least nbytes, cached per device.  It needs no
    initialisation; calls sharing it must not overlap in time (use one per
    stream when streams run concurrently)."""
    key = torch.device(device).index or 0
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            _retired.append(ws)       # HIP graphs captured earlier may still use it
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def gemm_w4a16_workspace_bytes(M: int, N: int, K: int, algo: int = ALGO_AUTO) -> int:
    return int(lib().gemm_w4a16_workspace_bytes(M, N, K, algo))


def gemm_w4a16(x: torch.Tensor, packed: PackedW4, out: torch.Tensor | None = None, algo: int = ALGO_AUTO,
               ws: torch.Tensor | None | bool = None, stream=None) -> torch.Tensor:
    """Y = X W^T.  ws: a workspace tensor, None to use the cached per-device
    workspace (enables the split-K small-M kernel), or False for none."""
    M, K = x.shape
    if K != packed.K:
        raise ValueError(f"gemm_w4a16: x has K={K}, weights K={packed.K}")
    dt = _TORCH_DT.get(x.dtype)
    if dt not in (F16, BF16):
        raise ValueError(f"gemm_w4a16: activations must be float16/bfloat16, got {x.dtype}")
    if out is None:
        out = torch.empty((M, packed.N), dtype=x.dtype, device=x.device)
    L = lib()
    if ws is False:
        _check(L.gemm_w4a16_ex(_ptr(x), dt, M, K, _ptr(packed.qweight), _ptr(packed.scales), _ptr(packed.zeros),
                               packed.N, packed.group, _ptr(out), algo, _stream(stream)), "gemm_w4a16")
        return out
    if ws is None:
        need = gemm_w4a16_workspace_bytes(M, packed.N, K, algo)
        ws = workspace(need, x.device) if need > 0 else None
    _check(L.gemm_w4a16_ws(_ptr(x), dt, M, K, _ptr(packed.qweight), _ptr(packed.scales), _ptr(packed.zeros),
                           packed.N, packed.group, _ptr(out), _ptr(ws), 0 if ws is None else ws.numel(), algo,
                           _stream(stream)), "gemm_w4a16")
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20   # BG_NOALLOC_SCRATCH_BYTES


def gemm_w4a16_noalloc(x: torch.Tensor, packed: PackedW4, out: torch.Tensor, stream=None) -> torch.Tensor:
    """Y = X W^T through gemm_w4a16_noalloc: the split-K partials go to the
    library's static per-device scratch, so the call allocates nothing (the
    caller supplies `out`).  Calls on one GPU must not overlap in time."""
    M, K = x.shape
    if K != packed.K:
        raise ValueError(f"gemm_w4a16_noalloc: x has K={K}, weights K={packed.K}")
    dt = _TORCH_DT.get(x.dtype)
    if dt not in (F16, BF16):
        raise ValueError(f"gemm_w4a16_noalloc: activations must be float16/bfloat16, got {x.dtype}")
    if out.shape != (M, packed.N) or out.dtype != x.dtype:
        raise ValueError(f"gemm_w4a16_noalloc: out must be [{M}, {packed.N}] of {x.dtype}")
    _check(lib().gemm_w4a16_noalloc(_ptr(x), dt, M, K, _ptr(packed.qweight), _ptr(packed.scales),
                                    _ptr(packed.zeros), packed.N, packed.group, _ptr(out), _stream(stream)),
           "gemm_w4a16_noalloc")
    return out


def gemm_w4a16_algo(M: int, N: int, K: int, x_dtype: torch.dtype = torch.bfloat16) -> int:
    return lib().gemm_w4a16_algo(M, N, K, _TORCH_DT[x_dtype])


# ------------------------------------------------------------------- W8A8 ----

def scale_shape(gran: int, rows: int, cols: int):
    return {GRAN_TENSOR: (2,), GRAN_ROW: (rows,), GRAN_ROW_G128: (rows, cols // 128),
            GRAN_BLOCK128: (rows // 128, cols // 128)}[gran]


def _act_quant(fn: str, x: torch.Tensor, gran: int, out_dtype: torch.dtype, stream=None, col_mul=None):
    R, C = x.shape
    dt = _TORCH_DT.get(x.dtype)
    if dt is None:
        raise ValueError(f"{fn}: unsupported dtype {x.dtype}")
    q = torch.empty((R, C), dtype=out_dtype, device=x.device)
    s = torch.empty(scale_shape(gran, R, C), dtype=torch.float32, device=x.device)
    if col_mul is None:
        _check(getattr(lib(), fn)(_ptr(x), dt, R, C, gran, _ptr(q), _ptr(s), _stream(stream)), fn)
    else:
        if col_mul.dtype != torch.float32 or col_mul.numel() != C:
            raise ValueError(f"{fn}: col_mul must be {C} float32 values")
        _check(getattr(lib(), fn)(_ptr(x), dt, R, C, gran, _ptr(col_mul), _ptr(q), _ptr(s), _stream(stream)), fn)
    return q, s


def act_quant_int8(x: torch.Tensor, gran: int = GRAN_ROW, stream=None):
    """-> (int8 codes [R][C], float32 scales in the layout of `gran`)."""
    return _act_quant("act_quant_int8", x, gran, torch.int8, stream)


def act_quant_fp8(x: torch.Tensor, gran: int = GRAN_ROW, stream=None):
    """-> (E4M3 bytes as uint8 [R][C], float32 scales in the layout of `gran`)."""
    return _act_quant("act_quant_fp8", x, gran, torch.uint8, stream)


def act_quant_int8_smooth(x: torch.Tensor, col_mul: torch.Tensor, gran: int = GRAN_ROW, stream=None):
    """INT8 codes and scales of X diag(col_mul) (the SmoothQuant fold: 1/s for
    activations, s for the weights)."""
    return _act_quant("act_quant_int8_smooth", x, gran, torch.int8, stream, col_mul)


def act_quant_fp8_smooth(x: torch.Tensor, col_mul: torch.Tensor, gran: int = GRAN_ROW, stream=None):
    """E4M3 codes and scales of X diag(col_mul)."""
    return _act_quant("act_quant_fp8_smooth", x, gran, torch.uint8, stream, col_mul)


_OUT_DT = {torch.bfloat16: BF16, torch.float16: F16, torch.float32: F32, torch.int32: I32}


def act_quant_mxfp8(x: torch.Tensor, stream=None):
    """-> (E4M3 bytes as uint8 [R][C], E8M0 scale bytes uint8 [C/32][R rounded
    up to 16], K-block-major)."""
    R, C = x.shape
    dt = _TORCH_DT.get(x.dtype)
    if dt is None:
        raise ValueError(f"act_quant_mxfp8: unsupported dtype {x.dtype}")
    q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    e = torch.empty((C // 32, (R + 15) // 16 * 16), dtype=torch.uint8, device=x.device)
    _check(lib().act_quant_mxfp8(_ptr(x), dt, R, C, _ptr(q), _ptr(e), _stream(stream)), "act_quant_mxfp8")
    return q, e


def gemm_mxfp8(a: torch.Tensor, a_e8m0: torch.Tensor, w: torch.Tensor, w_e8m0: torch.Tensor,
               out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y = (A X_a)(W X_w)^T for MXFP8 operands (act_quant_mxfp8 outputs)."""
    M, K = a.shape
    N, K2 = w.shape
    if K != K2:
        raise ValueError(f"gemm_mxfp8: K mismatch {K} vs {K2}")
    for t, rows in ((a_e8m0, M), (w_e8m0, N)):
        if t.dtype != torch.uint8 or tuple(t.shape) != (K // 32, (rows + 15) // 16 * 16):
            raise ValueError("gemm_mxfp8: scales must be uint8 [K/32][rows rounded up to 16]")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _check(lib().gemm_mxfp8(_ptr(a), _ptr(a_e8m0), _ptr(w), _ptr(w_e8m0), M, N, K, _ptr(out), _OUT_DT[out.dtype],
                            _stream(stream)), "gemm_mxfp8")
    return out


def act_quant_mxfp4(x: torch.Tensor, stream=None):
    """-> (packed E2M1 bytes uint8 [R][C/2], element 2i in the low nibble;
    E8M0 scale bytes uint8 [C/32][R rounded up to 16], K-block-major)."""
    R, C = x.shape
    dt = _TORCH_DT.get(x.dtype)
    if dt is None:
        raise ValueError(f"act_quant_mxfp4: unsupported dtype {x.dtype}")
    q = torch.empty((R, C // 2), dtype=torch.uint8, device=x.device)
    e = torch.empty((C // 32, (R + 15) // 16 * 16), dtype=torch.uint8, device=x.device)
    _check(lib().act_quant_mxfp4(_ptr(x), dt, R, C, _ptr(q), _ptr(e), _stream(stream)), "act_quant_mxfp4")
    return q, e


def gemm_mxfp4(a: torch.Tensor, a_e8m0: torch.Tensor, w: torch.Tensor, w_e8m0: torch.Tensor,
               out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y = (A X_a)(W X_w)^T for MXFP4 operands (act_quant_mxfp4 outputs:
    packed [rows][K/2] bytes)."""
    M, KH = a.shape
    N, KH2 = w.shape
    if KH != KH2:
        raise ValueError(f"gemm_mxfp4: K mismatch {2 * KH} vs {2 * KH2}")
    K = 2 * KH
    for t, rows in ((a_e8m0, M), (w_e8m0, N)):
        if t.dtype != torch.uint8 or tuple(t.shape) != (K // 32, (rows + 15) // 16 * 16):
            raise ValueError("gemm_mxfp4: scales must be uint8 [K/32][rows rounded up to 16]")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _check(lib().gemm_mxfp4(_ptr(a), _ptr(a_e8m0), _ptr(w), _ptr(w_e8m0), M, N, K, _ptr(out), _OUT_DT[out.dtype],
                            _stream(stream)), "gemm_mxfp4")
    return out


def act_quant_outlier_workspace_bytes(rows: int, cols: int) -> int:
    return int(lib().act_quant_outlier_workspace_bytes(rows, cols))


def act_quant_int8_outlier(x: torch.Tensor, tau: float = 6.0, ws: torch.Tensor | None = None, stream=None):
    """The LLM.int8() split of X: its outlier channels (columns whose largest
    magnitude reaches tau) and the per-token INT8 codes of the other columns
    (outlier columns quantize to 0).  -> (q int8 [R][C], scales f32 [R], idx
    int32 [C] of which the first count entries are the outlier columns in
    increasing order, count int32 [1]); idx and count stay on the device."""
    R, C = x.shape
    dt = _TORCH_DT.get(x.dtype)
    if dt is None:
        raise ValueError(f"act_quant_int8_outlier: unsupported dtype {x.dtype}")
    q = torch.empty((R, C), dtype=torch.int8, device=x.device)
    sc = torch.empty((R,), dtype=torch.float32, device=x.device)
    idx = torch.empty((C,), dtype=torch.int32, device=x.device)
    cnt = torch.empty((1,), dtype=torch.int32, device=x.device)
    if ws is None:
        ws = workspace(max(act_quant_outlier_workspace_bytes(R, C), 16), x.device)
    _check(lib().act_quant_int8_outlier(_ptr(x), dt, R, C, float(tau), _ptr(q), _ptr(sc), _ptr(idx), _ptr(cnt),
                                        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "act_quant_int8_outlier")
    return q, sc, idx, cnt


def gemm_w8a8_outlier(a: torch.Tensor, a_scales: torch.Tensor, w: torch.Tensor, w_scales: torch.Tensor,
                      w_gran: int, x: torch.Tensor, idx: torch.Tensor, count: torch.Tensor,
                      out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """Y = s_a s_w (A W^T) + s_w (X_O W_O^T): the INT8 GEMM of the common
    channels plus the side path over the outlier channels idx[:count] (the
    act_quant_int8_outlier outputs), which multiplies the unquantized
    activations x by the INT8 weight columns, fused into the GEMM."""
    M, K = a.shape
    N, K2 = w.shape
    if K != K2 or tuple(x.shape) != (M, K):
        raise ValueError(f"gemm_w8a8_outlier: shapes a {tuple(a.shape)}, w {tuple(w.shape)}, x {tuple(x.shape)}")
    if a.dtype != torch.int8 or w.dtype != torch.int8:
        raise ValueError("gemm_w8a8_outlier: a and w must be int8 codes")
    if idx.dtype != torch.int32 or count.dtype != torch.int32 or idx.numel() < K:
        raise ValueError("gemm_w8a8_outlier: idx must be int32 with room for K entries, count int32")
    dt = _TORCH_DT.get(x.dtype)
    if dt is None:
        raise ValueError(f"gemm_w8a8_outlier: unsupported dtype {x.dtype}")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _check(lib().gemm_w8a8_outlier(_ptr(a), _ptr(a_scales), _ptr(w), _ptr(w_scales), w_gran, _ptr(x), dt, _ptr(idx),
                                   _ptr(count), M, N, K, _ptr(out), _OUT_DT[out.dtype], _stream(stream)),
           "gemm_w8a8_outlier")
    return out


def gemm_w8a8_workspace_bytes(M: int, N: int, K: int, fp8: bool = False, a_gran: int = GRAN_ROW,
                              algo: int = ALGO_AUTO) -> int:
    return int(lib().gemm_w8a8_workspace_bytes(M, N, K, FP8_E4M3 if fp8 else I8, a_gran, algo))


def gemm_w8a8(a: torch.Tensor, a_scales: torch.Tensor | None, a_gran: int, w: torch.Tensor,
              w_scales: torch.Tensor | None, w_gran: int, out_dtype: torch.dtype = torch.bfloat16,
              out: torch.Tensor | None = None, algo: int = ALGO_AUTO, ws: torch.Tensor | None | bool = None,
              stream=None) -> torch.Tensor:
    """Y = A W^T on the INT8 / FP8 matrix cores.  ws: a workspace tensor, None
    to use the cached per-device workspace (enables split-K of the large-M
    kernel), or False for none."""
    M, K = a.shape
    N, K2 = w.shape
    if K != K2:
        raise ValueError(f"gemm_w8a8: K mismatch {K} vs {K2}")
    if a.dtype == torch.int8 and w.dtype == torch.int8:
        in_dt = I8
    elif a.dtype == torch.uint8 and w.dtype == torch.uint8:
        in_dt = FP8_E4M3
    else:
        raise ValueError("gemm_w8a8: operands must both be int8 or both E4M3 bytes (uint8)")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    L = lib()
    if ws is False:
        _check(L.gemm_w8a8_ex(_ptr(a), _ptr(a_scales), a_gran, _ptr(w), _ptr(w_scales), w_gran, in_dt, M, N, K,
                              _ptr(out), _OUT_DT[out.dtype], algo, _stream(stream)), "gemm_w8a8")
        return out
    if ws is None:
        need = int(L.gemm_w8a8_workspace_bytes(M, N, K, in_dt, a_gran, algo))
        ws = workspace(need, a.device) if need > 0 else None
    _check(L.gemm_w8a8_ws(_ptr(a), _ptr(a_scales), a_gran, _ptr(w), _ptr(w_scales), w_gran, in_dt, M, N, K,
                          _ptr(out), _OUT_DT[out.dtype], _ptr(ws), 0 if ws is None else ws.numel(), algo,
                          _stream(stream)), "gemm_w8a8")
    return out


def gemm_w4a8_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().gemm_w4a8_workspace_bytes(M, N, K))


def gemm_w4a8(a: torch.Tensor, a_scales: torch.Tensor, a_gran: int, packed: PackedW4,
              out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
              ws: torch.Tensor | None | bool = None, stream=None) -> torch.Tensor:
    """Y = (A s_a) W^T: INT8 activation codes (act_quant_int8 with GRAN_ROW or
    GRAN_TENSOR) times packed INT4 weights, on the INT8 matrix cores.  ws: a
    workspace tensor, None to use the cached per-device workspace (enables the
    K split when the output tiles do not fill the device), or False for none."""
    M, K = a.shape
    if a.dtype != torch.int8:
        raise ValueError(f"gemm_w4a8: activations must be int8 codes, got {a.dtype}")
    if K != packed.K:
        raise ValueError(f"gemm_w4a8: a has K={K}, weights K={packed.K}")
    if out is None:
        out = torch.empty((M, packed.N), dtype=out_dtype, device=a.device)
    if out.dtype not in (torch.bfloat16, torch.float16, torch.float32):
        raise ValueError(f"gemm_w4a8: output must be bfloat16/float16/float32, got {out.dtype}")
    L = lib()
    if ws is False:
        _check(L.gemm_w4a8(_ptr(a), _ptr(a_scales), a_gran, M, K, _ptr(packed.qweight), _ptr(packed.scales),
                           _ptr(packed.zeros), packed.N, packed.group, _ptr(out), _OUT_DT[out.dtype],
                           _stream(stream)), "gemm_w4a8")
        return out
    if ws is None:
        need = gemm_w4a8_workspace_bytes(M, packed.N, K)
        ws = workspace(need, a.device) if need > 0 else None
    _check(L.gemm_w4a8_ws(_ptr(a), _ptr(a_scales), a_gran, M, K, _ptr(packed.qweight), _ptr(packed.scales),
                          _ptr(packed.zeros), packed.N, packed.group, _ptr(out), _OUT_DT[out.dtype], _ptr(ws),
                          0 if ws is None else ws.numel(), _stream(stream)), "gemm_w4a8")
    return out


def gemm_w8a8_algo(M: int, N: int, K: int, fp8: bool = False) -> int:
    return lib().gemm_w8a8_algo(M, N, K, FP8_E4M3 if fp8 else I8)
