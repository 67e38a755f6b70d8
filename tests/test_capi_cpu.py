"""Host-side checks of the C ABI (no GPU needed).

* the library loads and exports every function that include/bitgemm.h declares;
* every entry point rejects ineligible calls with the documented status code
  before touching the device (fail-closed, "Low-precision LLM inference" §24
  eligibility checklist and §31 fallback_policy).  The pointers passed here
  are fake, 16-byte aligned addresses: a call that got past validation would
  fail in the HIP runtime, so a BG_ERR_* other than BG_ERR_HIP proves the
  check happened on the host first.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitgemm.h")

OK, E_NULL, E_SHAPE, E_ALIGN, E_DTYPE, E_UNSUP, E_HIP, E_WS = range(8)
F32, F16, BF16, I8, FP8, I32 = range(6)


@pytest.fixture(scope="module")
def L():
    from bit_gemm_w4_amd import build, ops
    if not os.path.exists(ops.LIB_PATH):
        build.build()
    return ops.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(L):
    from bit_gemm_w4_amd import ops
    names = _declared_functions()
    assert set(names) >= {"w4_pack", "gemm_w4a16", "act_quant_int8", "act_quant_fp8", "gemm_w8a8"}
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(ops.EXPORTS)


def test_internal_symbols_hidden():
    out = os.popen(f"nm -D --defined-only {os.path.join(ROOT, 'bit_gemm_w4_amd', 'libbitgemm.so')}").read()
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert exported == set(_declared_functions())


def test_status_strings_and_version(L):
    assert L.bg_status_string(0) == b"ok"
    assert L.bg_status_string(2) == b"unsupported shape"
    assert L.bg_status_string(99) == b"unknown status"
    assert L.bg_status_string(7) == b"workspace missing or too small"
    assert L.bg_pack_format_version() == 1


P = 0x10000          # fake, 16-byte aligned device addresses
Q = 0x20000


def _last(L):
    return L.bg_last_error().decode()


def test_w4_pack_validation(L):
    f = L.w4_pack
    assert f(None, F32, 16, 256, 128, 0, P, Q, None, None) == E_NULL
    assert f(P, F32, 16, 256, 128, 1, P, Q, None, None) == E_NULL          # asym without zeros
    assert f(P, F32, 16, 256, 128, 0, P, Q, P, None) == E_UNSUP            # sym with zeros
    assert f(P, I8, 16, 256, 128, 0, P, Q, None, None) == E_DTYPE
    assert f(P, F32, 16, 256, 64, 0, P, Q, None, None) == E_UNSUP          # group != 128
    assert f(P, F32, 0, 256, 128, 0, P, Q, None, None) == E_SHAPE
    assert f(P, F32, 16, 384, 128, 0, P, Q, None, None) == E_SHAPE         # K % 256
    assert "K=384" in _last(L)
    assert f(P + 4, F32, 16, 256, 128, 0, P, Q, None, None) == E_ALIGN


def test_gemm_w4a16_validation(L):
    f = L.gemm_w4a16_ex
    assert f(None, BF16, 1, 256, P, Q, None, 16, 128, P, 0, None) == E_NULL
    assert f(P, F32, 1, 256, P, Q, None, 16, 128, P, 0, None) == E_DTYPE
    assert f(P, BF16, 0, 256, P, Q, None, 16, 128, P, 0, None) == E_SHAPE
    assert f(P, BF16, 1, 256, P, Q, None, 24, 128, P, 0, None) == E_SHAPE   # N % 16
    assert f(P, BF16, 1, 128, P, Q, None, 16, 128, P, 0, None) == E_SHAPE   # K % 256
    assert f(P, BF16, 1, 256, P, Q, None, 16, 256, P, 0, None) == E_UNSUP   # group
    assert f(P, BF16, 1, 256, P, Q + 2, None, 16, 128, P, 0, None) == E_ALIGN
    assert f(P, BF16, 1, 256, P, Q, None, 16, 128, P, 9, None) == E_UNSUP   # algo
    assert f(P, BF16, 1, 256, P, Q, None, 16, 128, P, 4, None) == E_WS      # split-K needs _ws


def test_gemm_w4a8_workspace(L):
    # split while the 256 x 128 tiles fill less than one round: S = min(256 / tiles, groups / 4)
    assert L.gemm_w4a8_workspace_bytes(256, 4096, 14336) == 8 * 256 * 4096 * 4       # 32 tiles
    assert L.gemm_w4a8_workspace_bytes(300, 4096, 14336) == 4 * 300 * 4096 * 4       # 64 tiles
    assert L.gemm_w4a8_workspace_bytes(2048, 4096, 14336) == 0                       # 256 tiles
    assert L.gemm_w4a8_workspace_bytes(16, 1024, 512) == 0                           # 4 groups
    assert L.gemm_w4a8_workspace_bytes(16, 1000, 512) == 0                           # N % 16
    # M <= 32 runs the small-M kernel (no workspace), above it the split large-M kernel
    for n, k in ((6144, 4096), (4096, 4096), (28672, 4096), (4096, 14336)):
        for m in (1, 16, 17, 32):
            assert L.gemm_w4a8_workspace_bytes(m, n, k) == 0
    assert L.gemm_w4a8_workspace_bytes(33, 4096, 14336) > 0
    f = L.gemm_w4a8_ws
    assert f(P, P, 1, 33, 14336, P, Q, None, 4096, 128, P, BF16, None, 0, None) == E_WS


def test_gemm_w4a16_workspace(L):
    f = L.gemm_w4a16_ws
    need = L.gemm_w4a16_workspace_bytes(16, 4096, 14336, 0)
    assert need > 0 and need % 16 == 0
    assert L.gemm_w4a16_workspace_bytes(16, 4096, 14336, 3) == 0            # tiled: none
    # AUTO with a workspace: split-K from M = 8 on deep layers, M = 9 on wide ones, from
    # M = 17 on N > 4096, from M = 24 everywhere; the small-M kernel otherwise
    assert L.gemm_w4a16_workspace_bytes(8, 28672, 4096, 0) == 0
    assert L.gemm_w4a16_workspace_bytes(16, 28672, 4096, 0) == 0       # wide layer: one-round small-M
    assert L.gemm_w4a16_workspace_bytes(17, 28672, 4096, 0) > 0
    assert L.gemm_w4a16_workspace_bytes(7, 4096, 14336, 0) == 0
    assert L.gemm_w4a16_workspace_bytes(8, 4096, 14336, 0) > 0
    assert L.gemm_w4a16_workspace_bytes(16, 6144, 4096, 0) == 0
    assert L.gemm_w4a16_workspace_bytes(17, 6144, 4096, 0) > 0
    assert L.gemm_w4a16_workspace_bytes(23, 4096, 4096, 0) == 0
    assert L.gemm_w4a16_workspace_bytes(24, 4096, 4096, 0) > 0
    # past M = 64: split-K of the large-M kernel while its 256 x 128 tiles fill
    # less than one round (S = min(256 / tiles, groups / 4) slices of FP32 M x N)
    assert L.gemm_w4a16_workspace_bytes(1000, 4096, 14336, 0) == 2 * 1000 * 4096 * 4   # 128 tiles: S = 2
    assert L.gemm_w4a16_workspace_bytes(130, 4096, 14336, 4) == 8 * 130 * 4096 * 4     # 32 tiles: S = 8
    assert L.gemm_w4a16_workspace_bytes(130, 4096, 512, 4) == 0                        # 4 groups: no split
    assert L.gemm_w4a16_workspace_bytes(2048, 4096, 14336, 0) == 0                     # 256 tiles: one round
    assert f(P, BF16, 16, 14336, P, Q, None, 4096, 128, P, None, 0, 0, None) == E_WS
    assert f(P, BF16, 16, 14336, P, Q, None, 4096, 128, P, P, need - 16, 0, None) == E_WS
    assert "needed" in _last(L)
    assert f(P, BF16, 100, 14336, P, Q, None, 4096, 128, P, P, need, 4, None) == E_WS      # large-M split needs more
    assert f(P, BF16, 16, 14336, P, Q, None, 4096, 128, P, P + 8, need, 0, None) == E_ALIGN


def test_act_quant_validation(L):
    for f in (L.act_quant_int8, L.act_quant_fp8):
        assert f(P, BF16, 4, 128, 1, None, Q, None) == E_NULL
        assert f(P, I8, 4, 128, 1, P, Q, None) == E_DTYPE
        assert f(P, BF16, 4, 128, 7, P, Q, None) == E_UNSUP
        assert f(P, BF16, 0, 128, 1, P, Q, None) == E_SHAPE
        assert f(P, BF16, 4, 192, 1, P, Q, None) == E_SHAPE                 # cols % 128
        assert f(P, BF16, 100, 128, 3, P, Q, None) == E_SHAPE               # BLOCK128 rows % 128
        assert f(P, BF16, 4, 128, 1, P, Q + 8, None) == E_ALIGN


def test_gemm_w8a8_validation(L):
    f = L.gemm_w8a8_ex
    T, R, G, B = 0, 1, 2, 3
    assert f(None, P, R, P, Q, R, I8, 4, 16, 128, P, BF16, 0, None) == E_NULL
    assert f(P, None, R, P, Q, R, I8, 4, 16, 128, P, BF16, 0, None) == E_NULL   # scales needed
    assert f(P, P, R, P, Q, R, BF16, 4, 16, 128, P, BF16, 0, None) == E_DTYPE
    assert f(P, P, R, P, Q, R, FP8, 4, 16, 128, P, I32, 0, None) == E_DTYPE     # I32 needs I8
    assert f(P, P, R, P, Q, R, I8, 4, 16, 128, P, I8, 0, None) == E_DTYPE
    assert f(P, P, G, P, Q, B, I8, 4, 128, 128, P, BF16, 0, None) == E_UNSUP    # block needs FP8
    assert f(P, P, G, P, Q, R, FP8, 4, 128, 128, P, BF16, 0, None) == E_UNSUP   # mixed
    assert f(P, P, R, P, Q, B, FP8, 4, 128, 128, P, BF16, 0, None) == E_UNSUP
    assert f(P, P, G, P, Q, B, FP8, 4, 144, 128, P, BF16, 0, None) == E_SHAPE   # BLOCK128 N % 128
    assert f(P, P, R, P, Q, R, I8, 4, 24, 128, P, BF16, 0, None) == E_SHAPE     # N % 16
    assert f(P, P, R, P, Q, R, I8, 4, 16, 192, P, BF16, 0, None) == E_SHAPE     # K % 128
    assert f(P, P, R, P, Q, R, I8, 4, 16, 131072 + 128, P, BF16, 0, None) == E_SHAPE
    # K = 131072 with every code at -128 would sum to exactly 2^31: rejected
    assert f(P, P, R, P, Q, R, I8, 4, 16, 131072, P, BF16, 0, None) == E_SHAPE
    assert f(P, P, R, P, Q, R, I8, 4, 16, 128, P + 1, BF16, 0, None) == E_ALIGN
    assert f(P, P, R, P, Q, R, I8, 4, 16, 128, P, BF16, 5, None) == E_UNSUP     # algo


def test_auto_dispatch_thresholds(L):
    GEMV, SKINNY, TILED = 1, 2, 3
    assert L.gemm_w4a16_algo(1, 4096, 4096, BF16) == SKINNY
    assert L.gemm_w4a16_algo(4096, 4096, 4096, BF16) == TILED
    assert L.gemm_w8a8_algo(2048, 4096, 4096, I8) == TILED
    seen = {L.gemm_w4a16_algo(m, 4096, 4096, BF16) for m in range(1, 300)}
    assert seen == {SKINNY, TILED}
    assert GEMV not in seen        # the VALU GEMV is reachable through gemm_w4a16_ex only
    # W8A8: small-M kernel at decode sizes (through M = 16 on every shape),
    # tiled once the 256 x 128 tiles fill the device
    for n, k in ((6144, 4096), (4096, 4096), (4096, 14336), (28672, 4096)):
        assert L.gemm_w8a8_algo(1, n, k, I8) == SKINNY
        assert L.gemm_w8a8_algo(8, n, k, FP8) == SKINNY
        assert L.gemm_w8a8_algo(16, n, k, I8) == SKINNY
        assert L.gemm_w8a8_algo(129, n, k, I8) == TILED
    assert L.gemm_w8a8_algo(17, 28672, 4096, I8) == TILED      # 224 tiles already
    assert L.gemm_w8a8_algo(32, 4096, 14336, I8) == SKINNY
    assert L.gemm_w8a8_algo(128, 4096, 14336, I8) == SKINNY    # 32 tiles, long K
    assert L.gemm_w8a8_algo(128, 4096, 4096, I8) == TILED      # 32 tiles, short K
    # with a workspace: the split large-M kernel where it measured faster
    ws8 = L.gemm_w8a8_workspace_bytes
    for n, k in ((6144, 4096), (4096, 4096), (4096, 14336), (28672, 4096)):
        assert ws8(1, n, k, I8, 1, 0) == 0                      # small-M kernel through M = 16
        assert ws8(16, n, k, FP8, 0, 0) == 0
    assert ws8(17, 6144, 4096, I8, 1, 0) > 0                    # qkv above M = 16: split large-M
    assert ws8(17, 4096, 14336, FP8, 0, 0) > 0                  # down above M = 16
    assert ws8(24, 4096, 4096, I8, 1, 0) == 0                   # o through M = 32: small-M kernel
    assert ws8(32, 4096, 4096, I8, 1, 0) == 0
    assert ws8(48, 4096, 4096, I8, 1, 0) == 48 * 4096 * 4 * 4            # above: split large-M, S = 4
    assert ws8(2048, 28672, 4096, I8, 1, 0) == 0                # full grid: no split


def test_outlier_workspace_bytes(L):
    # [min(rows, 128)][cols] row-slice column maxima plus the [cols] multiplier, FP32
    assert L.act_quant_outlier_workspace_bytes(2048, 4096) == (128 * 4096 + 4096) * 4
    assert L.act_quant_outlier_workspace_bytes(5, 128) == (5 * 128 + 128) * 4
    assert L.act_quant_outlier_workspace_bytes(16, 100) == 0            # cols % 128
    assert L.act_quant_outlier_workspace_bytes(0, 128) == 0


def test_outlier_gemm_int8_k_bound(L):
    # the INT8 part accumulates K products of at most 128 * 128 in INT32: K = 131072
    # could reach 2^31, so the largest K accepted is 130944
    f = L.gemm_w8a8_outlier
    P = 1 << 20
    R = 1
    assert f(P, P, P, P, R, P, BF16, P, P, 4, 16, 131072, P, BF16, None) == E_SHAPE
    assert f(P, P, P, P, R, P, BF16, P, P, 4, 16, 131072 + 128, P, BF16, None) == E_SHAPE
    assert f(P, P, P, P, R, P, BF16, P, P, 4, 16, 192, P, BF16, None) == E_SHAPE    # K % 128
    assert f(P, P, P, P, R, P, BF16, P, P, 4, 16, 130944, P + 4, BF16, None) == E_ALIGN   # K passes


def test_noalloc_rejects_before_touching_the_device(L):
    # shapes whose split-K partials exceed the static scratch are refused on
    # the host, with the size in the message; so are the usual shape errors
    f = L.gemm_w4a16_noalloc
    P = 1 << 20
    limit = 16 << 20
    assert L.gemm_w4a16_workspace_bytes(256, 4096, 14336, 0) > limit      # down at M = 256: K split in 8
    assert f(P, BF16, 256, 14336, P, P, P, 4096, 128, P, None) == E_WS
    assert b"scratch" in L.bg_last_error()
    assert f(None, BF16, 16, 4096, P, P, P, 4096, 128, P, None) == E_NULL
    assert f(P, BF16, 0, 4096, P, P, P, 4096, 128, P, None) == E_SHAPE
    assert f(P, BF16, 16, 4096 + 128, P, P, P, 4096, 128, P, None) == E_SHAPE
    assert f(P, BF16, 16, 4096, P, P, P, 4100, 128, P, None) == E_SHAPE


def test_probe_library_exports():
    """The device-rate probes build into their own object (not the library)
    and export their entry points; nothing is launched here."""
    import ctypes
    import os
    from bit_gemm_w4_amd import probes
    if not os.path.exists(probes.LIB):
        probes.build()
    L = ctypes.CDLL(probes.LIB)
    for name in ("probe_mfma", "probe_lds", "probe_stream", "probe_empty", "probe_read_once"):
        assert hasattr(L, name), name
    main = ctypes.CDLL(os.path.join(os.path.dirname(probes.__file__), "libbitgemm.so"))
    assert not hasattr(main, "probe_mfma")
