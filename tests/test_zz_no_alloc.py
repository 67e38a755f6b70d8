"""gemm_w4a16_noalloc (the entry point for callers that cannot allocate)
against gemm_w4a16_ws, the entry point whose kernels it shares, and against
the oracle.

Two calls in a row on the static scratch, the second on a smaller input, are
each compared bit for bit with gemm_w4a16_ws on a caller workspace (the same
kernels on the same inputs give the same bits) and within the floating-point
bar (relative L2 <= 2e-3 against the oracle's binary64 product).
"""
import numpy as np
import pytest
import torch

from bit_gemm_w4_amd import synth

pytestmark = pytest.mark.gpu

REL_L2 = 2e-3


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_gemm_w4_amd import ops as _ops
    _ops.lib()
    return _ops


def _bits(x, dtype="bf16"):
    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16))
    return t.view({"f16": torch.float16, "bf16": torch.bfloat16}[dtype]).cuda()


def _host(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _prepare(ops, M, N, K, x_dtype, asym, seed):
    w, x = synth.layer(M, N, K, x_dtype, seed=seed, w_outlier_frac=0.01)
    p = ops.w4_pack(torch.from_numpy(w).cuda(), 128, asym)
    return w, x, p


@pytest.mark.parametrize("first,second", [
    ((32, 4096, 14336), (16, 1024, 8192)),      # small-M split-K, then a smaller split-K call
    ((130, 1040, 2048), (65, 272, 2048)),       # large-M kernel with K split, then smaller
    ((24, 28672, 4096), (17, 16400, 4096)),     # the wide layer at B = 24, then B = 17 (ragged)
])
@pytest.mark.parametrize("x_dtype,asym", [("bf16", True), ("f16", False)])
def test_noalloc_matches_workspace_entry(ops, orc, first, second, x_dtype, asym):
    cases = []
    for i, (M, N, K) in enumerate((first, second)):
        need = ops.gemm_w4a16_workspace_bytes(M, N, K, 0)
        assert 0 < need <= ops.NOALLOC_SCRATCH_BYTES, (M, N, K, need)
        w, x, p = _prepare(ops, M, N, K, x_dtype, asym, seed=40 + i)
        cases.append((M, N, K, w, x, p))
    # two calls in a row on the shared scratch, nothing in between
    outs = []
    for M, N, K, w, x, p in cases:
        y = torch.full((M, N), float("nan"), dtype=_bits(x[:1], x_dtype).dtype, device="cuda")
        ops.gemm_w4a16_noalloc(_bits(x, x_dtype), p, y)
        kern = ops.last_kernel()
        assert any(k in kern for k in ("splitk", "gemm", "mid")), kern
        outs.append(y)
    torch.cuda.synchronize()
    for (M, N, K, w, x, p), y in zip(cases, outs):
        need = ops.gemm_w4a16_workspace_bytes(M, N, K, 0)
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
        y_ws = ops.gemm_w4a16(_bits(x, x_dtype), p, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(_host(y), _host(y_ws)), (M, N, K)
        qw, s, z = orc.w4_pack(w, 128, asym)
        ref = orc.gemm_w4a16(x, x_dtype, qw, s, z)
        yv = orc.bits_to_f32(_host(y), x_dtype).astype(np.float64)
        err = orc.rel_l2(yv, ref)
        assert np.isfinite(yv).all() and err <= REL_L2, (M, N, K, err)


def test_noalloc_without_split(ops, orc):
    """Shapes that need no partials (B = 1) run the same single kernel."""
    M, N, K = 1, 4096, 4096
    assert ops.gemm_w4a16_workspace_bytes(M, N, K, 0) == 0
    w, x, p = _prepare(ops, M, N, K, "bf16", True, seed=7)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ops.gemm_w4a16_noalloc(_bits(x), p, y)
    y_ws = ops.gemm_w4a16(_bits(x), p)
    torch.cuda.synchronize()
    assert np.array_equal(_host(y), _host(y_ws))


def test_noalloc_rejects_oversized_scratch(ops):
    M, N, K = 256, 4096, 14336
    assert ops.gemm_w4a16_workspace_bytes(M, N, K, 0) > ops.NOALLOC_SCRATCH_BYTES
    p = ops.w4_pack(torch.zeros((N, K), dtype=torch.float32, device="cuda"), 128, True)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ops.BitGemmError, match="scratch"):
        ops.gemm_w4a16_noalloc(torch.zeros((M, K), dtype=torch.bfloat16, device="cuda"), p, y)
