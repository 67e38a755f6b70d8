"""Graph replay of every entry point (GPU).

The benchmark times each call as a replayed HIP graph, so a call must give
the same result when replayed: nothing it reads may depend on state a
previous call left behind (workspace contents, amax slots, counters), and
nothing it clears may rely on a memset node.  Each case captures the call
into a graph (after a warm eager call, on a side stream), then replays it
three times with eager work between the replays -- a differently shaped
call that reuses the cached workspace and overwrites the inputs' neighbours
-- and checks every replay bit for bit against the eager result (the same
kernels in the same order, so the outputs must be identical).
"""
import numpy as np
import pytest
import torch

from bit_gemm_w4_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_gemm_w4_amd import ops as _ops
    _ops.lib()
    return _ops


def _graph(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _bf16(M, K, seed, outliers=0):
    x = synth.activations(M, K, "bf16", seed=seed, n_outlier_cols=outliers)
    return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()


def _replays_match(fn, outs, disturb):
    """fn() writes into the tensors outs; compare three replays with eager."""
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = _graph(fn)
    for rep in range(3):
        for o in outs:
            o.fill_(0)
        disturb(rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o.view(torch.uint8) if o.dtype != torch.uint8 else o,
                               r.view(torch.uint8) if r.dtype != torch.uint8 else r), f"replay {rep}"


def _disturber(ops):
    """Eager work between replays: a W4A16 split-K call and an outlier
    detection of other shapes, both through the cached workspace."""
    w = synth.weights(8192, 2048, seed=7)
    p = ops.w4_pack(torch.from_numpy(w).cuda(), 128, True)
    x = _bf16(16, 2048, seed=8)
    xo = _bf16(300, 2048, seed=9, outliers=4)

    def disturb(rep):
        ops.gemm_w4a16(x, p)
        ops.act_quant_int8_outlier(xo, 6.0 + rep)
    return disturb


def test_graph_w4a16_decode_and_split(ops):
    disturb = _disturber(ops)
    for M, N, K in [(4, 4096, 4096), (16, 28672, 4096), (16, 4096, 14336)]:
        w = synth.weights(N, K, seed=M)
        p = ops.w4_pack(torch.from_numpy(w).cuda(), 128, True)
        x = _bf16(M, K, seed=M + 1)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        _replays_match(lambda: ops.gemm_w4a16(x, p, out=y), [y], disturb)


def test_graph_w4a16_large_m_split(ops):
    disturb = _disturber(ops)
    M, N, K = 130, 4096, 4096
    w = synth.weights(N, K, seed=11)
    p = ops.w4_pack(torch.from_numpy(w).cuda(), 128, True)
    x = _bf16(M, K, seed=12)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    _replays_match(lambda: ops.gemm_w4a16(x, p, out=y), [y], disturb)


def test_graph_act_quant_per_tensor(ops):
    """Per-tensor scaling clears its amax slot with a fill kernel each call."""
    disturb = _disturber(ops)
    x = _bf16(2048, 4096, seed=13, outliers=8)
    q = torch.empty((2048, 4096), dtype=torch.int8, device="cuda")
    s = torch.empty((2,), dtype=torch.float32, device="cuda")
    L = ops.lib()

    def call():
        ops._check(L.act_quant_int8(ops._ptr(x), ops._TORCH_DT[x.dtype], 2048, 4096, ops.GRAN_TENSOR, ops._ptr(q),
                                    ops._ptr(s), ops._stream(None)), "act_quant_int8")
    _replays_match(call, [q, s[:1]], disturb)


def test_graph_w8a8_split_and_w4a8(ops):
    disturb = _disturber(ops)
    M, N, K = 256, 4096, 4096
    x = _bf16(M, K, seed=14)
    w = torch.from_numpy(synth.weights(N, K, seed=15)).cuda()
    a, sa = ops.act_quant_int8(x, ops.GRAN_ROW)
    q, sw = ops.act_quant_int8(w, ops.GRAN_ROW)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    _replays_match(lambda: ops.gemm_w8a8(a, sa, ops.GRAN_ROW, q, sw, ops.GRAN_ROW, out=y), [y], disturb)
    p = ops.w4_pack(w, 128, True)
    y2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    _replays_match(lambda: ops.gemm_w4a8(a, sa, ops.GRAN_ROW, p, out=y2), [y2], disturb)


def test_graph_mxfp4(ops):
    disturb = _disturber(ops)
    M, N, K = 300, 1040, 1024
    x = _bf16(M, K, seed=16)
    w = torch.from_numpy(synth.weights(N, K, seed=17)).cuda()
    qa = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    ea = torch.empty((K // 32, (M + 15) // 16 * 16), dtype=torch.uint8, device="cuda")
    q, ew = ops.act_quant_mxfp4(w)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    L = ops.lib()

    def call():
        ops._check(L.act_quant_mxfp4(ops._ptr(x), ops._TORCH_DT[x.dtype], M, K, ops._ptr(qa), ops._ptr(ea),
                                     ops._stream(None)), "act_quant_mxfp4")
        ops.gemm_mxfp4(qa, ea, q, ew, out=y)
    _replays_match(call, [qa, ea[:, :M], y], disturb)


def test_graph_outlier_split(ops):
    """Detection (three kernels, no memsets), masked quantization and the
    GEMM with the fused side path, captured together."""
    disturb = _disturber(ops)
    M, N, K = 1000, 8208, 1024
    x = _bf16(M, K, seed=18, outliers=8)
    w = torch.from_numpy(synth.weights(N, K, seed=19)).cuda()
    wq, sw = ops.act_quant_int8(w, ops.GRAN_ROW)
    q = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sa = torch.empty((M,), dtype=torch.float32, device="cuda")
    idx = torch.empty((K,), dtype=torch.int32, device="cuda")
    cnt = torch.empty((1,), dtype=torch.int32, device="cuda")
    ws = torch.empty(ops.act_quant_outlier_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    L = ops.lib()

    def call():
        ops._check(L.act_quant_int8_outlier(ops._ptr(x), ops._TORCH_DT[x.dtype], M, K, 6.0, ops._ptr(q),
                                            ops._ptr(sa), ops._ptr(idx), ops._ptr(cnt), ops._ptr(ws), ws.numel(),
                                            ops._stream(None)), "act_quant_int8_outlier")
        ops.gemm_w8a8_outlier(q, sa, wq, sw, ops.GRAN_ROW, x, idx, cnt, out=y)
    fn_outs = [q, sa, cnt, y]
    _replays_match(call, fn_outs, disturb)
    n = int(cnt.item())
    assert n == 8
