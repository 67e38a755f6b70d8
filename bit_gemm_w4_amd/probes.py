"""Device-rate microbenchmarks (MI355X, gfx950) behind the kernels' ceilings.

    python3 -m bit_gemm_w4_amd.probes

prints a markdown table of: dense MFMA throughput per instruction shape
(independent accumulator chains, two waves per SIMD on all 1,024 SIMDs, and
dependent chains), LDS read bandwidth per CU (ds_read_b128), and streaming
throughput into registers and by buffer_load ... lds from an L2-resident
buffer (2 MiB) and from one that fits the 256 MB last-level cache but not
L2 (128 MiB); then the floors of the decode step's calls, timed the way the
step is (HIP graph replay, weights rotated over copies larger than the
last-level cache): an empty kernel per launch, and a plain read of exactly
each Llama-3-8B layer's packed W4 bytes.  `--floors` prints only those.

Not part of the library path: the kernels live in csrc_probes/probes.hip and
build into their own shared object (libprobes.so beside this file).
"""
import ctypes
import os
import subprocess

_PKG = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_PKG, "csrc_probes", "probes.hip")
LIB = os.path.join(_PKG, "libprobes.so")
CLOCK_GHZ = 2.4          # the spec clock, used only to express rates per cycle
SIMDS = 1024             # 256 CUs x 4

MFMA_KINDS = [           # (kind id, name, operations per instruction)
    (0, "v_mfma_f32_16x16x32_bf16", 16 * 16 * 32 * 2),
    (1, "v_mfma_f32_32x32x16_bf16", 32 * 32 * 16 * 2),
    (2, "v_mfma_i32_16x16x64_i8", 16 * 16 * 64 * 2),
    (3, "v_mfma_i32_32x32x32_i8", 32 * 32 * 32 * 2),
    (4, "v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3)", 16 * 16 * 128 * 2),
    (5, "v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3)", 32 * 32 * 64 * 2),
    (6, "v_mfma_f32_16x16x4_f32", 16 * 16 * 4 * 2),
]


def build() -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    # MFMA results in VGPRs: in the accumulator-register form the compiler
    # rotates the 16x16 probes' four-register accumulators through
    # v_accvgpr moves between the MFMAs, and the loop then times those moves
    # (about half the 16x16 shapes' real rate) instead of the matrix cores.
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-mfma-vgpr-form", SRC, "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"hipcc failed for {SRC}:\n{r.stderr}")
    return LIB


def _lib():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built: call bit_gemm_w4_amd.probes.build()")
    L = ctypes.CDLL(LIB)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.probe_mfma.argtypes = [i32, i32, vp, i32, i32, vp]
    L.probe_lds.argtypes = [vp, i32, i32, vp]
    L.probe_stream.argtypes = [i32, vp, i64, vp, i32, i32, vp]
    L.probe_empty.argtypes = [vp]
    L.probe_read_once.argtypes = [i32, i32, vp, i64, vp, i32, vp]
    return L


def _time(torch, launch, reps=3):
    launch(4)                                            # warm: clocks, code load
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        launch(None)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3
        best = t if best is None or t < best else best
    return best


def run():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("the probes need a GPU")
    L = _lib()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    blocks = 512                                         # two blocks of 4 waves per CU: two waves per SIMD
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    po = ctypes.c_void_p(out.data_ptr())
    rows = []
    for kind, name, ops in MFMA_KINDS:
        iters = 2000
        t = _time(torch, lambda it: L.probe_mfma(kind, 8, po, blocks, it or iters, s))
        n = blocks * 4 * iters * 8                       # instructions
        rows.append((name, f"{n * ops / t / 1e12:,.0f} TOP/s",
                     f"{t * CLOCK_GHZ * 1e9 / (n / SIMDS):.1f} cycles per instruction per SIMD at {CLOCK_GHZ} GHz"))
    # dependent chains: one wave per SIMD, each MFMA accumulating into the
    # result of the MFMA nacc instructions before it
    for kind, name, ops in MFMA_KINDS[:4]:
        for nacc in (1, 2, 4):
            iters = 16000 // nacc
            t = _time(torch, lambda it: L.probe_mfma(kind, nacc, po, blocks // 2, it or iters, s))
            n = blocks // 2 * 4 * iters * nacc
            rows.append((f"{name}, {nacc} chain{'s' if nacc > 1 else ''}, one wave per SIMD",
                         f"{n * ops / t / 1e12:,.0f} TOP/s",
                         f"{t * CLOCK_GHZ * 1e9 / (n / SIMDS):.1f} cycles per instruction per SIMD at {CLOCK_GHZ} GHz"))
    iters = 4000
    t = _time(torch, lambda it: L.probe_lds(po, blocks, it or iters, s))
    b = blocks * 256 * 16 * 8 * iters
    rows.append(("LDS ds_read_b128, 2 blocks per CU", f"{b / t / 1e12:.1f} TB/s", f"{b / t / 256 / (CLOCK_GHZ * 1e9):.0f} B per clock per CU"))
    for mib in (2, 128):
        src = torch.randint(0, 255, (mib << 20,), dtype=torch.uint8, device="cuda")
        for to_lds, how in ((0, "into registers"), (1, "by buffer_load ... lds")):
            iters = 400 if mib == 2 else 100
            t = _time(torch, lambda it: L.probe_stream(to_lds, ctypes.c_void_p(src.data_ptr()), src.numel(), po,
                                                       blocks, it or iters, s))
            b = blocks * 4 * 16 * 1024 * iters
            rows.append((f"stream {mib} MiB buffer {how}", f"{b / t / 1e12:.1f} TB/s",
                         f"{b / t / 256 / (CLOCK_GHZ * 1e9):.0f} B per clock per CU"))
        del src
    return rows


def _graph_us(torch, launches, replays=40):
    """Microseconds per launch of `launches` (callables taking a stream
    handle) captured together in one HIP graph: warm replays first (clocks
    ramp up from idle), then the median of five timed batches."""
    s = torch.cuda.Stream()
    h = ctypes.c_void_p(s.cuda_stream)
    with torch.cuda.stream(s):
        for f in launches:
            f(h)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for f in launches:
            f(h)
    torch.cuda.synchronize()
    for _ in range(replays):
        g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            e0.record(s)
            for _ in range(replays):
                g.replay()
            e1.record(s)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / replays / len(launches))
    return sorted(ts)[2]


def _read_once_us(torch, L, nbytes, tag, grids=(256, 512, 1024, 2048, 4096), depths=(4, 8, 16, 32)):
    """Best (us per launch, blocks, depth, copies) of a plain read of nbytes,
    graph-replayed over copies rotated past the last-level cache, over a few
    grids and load depths (16-byte loads in flight per thread)."""
    nbytes = (nbytes + 15) // 16 * 16
    copies = max(2, (512 << 20) // nbytes + 1)
    out = torch.empty(max(grids) * 256, dtype=torch.float32, device="cuda")
    po = ctypes.c_void_p(out.data_ptr())
    bufs = [torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda") for _ in range(copies)]
    best = None
    for depth in depths:
        for blocks in grids:
            t = _graph_us(torch, [lambda h, b=b, n=blocks, d=depth: L.probe_read_once(
                tag, d, ctypes.c_void_p(b.data_ptr()), nbytes, po, n, h) for b in bufs], replays=10)
            best = (t, blocks, depth, copies) if best is None or t < best[0] else best
    del bufs
    torch.cuda.empty_cache()
    return best


def hbm_read_tbps(torch, L):
    """Best read rate from HBM: a 1 GiB buffer (past the 256 MB last-level
    cache) streamed by the read-once kernel (best grid and depth) and by the
    long-running strided stream kernel (16 pieces of 1 KB in flight per wave,
    about 4 GiB read per launch)."""
    t, _, _, _ = _read_once_us(torch, L, 1 << 30, 0, grids=(1024, 2048, 4096, 8192))
    best = (1 << 30) / t / 1e6
    n = 1 << 30
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for blocks in (1024, 2048, 4096):
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
        po = ctypes.c_void_p(out.data_ptr())
        iters = 4 * n // (blocks * 4 * 16 * 1024)
        tk = _time(torch, lambda it: L.probe_stream(0, ctypes.c_void_p(src.data_ptr()), n, po, blocks, it or iters, s))
        best = max(best, blocks * 4 * 16 * 1024 * iters / tk / 1e12)
    del src
    torch.cuda.empty_cache()
    return best


def measured_peaks(torch):
    """Live ceilings of this device: the best HBM read rate (hbm_read_tbps)
    and the MFMA rates of the 32x32 BF16, INT8 and FP8 shapes (eight
    independent chains per wave, two waves per SIMD)."""
    L = _lib()
    hbm = hbm_read_tbps(torch, L)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    blocks = 512
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    po = ctypes.c_void_p(out.data_ptr())
    mfma = {}
    for kind, key in ((1, "bf16"), (3, "i8"), (5, "fp8")):
        ops = next(o for k, _, o in MFMA_KINDS if k == kind)
        iters = 2000
        tk = _time(torch, lambda it: L.probe_mfma(kind, 8, po, blocks, it or iters, s))
        mfma[key] = round(blocks * 4 * iters * 8 * ops / tk / 1e12, 1)
    return {"hbm_read_gbps": round(hbm * 1e3, 1), "mfma_tflops": mfma}


def layer_floors_us(torch):
    """Per Llama-3-8B layer: microseconds of a plain read of its packed W4
    bytes (best grid), graph-replayed past the last-level cache."""
    from . import synth
    L = _lib()
    res = {}
    for tag, name in enumerate(("qkv", "o", "gate_up", "down")):
        K, N = synth.LLAMA3_8B_SHAPES[name]
        res[name] = round(_read_once_us(torch, L, N * K // 2 + N * K // 128 * 2 + N * K // 256, tag)[0], 3)
    return res


def floors():
    """Rows (what, us per launch, rate) of the launch and streaming floors."""
    import torch
    from . import synth
    if not torch.cuda.is_available():
        raise RuntimeError("the probes need a GPU")
    L = _lib()
    rows = []
    t = _graph_us(torch, [lambda h: L.probe_empty(h)] * 100)
    rows.append(("empty kernel (1 block), per launch in a graph of 100", f"{t:.2f} us", "-"))
    for tag, name in enumerate(("qkv", "o", "gate_up", "down")):
        K, N = synth.LLAMA3_8B_SHAPES[name]
        nbytes = N * K // 2 + N * K // 128 * 2 + N * K // 256      # packed codes, FP16 scales, 4-bit zeros
        t, blocks, depth, copies = _read_once_us(torch, L, nbytes, tag)
        rows.append((f"read once: {name}'s packed W4 bytes ({nbytes / 1e6:.2f} MB), {copies} copies rotated, "
                     f"best of 5 grids x 4 depths ({blocks} blocks, {depth} loads in flight)", f"{t:.2f} us",
                     f"{nbytes / t / 1e3:,.0f} GB/s"))
    rows.append(("HBM read rate: 1 GiB buffer, best of the read-once and the strided stream kernel", "-",
                 f"{hbm_read_tbps(torch, L) * 1e3:,.0f} GB/s"))
    return rows


def main():
    import sys
    if not os.path.exists(LIB):
        build()
    if "--floors" not in sys.argv:
        rows = run()
        print("| probe | rate | per unit |")
        print("|---|---|---|")
        for r in rows:
            print(f"| {r[0]} | {r[1]} | {r[2]} |")
        print()
    print("| floor | time | rate |")
    print("|---|---|---|")
    for r in floors():
        print(f"| {r[0]} | {r[1]} | {r[2]} |")


if __name__ == "__main__":
    main()
