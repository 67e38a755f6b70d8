#!/usr/bin/env python3
"""Benchmark of the W4A16 / W8A8 quantized linear layer on one MI355X.

One step = the W4A16 decode linears of a Llama-3-8B-shaped decoder layer
(qkv 4096->6144, o 4096->4096, gate_up 4096->28672, down 14336->4096) at
batch B = 1, 4 and 16, on asymmetric INT4 weights (G=128, FP16 scales, 4-bit
zero-points), BF16 activations: 12 gemm_w4a16 calls.  `value` is the
algorithmic HBM bytes of a step (packed weights + scales + zeros +
activations + outputs) divided by the step time, in GB/s.

Inputs are resident in HBM before timing.  Each layer has R packed copies and
every call reads a different copy, so a weight copy is read again only after
~0.9 GB of other traffic: MI355X's 256 MB Infinity Cache cannot serve it.
Steps are captured into HIP graphs (one per rotation phase) and replayed, so
host launch overhead stays out of the timed region.

Also reported (one JSON line, rank 0): the roofline of the dominant kernel
(HIP-event timing of that kernel alone), the oracle timed on the host cores
on a bounded sample, and secondary results: W8A8 INT8 / FP8 TFLOP/s at
M=2048 and the W4A16 large-batch points.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BATCHES = (1, 4, 16)
LAYERS = ("qkv", "o", "gate_up", "down")
R_COPIES = 8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the live device ceilings (thousands of probe launches: leave them out of profiled runs)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for cpu_baseline")
    ap.add_argument("--large-m-once", action="store_true",
                    help="run each large-M GEMM three times untimed (for counter collection) and exit")
    return ap.parse_args()


def graph_of(fn, torch):
    """Capture fn() into a CUDA/HIP graph on a side stream (after a warm call)."""
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


def time_graph(g, reps, torch, trials=5, warm_ms=20.0, trial_ms=2.0):
    """Milliseconds per replay of g, HIP events on the replay stream: replays
    for about warm_ms first (the clocks ramp up from idle), then the median of
    `trials` runs of at least `reps` replays and at least trial_ms each."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    g.replay()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    one = max(e0.elapsed_time(e1), 1e-3)
    for _ in range(min(5000, int(warm_ms / one) + 2)):
        g.replay()
    n = max(reps, min(5000, int(trial_ms / one) + 1))
    ts = []
    for _ in range(trials):
        e0.record()
        for _ in range(n):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / n)
    return sorted(ts)[len(ts) // 2]


def per_call(fns, reps, torch):
    """Milliseconds per call of the calls in fns, captured together in one
    graph: a graph holding one short call would time the graph launch."""
    g = graph_of(lambda: [f() for f in fns], torch)
    return time_graph(g, reps, torch) / len(fns)


def rotated(t, min_bytes=320 << 20):
    """t and enough copies of it that they do not all fit the 256 MB MALL."""
    n = max(1, -(-min_bytes // (t.numel() * t.element_size())))
    return [t] + [t.clone() for _ in range(n - 1)]


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures a single GPU, so --gpus must be 1 (the path would shard column-parallel "
              "across GPUs, each owning a slice of the output channels, with no exchange between them)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from bit_gemm_w4_amd import ops, roofline, synth
    if not os.path.exists(ops.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.large_m_once:
        large_m_once(ops, synth, torch, np, dev)
        return

    # ------------------------------------------------------------ inputs ----
    t0 = time.time()
    packs, xs, ys, w_host = {}, {}, {}, {}
    for name in LAYERS:
        K, N = synth.LLAMA3_8B_SHAPES[name]
        w, x = synth.decode_layer(max(BATCHES), N, K, seed=0)
        w_host[name] = w
        wd = torch.from_numpy(w).to(dev)
        p0 = ops.w4_pack(wd, 128, True)
        del wd
        copies = [p0]
        for _ in range(R_COPIES - 1):
            copies.append(ops.PackedW4(p0.qweight.clone(), p0.scales.clone(), p0.zeros.clone(), N, K))
        packs[name] = copies
        xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        for B in BATCHES:
            xs[(name, B)] = xt[:B].contiguous()
            ys[(name, B)] = torch.empty((B, N), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s; {R_COPIES} copies/layer, "
        f"{sum(p.nbytes for c in packs.values() for p in c) / 1e9:.2f} GB of packed weights")

    calls = [(name, B) for B in BATCHES for name in LAYERS]
    call_bytes = {c: roofline.w4a16_bytes(c[1], *reversed(synth.LLAMA3_8B_SHAPES[c[0]])) for c in calls}
    step_bytes = sum(call_bytes.values())
    uses_per_step = len(BATCHES)                       # each layer is read once per batch size
    n_phases = R_COPIES // np.gcd(R_COPIES, uses_per_step)

    def step(phase):
        for i, (name, B) in enumerate(calls):
            b_idx = BATCHES.index(B)
            copy = (phase * uses_per_step + b_idx) % R_COPIES
            ops.gemm_w4a16(xs[(name, B)], packs[name][copy], out=ys[(name, B)])

    graphs = [graph_of(lambda ph=ph: step(ph), torch) for ph in range(n_phases)]

    # ------------------------------------------------------- timed steps ----
    for s in range(args.warmup):
        graphs[s % n_phases].replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(args.steps):
        graphs[s % n_phases].replay()
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"step: {ms_per_step * 1e3:.1f} us, {step_bytes / 1e6:.1f} MB algorithmic -> {value:.0f} GB/s")

    # ------------------------------------------- per-call / per-kernel timing ----
    per_call = {}
    kernel_of = {}
    for name, B in calls:
        def one(name=name, B=B):
            for c in range(R_COPIES):
                ops.gemm_w4a16(xs[(name, B)], packs[name][c], out=ys[(name, B)])
        ops.gemm_w4a16(xs[(name, B)], packs[name][0], out=ys[(name, B)])
        kernel_of[(name, B)] = call_kernels(ops, ops.last_kernel(), B, *reversed(synth.LLAMA3_8B_SHAPES[name]))
        g = graph_of(one, torch)
        ms = time_graph(g, 20, torch) / R_COPIES
        per_call[(name, B)] = ms
        log(f"  {name:8s} B={B:3d} {ms * 1e3:8.2f} us {call_bytes[(name, B)] / ms / 1e6:8.0f} GB/s  "
            f"{kernel_of[(name, B)]}")
    by_kernel = {}
    for c, k in kernel_of.items():
        t, b, n = by_kernel.get(k, (0.0, 0, 0))
        by_kernel[k] = (t + per_call[c], b + call_bytes[c], n + 1)
    dom = max(by_kernel, key=lambda k: by_kernel[k][0])
    t_dom, b_dom, n_dom = by_kernel[dom]
    achieved = b_dom / (t_dom * 1e-3) / 1e9
    traffic = measured_traffic(dom)
    roof = {"bound": "hbm", "kernel": dom, "kernels_per_call": len(dom.split(" + ")), "launches_per_step": n_dom,
            "bytes_per_launch": b_dom / n_dom, "avg_launch_us": t_dom / n_dom * 1e3,
            "achieved": round(achieved, 1), "peak": roofline.HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / roofline.HBM_GBPS, 4),
            "traffic": None if traffic is None else round(traffic)}
    calibration_copy(torch, dev)
    ceilings = None if args.no_ceilings else measured_ceilings(torch, calls, ms_per_step)
    if ceilings is not None:
        roof["achievable"] = ceilings["hbm_read_gbps"]
        roof["frac_of_achievable"] = round(achieved / ceilings["hbm_read_gbps"], 4)

    out = {
        "metric": "W4A16/W8A8 linear: HBM GB/s at B=1..16, TFLOPS at M=2048; % of roofline",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int4-weights x bf16 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": "W4A16 decode, Llama-3-8B layer shapes (qkv, o, gate_up, down), "
                               "B in {1,4,16}, asymmetric INT4 G=128 + FP16 scales + 4-bit zeros, "
                               "BF16 activations, 1% input channels x20",
                   "calls_per_step": len(calls), "bytes_per_step": step_bytes,
                   "weight_copies_rotated": R_COPIES, "timing": "HIP graph replay"},
        "roofline": roof,
        "measured_ceilings": ceilings,
        "per_call_gbps": {f"{n}@B{B}": round(call_bytes[(n, B)] / per_call[(n, B)] / 1e6, 1) for n, B in calls},
    }

    # -------------------------------------------------------- secondary ----
    if not args.no_secondary:
        out["secondary"] = secondary(ops, synth, roofline, torch, np, dev, packs, graph_of, time_graph)
        out["secondary"]["crossover_down"] = crossover(ops, synth, roofline, torch, np, dev, graph_of, time_graph)
        out["secondary"]["qwen_1024_b1"] = qwen_single(ops, synth, roofline, torch, np, dev, graph_of, time_graph)
        out["secondary"]["w8a8_decode"] = w8a8_decode(ops, synth, roofline, torch, np, dev, graph_of, time_graph)
        out["secondary"]["fp8_prefill_m"] = fp8_sizes(ops, synth, roofline, torch, np, dev, graph_of, time_graph)
        out["secondary"]["tensor_metrics"] = tensor_metrics(ops, synth, torch, np, dev, packs)

    # ----------------------------------------------------- cpu baseline ----
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w_host, xs, calls, args.cpu_seconds, np, synth, roofline)

    print(json.dumps(out), flush=True)


def measured_ceilings(torch, calls, ms_per_step):
    """What this device reaches, measured in the same run with the probe
    kernels (bit_gemm_w4_amd/csrc_probes): a plain read of a 1 GiB buffer,
    the MFMA-only rates of the 32x32 BF16 / INT8 / FP8 shapes, and the
    step's streaming floor -- the sum over its calls of a plain read of the
    call's packed weight bytes, graph-replayed past the last-level cache.
    None when the probe library is not built."""
    from bit_gemm_w4_amd import probes
    if not os.path.exists(probes.LIB):
        log("probe library not built: no measured ceilings")
        return None
    peaks = probes.measured_peaks(torch)
    floors = probes.layer_floors_us(torch)
    floor_us = sum(floors[name] for name, _ in calls)
    step_us = ms_per_step * 1e3
    res = dict(peaks, layer_read_floor_us=floors, step_read_floor_us=round(floor_us, 2),
               step_frac_of_read_floor=round(floor_us / step_us, 4))
    log(f"measured ceilings: read {peaks['hbm_read_gbps']:.0f} GB/s, MFMA {peaks['mfma_tflops']}; "
        f"step read floor {floor_us:.1f} us ({floor_us / step_us:.1%} of the step)")
    return res


CALIB_BYTES = 512 << 20
TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "hbm_traffic_w4a16_decode_llama3_8b.md")


def large_m_once(ops, synth, torch, np, dev):
    """Each large-M GEMM of the M = 2048 prefill rows, three times, untimed, for
    counter collection: W8A8 INT8 per token x per channel and W4A8 (the packed
    INT4 weights) on the four projections, FP8 per-tensor, 128 x 128 block,
    MXFP8 and MXFP4 on gate_up and down, W4A16 on the four projections.  Every
    call runs once first (workspaces, code loading); the manifest on stdout
    names the calls in order, then the plain copy that calibrates FETCH_SIZE /
    WRITE_SIZE runs."""
    M = 2048
    jobs, keep = [], []
    for name in LAYERS:
        K, N = synth.LLAMA3_8B_SHAPES[name]
        w, x = synth.prefill_layer(M, N, K, seed=0)
        xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        wt = torch.from_numpy(w).to(dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        a8, s8 = ops.act_quant_int8(xt, ops.GRAN_ROW)
        w8, sw8 = ops.act_quant_int8(wt, ops.GRAN_ROW)
        p = ops.w4_pack(wt, 128, True)
        keep += [xt, wt, y, a8, s8, w8, sw8, p]
        jobs.append((f"W8A8 INT8 {name}", lambda a=a8, s=s8, w=w8, sw=sw8, y=y:
                     ops.gemm_w8a8(a, s, ops.GRAN_ROW, w, sw, ops.GRAN_ROW, out=y)))
        if name in ("gate_up", "down"):
            for tag, ag, wg in (("FP8 tensor", ops.GRAN_TENSOR, ops.GRAN_TENSOR),
                                ("FP8 block", ops.GRAN_ROW_G128, ops.GRAN_BLOCK128)):
                af, sf = ops.act_quant_fp8(xt, ag)
                wf, swf = ops.act_quant_fp8(wt, wg)
                keep += [af, sf, wf, swf]
                jobs.append((f"W8A8 {tag} {name}", lambda a=af, s=sf, w=wf, sw=swf, ag=ag, wg=wg, y=y:
                             ops.gemm_w8a8(a, s, ag, w, sw, wg, out=y)))
            am, em = ops.act_quant_mxfp8(xt)
            wm, ewm = ops.act_quant_mxfp8(wt)
            a4, e4 = ops.act_quant_mxfp4(xt)
            w4, ew4 = ops.act_quant_mxfp4(wt)
            keep += [am, em, wm, ewm, a4, e4, w4, ew4]
            jobs.append((f"MXFP8 {name}", lambda a=am, e=em, w=wm, ew=ewm, y=y: ops.gemm_mxfp8(a, e, w, ew, out=y)))
            jobs.append((f"MXFP4 {name}", lambda a=a4, e=e4, w=w4, ew=ew4, y=y: ops.gemm_mxfp4(a, e, w, ew, out=y)))
        jobs.append((f"W4A8 {name}", lambda a=a8, s=s8, p=p, y=y: ops.gemm_w4a8(a, s, ops.GRAN_ROW, p, out=y)))
        jobs.append((f"W4A16 {name}", lambda x=xt, p=p, y=y: ops.gemm_w4a16(x, p, out=y)))
    for _, fn in jobs:
        fn()
    torch.cuda.synchronize()
    for label, fn in jobs:
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        print(f"{label}\t{ops.last_kernel()}", flush=True)
    calibration_copy(torch, dev)


def calibration_copy(torch, dev):
    """A plain copy of known size (torch.neg over 512 MiB of FP32: reads and
    writes CALIB_BYTES each) that hardware-counter runs of this script use to
    scale FETCH_SIZE / WRITE_SIZE to bytes.  Not part of any timed region."""
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def library_digest() -> str:
    """sha256 over the HIP sources, so counters taken on other code are not reused."""
    import glob
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bit_gemm_w4_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(csrc, "*"))):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def call_kernels(ops, main: str, M: int, N: int, K: int) -> str:
    """The kernels one gemm_w4a16 call enqueues, joined by " + ": the split-K,
    tiled and mid-batch paths add a fixed-order reduction kernel when they
    split K."""
    if ops.gemm_w4a16_workspace_bytes(M, N, K) > 0 and "k_w4a16_splitk<" in main:
        return main + " + " + main.replace("k_w4a16_splitk<", "k_w4a16_splitk_reduce<")
    if ops.gemm_w4a16_workspace_bytes(M, N, K) > 0 and ("k_w4a16_gemm<" in main or "k_w4a16_mid<" in main):
        return main + " + " + "k_w4a16_gemm_reduce<" + main.split("<", 1)[1].split(",")[0] + ">"
    return main


def measured_traffic(call: str):
    """HBM bytes per call from the committed counter summary (FETCH_SIZE +
    WRITE_SIZE per dispatch, each scaled by the calibration copy, summed over
    the call's kernels), or None when a kernel has no row or the sources
    changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    digest = library_digest()
    rows = {}
    for line in open(TRAFFIC_FILE):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 7 and cells[1] == digest:
            try:
                rows[cells[0].strip("`")] = float(cells[6])
            except ValueError:
                pass
    parts = call.split(" + ")
    if not all(k in rows for k in parts):
        return None
    return sum(rows[k] for k in parts)


def secondary(ops, synth, roofline, torch, np, dev, packs, graph_of, time_graph):
    """W8A8 at M=2048 (INT8 per-token x per-channel; FP8 per-tensor and
    128x128 / 1x128 blocks), W4A8 at M=2048 (the decode step's packed INT4
    weights x per-token INT8 activations) and W4A16 at B=74/256, each timed
    alone."""
    res = {"w8a8_m2048": {}, "w4a8_m2048": {}, "smoothquant_m2048": {}, "llm_int8_m2048": {}, "w4a16_large_batch": {}}
    M = 2048
    for name in LAYERS:
        K, N = synth.LLAMA3_8B_SHAPES[name]
        w, x = synth.prefill_layer(M, N, K, seed=0)
        xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        wt = torch.from_numpy(w).to(dev)
        xrot = rotated(xt)                              # quantizer timings read X from HBM
        variants = [("int8_row", False, 1, 1)]
        if name in ("gate_up", "down"):
            variants += [("fp8_tensor", True, 0, 0), ("fp8_block", True, 2, 3)]
        for tag, fp8, ag, wg in variants:
            quant = ops.act_quant_fp8 if fp8 else ops.act_quant_int8
            a, a_s = quant(xt, ag)
            wq, w_s = quant(wt, wg)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            ms = per_call([lambda: ops.gemm_w8a8(a, a_s, ag, wq, w_s, wg, out=y)] * 4, 10, torch)
            kname = ops.last_kernel()
            ms_q = per_call([lambda x=x: quant(x, ag) for x in xrot], 20, torch)
            tf = roofline.gemm_flops(M, N, K) / (ms * 1e-3) / 1e12
            peak = roofline.PEAK_TFLOPS["fp8" if fp8 else "i8"]
            res["w8a8_m2048"][f"{name}/{tag}"] = {
                "gemm_us": round(ms * 1e3, 1), "tflops": round(tf, 1), "frac": round(tf / peak, 4),
                "act_quant_us": round(ms_q * 1e3, 1),
                "act_quant_gbps": round(roofline.act_quant_bytes(M, K) / (ms_q * 1e-3) / 1e9, 1),
                "kernel": kname}
            log(f"  w8a8 {name:8s} {tag:10s} {ms * 1e3:8.1f} us {tf:7.1f} TFLOP/s ({tf / peak:.1%}) "
                f"act_quant {ms_q * 1e3:6.1f} us")
        res["smoothquant_m2048"][name] = smoothquant(ops, torch, np, dev, xt, wt, x, w, graph_of, time_graph)
        res["llm_int8_m2048"][name] = llm_int8(ops, torch, np, dev, xt, wt, x, w, graph_of, time_graph)
        # W4A8: the same activations as per-token INT8 codes, the packed weights
        a, a_s = ops.act_quant_int8(xt, ops.GRAN_ROW)
        p = packs[name][0]
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ms = per_call([lambda: ops.gemm_w4a8(a, a_s, ops.GRAN_ROW, p, out=y)] * 4, 10, torch)
        tf = roofline.gemm_flops(M, N, K) / (ms * 1e-3) / 1e12
        peak = roofline.PEAK_TFLOPS["i8"]
        res["w4a8_m2048"][name] = {"gemm_us": round(ms * 1e3, 1), "tflops": round(tf, 1),
                                   "frac": round(tf / peak, 4), "kernel": ops.last_kernel()}
        log(f"  w4a8 {name:8s} {ms * 1e3:8.1f} us {tf:7.1f} TOP/s ({tf / peak:.1%})")
        if name in ("gate_up", "down"):
            # MXFP8: E8M0 scales per 32 K elements, applied by the MFMA
            a, ea = ops.act_quant_mxfp8(xt)
            q, ew = ops.act_quant_mxfp8(wt)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            ms = per_call([lambda: ops.gemm_mxfp8(a, ea, q, ew, out=y)] * 4, 10, torch)
            kname = ops.last_kernel()
            ms_q = per_call([lambda x=x: ops.act_quant_mxfp8(x) for x in xrot], 20, torch)
            tf = roofline.gemm_flops(M, N, K) / (ms * 1e-3) / 1e12
            peak = roofline.PEAK_TFLOPS["fp8"]
            res["w8a8_m2048"][f"{name}/mxfp8"] = {
                "gemm_us": round(ms * 1e3, 1), "tflops": round(tf, 1), "frac": round(tf / peak, 4),
                "act_quant_us": round(ms_q * 1e3, 1),
                "act_quant_gbps": round(roofline.act_quant_bytes(M, K) / (ms_q * 1e-3) / 1e9, 1),
                "kernel": kname}
            log(f"  w8a8 {name:8s} {'mxfp8':10s} {ms * 1e3:8.1f} us {tf:7.1f} TFLOP/s ({tf / peak:.1%}) "
                f"act_quant {ms_q * 1e3:6.1f} us")
            # MXFP4: E2M1 elements in both operands, the same E8M0 blocks
            a, ea = ops.act_quant_mxfp4(xt)
            q, ew = ops.act_quant_mxfp4(wt)
            ms = per_call([lambda: ops.gemm_mxfp4(a, ea, q, ew, out=y)] * 4, 10, torch)
            kname = ops.last_kernel()
            ms_q = per_call([lambda x=x: ops.act_quant_mxfp4(x) for x in xrot], 20, torch)
            tf = roofline.gemm_flops(M, N, K) / (ms * 1e-3) / 1e12
            peak = roofline.PEAK_TFLOPS["fp4"]
            qbytes = M * K * 2 + M * K // 2 + M * K // 32
            res["w8a8_m2048"][f"{name}/mxfp4"] = {
                "gemm_us": round(ms * 1e3, 1), "tflops": round(tf, 1), "frac": round(tf / peak, 4),
                "act_quant_us": round(ms_q * 1e3, 1),
                "act_quant_gbps": round(qbytes / (ms_q * 1e-3) / 1e9, 1),
                "kernel": kname}
            log(f"  w8a8 {name:8s} {'mxfp4':10s} {ms * 1e3:8.1f} us {tf:7.1f} TFLOP/s ({tf / peak:.1%}) "
                f"act_quant {ms_q * 1e3:6.1f} us")
        del wt
    for name in LAYERS:
        K, N = synth.LLAMA3_8B_SHAPES[name]
        for B in (74, 256):
            x = synth.activations(B, K, "bf16", seed=1)
            xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
            y = torch.empty((B, N), dtype=torch.bfloat16, device=dev)
            ms = per_call([lambda p=p: ops.gemm_w4a16(xt, p, out=y) for p in packs[name]], 10, torch)
            tf = roofline.gemm_flops(B, N, K) / (ms * 1e-3) / 1e12
            res["w4a16_large_batch"][f"{name}@B{B}"] = {
                "us": round(ms * 1e3, 1), "tflops": round(tf, 1), "frac_bf16_peak": round(tf / 2500.0, 4),
                "kernel": ops.last_kernel()}
            log(f"  w4a16 {name:8s} B={B:3d} {ms * 1e3:8.1f} us {tf:7.1f} TFLOP/s")
    return res


def qwen_single(ops, synth, roofline, torch, np, dev, graph_of, time_graph):
    """The single Qwen3-0.6B-sized linear (K = N = 1024, B = 1, FP16
    activations, symmetric INT4 G=128, FP16 output), rotated over copies that
    exceed the 256 MB last-level cache.  0.54 MB per call: at 8 TB/s that is
    0.07 us, far below the cost of a kernel launch, so the call is bound by
    launch latency and the fraction of the HBM roofline is reported as such."""
    w, x = synth.qwen_layer(seed=0)
    p0 = ops.w4_pack(torch.from_numpy(w).to(dev), 128, False)
    n = -(-(320 << 20) // p0.nbytes)
    cps = [p0] + [ops.PackedW4(p0.qweight.clone(), p0.scales.clone(), None, 1024, 1024) for _ in range(n - 1)]
    xt = torch.from_numpy(x.view(np.int16)).view(torch.float16).to(dev)
    y = torch.empty((1, 1024), dtype=torch.float16, device=dev)
    g = graph_of(lambda: [ops.gemm_w4a16(xt, c, out=y) for c in cps], torch)
    ms = time_graph(g, 20, torch) / len(cps)
    byts = roofline.w4a16_bytes(1, 1024, 1024, asym=False)
    gbps = byts / (ms * 1e-3) / 1e9
    log(f"  qwen 1024x1024 B=1 fp16 sym: {ms * 1e3:.2f} us {gbps:.0f} GB/s ({gbps / roofline.HBM_GBPS:.1%}, launch-bound)")
    return {"us": round(ms * 1e3, 2), "bytes": byts, "gbps": round(gbps, 1),
            "frac": round(gbps / roofline.HBM_GBPS, 4), "bound": "launch latency (0.07 us of HBM time at 8 TB/s)",
            "kernel": ops.last_kernel()}


def w8a8_decode(ops, synth, roofline, torch, np, dev, graph_of, time_graph):
    """W8A8 at decode batches B = 1, 4, 16 on the four projection shapes:
    INT8 (per-token x per-channel) and FP8 (per-tensor), the GEMM alone and
    with the activation quantization it needs, weights rotated over copies
    that exceed the last-level cache.  GB/s = the GEMM call's algorithmic
    bytes (8-bit weights and activations, scales, BF16 output) over its time."""
    res = {}
    for name in LAYERS:
        K, N = synth.LLAMA3_8B_SHAPES[name]
        w = synth.weights(N, K, seed=0)
        wd = torch.from_numpy(w).to(dev)
        n = max(2, -(-(320 << 20) // (N * K)))
        q8, s8 = ops.act_quant_int8(wd, ops.GRAN_ROW)
        qf, sf = ops.act_quant_fp8(wd, ops.GRAN_TENSOR)
        i8 = [(q8, s8)] + [(q8.clone(), s8.clone()) for _ in range(n - 1)]
        f8 = [(qf, sf)] + [(qf.clone(), sf.clone()) for _ in range(n - 1)]
        del wd
        for B in BATCHES:
            x = torch.from_numpy(synth.activations(B, K, "bf16", seed=B).view(np.int16)).view(torch.bfloat16).to(dev)
            y = torch.empty((B, N), dtype=torch.bfloat16, device=dev)
            for tag, fp8, gran, wl in (("int8", False, ops.GRAN_ROW, i8), ("fp8", True, ops.GRAN_TENSOR, f8)):
                quant = ops.act_quant_fp8 if fp8 else ops.act_quant_int8
                a, a_s = quant(x, gran)
                g = graph_of(lambda: [ops.gemm_w8a8(a, a_s, gran, c[0], c[1], gran, out=y) for c in wl], torch)
                ms = time_graph(g, 20, torch) / len(wl)
                kname = ops.last_kernel()
                def with_q():
                    for c in wl:
                        aa, ss = quant(x, gran)
                        ops.gemm_w8a8(aa, ss, gran, c[0], c[1], gran, out=y)
                ms_q = time_graph(graph_of(with_q, torch), 20, torch) / len(wl)
                byts = roofline.w8a8_bytes(B, N, K, w_scales=1 if fp8 else None)
                gbps = byts / (ms * 1e-3) / 1e9
                res[f"{name}/{tag}@B{B}"] = {"gemm_us": round(ms * 1e3, 2), "gbps": round(gbps, 1),
                                             "frac": round(gbps / roofline.HBM_GBPS, 4),
                                             "with_act_quant_us": round(ms_q * 1e3, 2), "kernel": kname}
                log(f"  w8a8 decode {name:8s} {tag:4s} B={B:2d} {ms * 1e3:7.2f} us {gbps:6.0f} GB/s "
                    f"({gbps / roofline.HBM_GBPS:.1%}); with act_quant {ms_q * 1e3:7.2f} us  {kname}")
        del i8, f8
    return res


def fp8_sizes(ops, synth, roofline, torch, np, dev, graph_of, time_graph):
    """FP8 E4M3 W8A8 at the other prefill sizes of the FP8 workload, M = 512
    and 8192 (M = 2048 is with the other prefill rows), on gate_up and down:
    (a) per-tensor scales, (b) 128 x 128 weight blocks with 1 x 128 activation
    groups."""
    res = {}
    for name in ("gate_up", "down"):
        K, N = synth.LLAMA3_8B_SHAPES[name]
        w = synth.weights(N, K, seed=0)
        wt = torch.from_numpy(w).to(dev)
        for M in (512, 8192):
            x = synth.activations(M, K, "bf16", seed=M, n_outlier_cols=8)
            xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            for tag, ag, wg in (("tensor", 0, 0), ("block", 2, 3)):
                a, a_s = ops.act_quant_fp8(xt, ag)
                wq, w_s = ops.act_quant_fp8(wt, wg)
                ms = per_call([lambda: ops.gemm_w8a8(a, a_s, ag, wq, w_s, wg, out=y)] * 2, 10, torch)
                tf = roofline.gemm_flops(M, N, K) / (ms * 1e-3) / 1e12
                peak = roofline.PEAK_TFLOPS["fp8"]
                res[f"{name}/fp8_{tag}@M{M}"] = {"gemm_us": round(ms * 1e3, 1), "tflops": round(tf, 1),
                                                 "frac": round(tf / peak, 4), "kernel": ops.last_kernel()}
                log(f"  fp8 {name:8s} {tag:6s} M={M:5d} {ms * 1e3:8.1f} us {tf:7.1f} TFLOP/s ({tf / peak:.1%})")
            del xt, y
        del wt
    return res


def w4_codes(qweight, scales, zeros, np):
    """4-bit codes [N][K] and dequantized weights (u - z) * s of the tiled
    w4_pack layout, read back on the host: 16 channels x 128-wide group per
    tile; column n, offset c in the group sits in slot 16 * (c / 32) + n % 16,
    word (c % 32) / 8; of the 8 codes of a word, even k fill the low half-word
    and odd k the high one, lowest k in the lowest nibble."""
    T, G = qweight.shape[0], qweight.shape[1]
    N, K = 16 * T, 128 * G
    shifts = np.array([0, 16, 4, 20, 8, 24, 12, 28], dtype=np.uint32)
    qw = qweight.view(np.uint32).reshape(T, G, 4, 16, 4)
    u = ((qw[..., None] >> shifts) & 0xF).transpose(0, 3, 1, 2, 4, 5).reshape(N, K)
    sc = np.asarray(scales).view(np.float16).astype(np.float64).transpose(0, 2, 1).reshape(N, G)
    if zeros is None:
        z = np.full((N, G), 8.0)
    else:
        zb = zeros.transpose(0, 2, 1).reshape(N, G // 2)
        z = np.stack([zb & 0xF, zb >> 4], axis=-1).reshape(N, G).astype(np.float64)
    return u, (u - np.repeat(z, 128, axis=1)) * np.repeat(sc, 128, axis=1)


def tensor_metrics(ops, synth, torch, np, dev, packs, rows=2048):
    """Tensor-level quantization metrics of the benchmark's quantized tensors
    (host-side analysis of the codes the kernels produced): saturation ratio
    (share of codes at the format's extreme magnitude), code utilisation
    (distinct codes used / codes of the format), MSE and cosine similarity of
    the dequantized tensor against the original.  INT8 / FP8 activations
    (per token; 8 channels x50) of the gate_up prefill layer at M = 2048 and
    its weights (per channel, per tensor), and the packed INT4 weights of the
    four decode layers; each tensor is quantized whole and its first `rows`
    rows are analysed."""
    def stats(orig, deq, codes, n_codes, extreme):
        o = orig.astype(np.float64).ravel()
        d = deq.astype(np.float64).ravel()
        cos = float(o @ d / (np.linalg.norm(o) * np.linalg.norm(d) + 1e-300))
        return {"saturation": round(float(np.mean(extreme)), 6),
                "code_utilisation": round(len(np.unique(codes)) / n_codes, 4),
                "mse": float(np.mean((o - d) ** 2)), "cosine": round(cos, 7)}

    def e4m3_value(b):
        b = b.astype(np.int64)
        e, m = (b >> 3) & 0xF, (b & 7).astype(np.float64)
        v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7.0))
        return np.where(b & 0x80, -v, v)

    res = {}
    K, N = synth.LLAMA3_8B_SHAPES["gate_up"]
    w, x = synth.prefill_layer(2048, N, K, seed=0)
    x32 = (x.astype(np.uint32) << 16).view(np.float32)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    wt = torch.from_numpy(w).to(dev)
    cases = (("act_per_token", xt, x32, ops.GRAN_ROW, ("int8", "fp8")),
             ("weight_per_channel", wt, w, ops.GRAN_ROW, ("int8", "fp8")),
             ("weight_per_tensor", wt, w, ops.GRAN_TENSOR, ("fp8",)))
    for tag, t, t32, gran, fmts in cases:
        for fmt in fmts:
            q, s = (ops.act_quant_fp8 if fmt == "fp8" else ops.act_quant_int8)(t, gran)
            qn = q[:rows].cpu().view(torch.uint8 if fmt == "fp8" else torch.int8).numpy()
            sn = s.cpu().numpy().astype(np.float64)
            scale = sn[:rows, None] if gran == ops.GRAN_ROW else sn[0]
            if fmt == "fp8":
                res[f"{tag}/{fmt}"] = stats(t32[:rows], e4m3_value(qn) * scale, qn, 254, (qn & 0x7F) == 0x7E)
            else:
                res[f"{tag}/{fmt}"] = stats(t32[:rows], qn * scale, qn, 255, np.abs(qn.astype(np.int64)) >= 127)
    del xt, wt
    for name in LAYERS:
        Kd, Nd = synth.LLAMA3_8B_SHAPES[name]
        wd = synth.decode_layer(1, Nd, Kd, seed=0)[0][:rows]
        p, T = packs[name][0], rows // 16
        u, deq = w4_codes(p.qweight[:T].cpu().numpy(), p.scales[:T].cpu().numpy(), p.zeros[:T].cpu().numpy(), np)
        res[f"w4_{name}"] = stats(wd, deq, u, 16, (u == 0) | (u == 15))
    log("  tensor metrics: " + ", ".join(f"{k} sat {v['saturation']:.4f} cos {v['cosine']:.5f}" for k, v in res.items()))
    return res


def smoothquant(ops, torch, np, dev, xt, wt, x_bits, w, graph_of, time_graph):
    """The SmoothQuant fold on the INT8 prefill recipe (8 activation channels
    x50): S from the column maxima of 256 calibration rows and of W (alpha =
    1/2), activations quantized with 1/s in the quantizer's load, weights
    folded with s.  Reports the INT8 W8A8 output error against the unquantized
    product (relative L2 over 16 rows outside the calibration rows) without and
    with the fold, for per-token and per-tensor activation scales, and the
    quantizer time with and without the fused column factors."""
    M = xt.shape[0]
    x32 = (x_bits.astype(np.uint32) << 16).view(np.float32)           # BF16 -> binary32, exact
    ax = np.abs(x32[:256]).max(axis=0)
    aw = np.abs(w).max(axis=0)
    ok = (ax > 0) & (aw > 0)
    s = np.where(ok, np.sqrt(ax.astype(np.float64)) / np.sqrt(np.where(ok, aw, 1).astype(np.float64)), 1.0)
    s = s.astype(np.float32)
    inv = (np.float32(1.0) / s).astype(np.float32)
    sd, invd = torch.from_numpy(s).to(dev), torch.from_numpy(inv).to(dev)
    rows = np.linspace(256, M - 1, 16).astype(np.int64)
    exact = x32[rows].astype(np.float64) @ w.astype(np.float64).T
    out = {}
    for tag, ag in (("per_token", ops.GRAN_ROW), ("per_tensor", ops.GRAN_TENSOR)):
        errs = {}
        for fold in (False, True):
            if fold:
                a, a_s = ops.act_quant_int8_smooth(xt, invd, ag)
                wq, w_s = ops.act_quant_int8_smooth(wt, sd, ops.GRAN_ROW)
            else:
                a, a_s = ops.act_quant_int8(xt, ag)
                wq, w_s = ops.act_quant_int8(wt, ops.GRAN_ROW)
            y = ops.gemm_w8a8(a, a_s, ag, wq, w_s, ops.GRAN_ROW, out_dtype=torch.float32)
            yv = y[torch.from_numpy(rows).to(dev)].double().cpu().numpy()
            errs["folded" if fold else "plain"] = float(np.linalg.norm(yv - exact) / np.linalg.norm(exact))
        out[tag] = {k: round(v, 5) for k, v in errs.items()}
    xr = rotated(xt)
    t0 = per_call([lambda x=x: ops.act_quant_int8(x, ops.GRAN_ROW) for x in xr], 20, torch)
    t1 = per_call([lambda x=x: ops.act_quant_int8_smooth(x, invd, ops.GRAN_ROW) for x in xr], 20, torch)
    out["act_quant_us"] = {"plain": round(t0 * 1e3, 1), "folded": round(t1 * 1e3, 1)}
    log(f"  smoothquant rel-L2 err per-token {out['per_token']['plain']:.4f} -> {out['per_token']['folded']:.4f}, "
        f"per-tensor {out['per_tensor']['plain']:.4f} -> {out['per_tensor']['folded']:.4f}; act_quant "
        f"{out['act_quant_us']['plain']} -> {out['act_quant_us']['folded']} us")
    return out


def llm_int8(ops, torch, np, dev, xt, wt, x_bits, w, graph_of, time_graph, tau=6.0):
    """The LLM.int8() split on the INT8 prefill recipe (8 activation channels
    x50): outlier channels with max |x| >= tau go to the side path, the rest
    to per-token INT8 (per-channel INT8 weights).  Reports the output error
    against the unquantized product (relative L2 over 16 rows) of plain
    per-token W8A8 and of the split, the outlier count, and the times of
    detection + quantization and of the GEMM with the fused side path against
    plain per-token quantization and GEMM."""
    M, N = xt.shape[0], wt.shape[0]
    x32 = (x_bits.astype(np.uint32) << 16).view(np.float32)           # BF16 -> binary32, exact
    rows = np.linspace(0, M - 1, 16).astype(np.int64)
    exact = x32[rows].astype(np.float64) @ w.astype(np.float64).T
    ridx = torch.from_numpy(rows).to(dev)
    wq, w_s = ops.act_quant_int8(wt, ops.GRAN_ROW)
    a, a_s = ops.act_quant_int8(xt, ops.GRAN_ROW)
    y0 = ops.gemm_w8a8(a, a_s, ops.GRAN_ROW, wq, w_s, ops.GRAN_ROW, out_dtype=torch.float32)
    q, sa, idx, cnt = ops.act_quant_int8_outlier(xt, tau)
    y1 = ops.gemm_w8a8_outlier(q, sa, wq, w_s, ops.GRAN_ROW, xt, idx, cnt, out_dtype=torch.float32)
    e0 = float(np.linalg.norm(y0[ridx].double().cpu().numpy() - exact) / np.linalg.norm(exact))
    e1 = float(np.linalg.norm(y1[ridx].double().cpu().numpy() - exact) / np.linalg.norm(exact))
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    t = {}
    xr = rotated(xt)
    t["plain_quant_us"] = per_call([lambda x=x: ops.act_quant_int8(x, ops.GRAN_ROW) for x in xr], 20, torch)
    t["plain_gemm_us"] = per_call(
        [lambda: ops.gemm_w8a8(a, a_s, ops.GRAN_ROW, wq, w_s, ops.GRAN_ROW, out=y)] * 4, 10, torch)
    t["detect_quant_us"] = per_call([lambda x=x: ops.act_quant_int8_outlier(x, tau) for x in xr], 20, torch)
    t["gemm_side_us"] = per_call(
        [lambda: ops.gemm_w8a8_outlier(q, sa, wq, w_s, ops.GRAN_ROW, xt, idx, cnt, out=y)] * 4, 10, torch)
    kname = ops.last_kernel()
    out = {"tau": tau, "outlier_channels": int(cnt.item()), "err_plain": round(e0, 5), "err_split": round(e1, 5)}
    out.update({k: round(v * 1e3, 1) for k, v in t.items()})
    out["kernel"] = kname
    log(f"  llm.int8 {out['outlier_channels']} ch: rel-L2 err {e0:.4f} -> {e1:.4f}; quant {out['plain_quant_us']} -> "
        f"{out['detect_quant_us']} us, gemm {out['plain_gemm_us']} -> {out['gemm_side_us']} us")
    return out


def crossover(ops, synth, roofline, torch, np, dev, graph_of, time_graph):
    """Down-projection shape (K=14336, N=4096), B = 1, 2, 4, ..., 4096: a BF16
    GEMM (torch.matmul, the library GEMM) against W4A16 (asymmetric INT4, G=128)
    and W8A8 INT8 (per-token x per-channel) and FP8 (per-tensor), the W8A8
    times including the activation quantization they need.  Weights are
    rotated over copies that together exceed the 256 MB last-level cache, so
    every call reads them from HBM.  Returns the times and the first batch
    where each W8A8 variant beats W4A16."""
    K, N = synth.LLAMA3_8B_SHAPES["down"]
    w = synth.weights(N, K, seed=0, outlier_frac=0.01)
    wd = torch.from_numpy(w).to(dev)
    def copies(nbytes):
        return max(2, -(-(320 << 20) // nbytes))
    p0 = ops.w4_pack(wd, 128, True)
    w4 = [p0] + [ops.PackedW4(p0.qweight.clone(), p0.scales.clone(), p0.zeros.clone(), N, K)
                 for _ in range(copies(p0.nbytes) - 1)]
    q8, s8 = ops.act_quant_int8(wd, ops.GRAN_ROW)
    i8 = [(q8, s8)] + [(q8.clone(), s8.clone()) for _ in range(copies(N * K) - 1)]
    qf, sf = ops.act_quant_fp8(wd, ops.GRAN_TENSOR)
    f8 = [(qf, sf)] + [(qf.clone(), sf.clone()) for _ in range(copies(N * K) - 1)]
    wb = wd.to(torch.bfloat16)
    bf = [wb] + [wb.clone() for _ in range(copies(2 * N * K) - 1)]
    del wd
    rows, res = [], {"batches": [], "us": {"bf16": [], "w4a16": [], "w4a8": [], "w8a8_int8": [], "w8a8_fp8": []}}
    for lb in range(13):
        B = 1 << lb
        g = torch.Generator(device="cpu")
        g.manual_seed(lb)
        x = torch.randn((B, K), generator=g).to(torch.bfloat16).to(dev)
        y = torch.empty((B, N), dtype=torch.bfloat16, device=dev)
        def t_of(fn, n):
            gr = graph_of(lambda: [fn(c) for c in range(n)], torch)
            return time_graph(gr, 5, torch) / n * 1e3
        def i8_call(c):
            a, a_s = ops.act_quant_int8(x, ops.GRAN_ROW)
            ops.gemm_w8a8(a, a_s, ops.GRAN_ROW, i8[c][0], i8[c][1], ops.GRAN_ROW, out=y)
        def w4a8_call(c):
            a, a_s = ops.act_quant_int8(x, ops.GRAN_ROW)
            ops.gemm_w4a8(a, a_s, ops.GRAN_ROW, w4[c], out=y)
        def f8_call(c):
            a, a_s = ops.act_quant_fp8(x, ops.GRAN_TENSOR)
            ops.gemm_w8a8(a, a_s, ops.GRAN_TENSOR, f8[c][0], f8[c][1], ops.GRAN_TENSOR, out=y)
        t = {"bf16": t_of(lambda c: torch.matmul(x, bf[c].t(), out=y), len(bf)),
             "w4a16": t_of(lambda c: ops.gemm_w4a16(x, w4[c], out=y), len(w4)),
             "w4a8": t_of(w4a8_call, len(w4)),
             "w8a8_int8": t_of(i8_call, len(i8)),
             "w8a8_fp8": t_of(f8_call, len(f8))}
        res["batches"].append(B)
        for k, v in t.items():
            res["us"][k].append(round(v, 2))
        log(f"  crossover down B={B:5d}  bf16 {t['bf16']:8.1f}  w4a16 {t['w4a16']:8.1f}  w4a8 {t['w4a8']:8.1f}  "
            f"int8 {t['w8a8_int8']:8.1f}  fp8 {t['w8a8_fp8']:8.1f} us")
    for k in ("w4a8", "w8a8_int8", "w8a8_fp8"):
        won = [B for B, a, b in zip(res["batches"], res["us"][k], res["us"]["w4a16"]) if a < b]
        res[f"crossover_batch_{k}"] = won[0] if won else None
    res["roofline_crossover_batch"] = round(roofline.PEAK_TFLOPS["bf16"] * 1e12 / (2 * roofline.HBM_GBPS * 1e9), 1)
    return res


def cpu_baseline(w_host, xs, calls, target_s, np, synth, roofline):
    """The oracle's W4A16 GEMM (binary64, OpenMP) on the same step, restricted
    to a sample of output channels (rows are independent), sized for ~target_s."""
    import oracle
    sample = 128
    done_bytes, done_s = 0, 0.0
    packed = {}
    t_start = time.time()
    while True:
        b_round, s_round = 0, 0.0
        for name, B in calls:
            K, N = synth.LLAMA3_8B_SHAPES[name]
            n = min(sample, N)
            key = (name, n)
            if key not in packed:
                packed[key] = oracle.w4_pack(w_host[name][:n], 128, True)
            qw, s, z = packed[key]
            x = xs[(name, B)].cpu().view(__import__("torch").int16).numpy().view(np.uint16)
            t = time.perf_counter()
            oracle.gemm_w4a16(x, "bf16", qw, s, z)
            s_round += time.perf_counter() - t
            b_round += roofline.w4a16_bytes(B, n, K)
        done_bytes += b_round
        done_s += s_round
        if done_s >= target_s or time.time() - t_start > 3 * target_s or sample >= 28672:
            break
        sample = min(28672, int(sample * max(2.0, min(8.0, target_s / max(s_round, 1e-3)))))
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(done_bytes / done_s / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model, "kind": "oracle",
            "sample": f"same 12 W4A16 decode calls restricted to the first <= {sample} output channels "
                      f"of each layer; {done_s:.1f} s of oracle time (binary64 dequantized GEMM)"}


if __name__ == "__main__":
    main()
