"""Workload for the decode counter comparison: the W4A16 small-M kernel with
its VALU (dot2) inner product and with its MFMA one, on the Llama-3-8B qkv,
gate_up and down layers at B = 1 and 4, each call run four times.  Run it
under rocprofv3 (--kernel-trace for durations, --pmc for counters); it
prints the kernel each call launched.
"""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))


def main():
    import torch
    from bit_gemm_w4_amd import ops, synth
    dev = torch.device("cuda:0")
    for name in ("qkv", "gate_up", "down"):
        K, N = synth.LLAMA3_8B_SHAPES[name]
        p = ops.w4_pack(torch.randn((N, K), device=dev) * 0.02, 128, True)
        for B in (1, 4):
            x = torch.randn((B, K), device=dev).to(torch.bfloat16)
            for algo in (ops.ALGO_GEMV, ops.ALGO_SKINNY):
                for _ in range(4):
                    ops.gemm_w4a16(x, p, algo=algo, ws=False)
                torch.cuda.synchronize()
                print(name, B, algo, ops.last_kernel(), flush=True)


if __name__ == "__main__":
    main()
