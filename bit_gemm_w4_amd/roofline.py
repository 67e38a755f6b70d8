"""Roofline arithmetic for the quantized linear layer.

"Quantization throughput by method" (hrletsgo.me), arithmetic-intensity
section: AI = FLOPs / bytes; a kernel below the ridge point (peak FLOP/s over
peak bytes/s) is bandwidth-bound; for a decode linear at batch B,
AI ~= 2B / bytes_per_weight, so the batch where INT4 weights (0.5 B/weight)
turn compute-bound is ridge * 0.5 / 2 (about 74 for the page's H100 ridge of
~295).  "Low-precision LLM inference" §5: effective bits per weight
b + m/G (4 + 16/128 = 4.125 with FP16 scales per 128).

MI355X peaks used for the fractions (AMD's published dense figures).
"""
from __future__ import annotations

HBM_GBPS = 8000.0                 # HBM3E, GB/s
PEAK_TFLOPS = {                    # dense matrix-core peaks
    "bf16": 2500.0, "f16": 2500.0, "fp8": 5000.0, "i8": 5000.0,
    "fp6": 10100.0, "fp4": 10100.0, "f32": 157.3, "f64": 78.6,
}


def ai_decode(batch: int, bytes_per_weight: float) -> float:
    """FLOP per weight byte of a decode linear (weights dominate the traffic)."""
    return 2.0 * batch / bytes_per_weight


def ridge(peak_tflops: float, hbm_gbps: float) -> float:
    return peak_tflops * 1e12 / (hbm_gbps * 1e9)


def critical_batch(ridge_flop_per_byte: float, bytes_per_weight: float) -> float:
    """Batch at which AI(decode, B) reaches the ridge point."""
    return ridge_flop_per_byte * bytes_per_weight / 2.0


def effective_bits(bits: int, meta_bits: int, group: int) -> float:
    return bits + meta_bits / group


def w4a16_bytes(M: int, N: int, K: int, group: int = 128, asym: bool = True, act_bytes: int = 2) -> int:
    """Algorithmic HBM bytes of one W4A16 call: packed codes, FP16 scales,
    4-bit zero-points, activations in, outputs out."""
    w = N * K // 2 + N * (K // group) * 2 + (N * (K // group) // 2 if asym else 0)
    return w + M * K * act_bytes + M * N * act_bytes


def gemm_flops(M: int, N: int, K: int) -> float:
    return 2.0 * M * N * K


def act_quant_bytes(R: int, C: int, in_bytes: int = 2, n_scales: int | None = None) -> int:
    """Read the tensor once, write one byte per element plus FP32 scales."""
    return R * C * in_bytes + R * C + 4 * (R if n_scales is None else n_scales)


def w8a8_bytes(M: int, N: int, K: int, out_bytes: int = 2, w_scales: int | None = None) -> int:
    """Algorithmic HBM bytes of one W8A8 GEMM call: 8-bit weights and
    activations, FP32 scales (per channel and per token unless given), output."""
    return N * K + M * K + 4 * (N if w_scales is None else w_scales) + 4 * M + M * N * out_bytes
