"""Seeded synthetic inputs for the quantized linear layer.

This module only draws random tensors and casts them to the storage dtype of
the workload; it holds none of the quantization or GEMM arithmetic, so both
the HIP path and the CPU oracle can be fed from it.

Workloads (layer shapes stand in for Llama-3-8B and Qwen3-0.6B projections;
no weights or datasets are used):

* weights  W ~ N(0, 0.02) binary32 [N][K]; for the decode sweep, round(0.01*K)
  input channels (columns of W), chosen by a seeded permutation, are scaled x20;
* activations X ~ N(0, 1) binary32, cast round-to-nearest-even to FP16/BF16;
  for the W8A8 workloads 8 seeded input channels (columns of X) are scaled x50.

Draw order for one seed: W, then the weight-outlier permutation, then X, then
the activation-outlier permutation -- so that a W is identical whatever X is
drawn with it.
"""
from __future__ import annotations

import numpy as np
import torch

# (K, N) of the Llama-3-8B decoder projections used by the decode/prefill sweeps
LLAMA3_8B_SHAPES = {
    "qkv": (4096, 6144),
    "o": (4096, 4096),
    "gate_up": (4096, 28672),
    "down": (14336, 4096),
}
# Qwen3-0.6B hidden size (1024 x 1024 projection)
QWEN3_06B_SHAPE = (1024, 1024)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def weights(N: int, K: int, seed: int = 0, std: float = 0.02,
            outlier_frac: float = 0.0, outlier_gain: float = 20.0,
            gen: torch.Generator | None = None) -> np.ndarray:
    """W [N][K] binary32 ~ N(0, std); round(outlier_frac*K) input channels x gain."""
    g = gen if gen is not None else _gen(seed)
    w = torch.randn((N, K), generator=g, dtype=torch.float32) * std
    n_out = int(round(outlier_frac * K))
    if n_out:
        cols = torch.randperm(K, generator=g)[:n_out]
        w[:, cols] *= outlier_gain
    return w.numpy()


def activations(M: int, K: int, dtype: str, seed: int = 0, n_outlier_cols: int = 0,
                outlier_gain: float = 50.0, gen: torch.Generator | None = None) -> np.ndarray:
    """X [M][K] ~ N(0,1) cast RNE to 'f16' / 'bf16' (returned as uint16 bits) or
    kept as 'f32'; n_outlier_cols seeded columns are scaled by outlier_gain first."""
    g = gen if gen is not None else _gen(seed)
    x = torch.randn((M, K), generator=g, dtype=torch.float32)
    if n_outlier_cols:
        cols = torch.randperm(K, generator=g)[:n_outlier_cols]
        x[:, cols] *= outlier_gain
    if dtype == "f32":
        return x.numpy()
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return x.to(tdt).view(torch.int16).numpy().view(np.uint16)


def layer(M: int, N: int, K: int, x_dtype: str, seed: int = 0, w_outlier_frac: float = 0.0,
          x_outlier_cols: int = 0):
    """One seeded (W, X) pair drawn in the fixed order W, W-outliers, X, X-outliers."""
    g = _gen(seed)
    w = weights(N, K, outlier_frac=w_outlier_frac, gen=g)
    x = activations(M, K, x_dtype, n_outlier_cols=x_outlier_cols, gen=g)
    return w, x


def decode_layer(M: int, N: int, K: int, seed: int = 0):
    """W4A16 decode-sweep workload: 1% of input channels x20, BF16 activations."""
    return layer(M, N, K, "bf16", seed, w_outlier_frac=0.01)


def prefill_layer(M: int, N: int, K: int, seed: int = 0):
    """W8A8 prefill workload: plain weights, BF16 activations with 8 columns x50."""
    return layer(M, N, K, "bf16", seed, x_outlier_cols=8)


def qwen_layer(seed: int = 0):
    """W4A16 single linear on the 1024x1024 layer, batch 1, FP16 activations."""
    K, N = QWEN3_06B_SHAPE
    return layer(1, N, K, "f16", seed)
