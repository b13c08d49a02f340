"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random tensors; it holds none of the quantization
arithmetic. Both the CPU oracle and the GPU path receive the very same arrays.

Recipe (the shapes and distributions of the workloads the AWQ pages discuss):

* weights: fp16, i.i.d. N(0, 0.02^2), round-to-nearest-even conversion to fp16;
* activations: fp16, i.i.d. N(0, 1), with round(1% of K) "outlier" input channels
  (chosen without replacement) multiplied by 20, standing in for the few channels
  with much larger activations that make weights salient ("AWQ量化实战" §1.3 and
  "什么是激活感知权重量化（AWQ）" "工作机制": about 1% of weights matter);
* the calibration set and the run-time activations of one layer use the same
  outlier channels (they come from the same model);
* seeds: BASE_SEED + a fixed per-tensor offset.

Calibration text (pile / wikitext) and trained checkpoints are not available; these
tensors stand in for them.
"""

from __future__ import annotations

import numpy as np

BASE_SEED = 20261203
W_STD = 0.02
OUTLIER_FRAC = 0.01
OUTLIER_MULT = 20.0

# Llama-2-7B decoder-layer linears: name -> (N = out features, K = in features)
LLAMA2_7B_LINEARS = {
    "q_proj": (4096, 4096), "k_proj": (4096, 4096), "v_proj": (4096, 4096),
    "o_proj": (4096, 4096), "gate_proj": (11008, 4096), "up_proj": (11008, 4096),
    "down_proj": (4096, 11008),
}
# Linears sharing one input (and therefore one scale vector), concatenated along N.
LLAMA2_7B_SEARCH_GROUPS = {
    "qkv": (12288, 4096), "o": (4096, 4096), "gate_up": (22016, 4096), "down": (4096, 11008),
}
# Llama-2-70B decoder-layer linears (GQA: 64 query heads, 8 kv heads, head dim 128).
LLAMA2_70B_LINEARS = {
    "qkv_proj": (10240, 8192), "o_proj": (8192, 8192), "gate_proj": (28672, 8192),
    "up_proj": (28672, 8192), "down_proj": (8192, 28672),
}
LLAMA2_70B_LAYERS = 80


def n_outliers(K: int) -> int:
    return int(round(OUTLIER_FRAC * K))


def rng(offset: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(BASE_SEED + offset))


def weights(N: int, K: int, offset: int = 0, std: float = W_STD) -> np.ndarray:
    """fp16 [N][K] weights ~ N(0, std^2)."""
    g = rng(offset)
    return (g.standard_normal((N, K), dtype=np.float32) * np.float32(std)).astype(np.float16)


def outlier_channels(K: int, offset: int = 0) -> np.ndarray:
    g = rng(10_000 + offset)
    return np.sort(g.choice(K, size=n_outliers(K), replace=False))


def activations(T: int, K: int, offset: int = 0, channel_offset: int = 0,
                heavy_tail: bool = True) -> np.ndarray:
    """fp16 [T][K] activations ~ N(0, 1), with 1% of the channels scaled by 20."""
    g = rng(1_000 + offset)
    x = g.standard_normal((T, K), dtype=np.float32)
    if heavy_tail:
        x[:, outlier_channels(K, channel_offset)] *= np.float32(OUTLIER_MULT)
    return x.astype(np.float16)


# ---------------------------------------------------------------- device versions
def torch_weights(N: int, K: int, offset: int, device, std: float = W_STD):
    """Same recipe drawn by torch on ``device`` (for sizes too large to draw on the host)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(BASE_SEED + offset)
    w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32)
    return (w * std).to(torch.float16)


def torch_activations(T: int, K: int, offset: int, device, channel_offset: int = 0):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(BASE_SEED + 1_000 + offset)
    x = torch.randn((T, K), generator=g, device=device, dtype=torch.float32)
    ch = torch.from_numpy(outlier_channels(K, channel_offset)).to(device)
    x[:, ch] *= OUTLIER_MULT
    return x.to(torch.float16)


def activations_wide(T: int, K: int, offset: int, log2_lo: float, log2_hi: float,
                     n_zero: int = 0) -> np.ndarray:
    """fp16 [T][K] activations N(0, 1) times a per-channel magnitude 2^u, u uniform in
    [log2_lo, log2_hi] (activation magnitudes spread over many octaves), with n_zero
    channels (chosen without replacement) set to zero: dead channels."""
    g = rng(2_000 + offset)
    x = g.standard_normal((T, K), dtype=np.float32)
    x *= np.exp2(g.uniform(log2_lo, log2_hi, K)).astype(np.float32)[None, :]
    if n_zero:
        x[:, g.choice(K, size=n_zero, replace=False)] = 0.0
    return x.astype(np.float16)
