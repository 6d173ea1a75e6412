"""Seeded synthetic inputs for the workloads (weights and activations).

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no quantization, slicing or product).  Both the CPU
oracle's callers and the HIP path's callers take their inputs from here.

Workloads (shapes of the models the MatQuant pages evaluate: Gemma-2 9B and
Mistral 7B feed-forward and attention projections; the trained weights and the
evaluation data are not used, Gaussian weights of those shapes stand in):

  tiny_linear    K=512 -> N=256, per-channel, W ~ N(0, 0.02), x ~ N(0, 1), M in {1, 4}
  gemma9b_mlp    up/gate 3584 -> 14336, down 14336 -> 3584, per-channel, M = 1,
                 W ~ N(0, 0.02) with a Bernoulli(1e-3) mask of entries scaled x10
  mistral_small  (N, K) in {(14336, 4096), (4096, 14336)}, group 128, M in {16, 64},
                 x ~ N(0, 1) with 8 seeded input channels scaled x20
  mistral_stack  32 layers x {q, k, v, o, up, gate, down}, per-channel, M = 1
  prefill        M = 2048, K = 4096, N = 14336, group 128

Seeds: numpy's default_rng([workload_id, tag, layer, matrix]) with tags
W = 0, x = 1, outlier mask = 2, heavy-channel pick = 3.  Large weight tensors
made on the GPU use torch's device generator seeded from the same key.
"""

from __future__ import annotations

import numpy as np

WORKLOAD_IDS = {
    "tiny_linear": 1,
    "gemma9b_mlp": 2,
    "mistral_small": 3,
    "mistral_stack": 4,
    "prefill": 5,
}

TAG_W, TAG_X, TAG_OUTLIER, TAG_HEAVY = 0, 1, 2, 3

WEIGHT_STD = 0.02

# (N_out, K_in) of each linear
GEMMA9B_MLP = {"up": (14336, 3584), "gate": (14336, 3584), "down": (3584, 14336)}
MISTRAL_LAYER = {
    "q": (4096, 4096),
    "k": (1024, 4096),
    "v": (1024, 4096),
    "o": (4096, 4096),
    "up": (14336, 4096),
    "gate": (14336, 4096),
    "down": (4096, 14336),
}
MISTRAL_SMALL_SHAPES = ((14336, 4096), (4096, 14336))
PREFILL_SHAPE = (2048, 4096, 14336)  # (M, K, N)


def _key(workload: str, tag: int, layer: int = 0, matrix: int = 0):
    return [WORKLOAD_IDS[workload], tag, layer, matrix]


def rng(workload: str, tag: int, layer: int = 0, matrix: int = 0) -> np.random.Generator:
    return np.random.default_rng(_key(workload, tag, layer, matrix))


def seed64(workload: str, tag: int, layer: int = 0, matrix: int = 0) -> int:
    """A 63-bit integer seed derived from the key (for torch generators)."""
    ss = np.random.SeedSequence(_key(workload, tag, layer, matrix))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


def gaussian_weights(workload: str, n: int, k: int, layer: int = 0, matrix: int = 0,
                     std: float = WEIGHT_STD, outlier_frac: float = 0.0,
                     outlier_scale: float = 10.0) -> np.ndarray:
    """float32 [N, K] ~ N(0, std), with an optional Bernoulli(outlier_frac)
    mask of entries multiplied by outlier_scale."""
    w = rng(workload, TAG_W, layer, matrix).standard_normal((n, k), dtype=np.float32)
    w *= np.float32(std)
    if outlier_frac > 0:
        mask = rng(workload, TAG_OUTLIER, layer, matrix).random((n, k)) < outlier_frac
        w[mask] *= np.float32(outlier_scale)
    return w


def activations_f32(workload: str, m: int, k: int, layer: int = 0, matrix: int = 0,
                    heavy_channels: int = 0, heavy_scale: float = 20.0) -> np.ndarray:
    """float32 [M, K] ~ N(0, 1), with `heavy_channels` seeded input channels
    (the same for every row) multiplied by heavy_scale."""
    x = rng(workload, TAG_X, layer, matrix).standard_normal((m, k), dtype=np.float32)
    if heavy_channels:
        idx = rng(workload, TAG_HEAVY, layer, matrix).choice(k, heavy_channels, replace=False)
        x[:, idx] *= np.float32(heavy_scale)
    return x


def to_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 with torch's conversion (nearest, ties to even)
    and return the bit patterns as uint16."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def activations_bf16(workload: str, m: int, k: int, layer: int = 0, matrix: int = 0,
                     heavy_channels: int = 0, heavy_scale: float = 20.0) -> np.ndarray:
    """bf16 bit patterns uint16 [M, K] of activations_f32()."""
    return to_bf16_bits(activations_f32(workload, m, k, layer, matrix,
                                        heavy_channels, heavy_scale))


def device_gaussian_weights(workload: str, n: int, k: int, device, layer: int = 0,
                            matrix: int = 0, std: float = WEIGHT_STD,
                            outlier_frac: float = 0.0, outlier_scale: float = 10.0):
    """Like gaussian_weights but drawn on `device` with torch's generator
    (a different stream of numbers; same law).  For tensors too large to draw
    on the host in reasonable time."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed64(workload, TAG_W, layer, matrix))
    w = torch.randn((n, k), generator=g, device=device, dtype=torch.float32)
    w.mul_(std)
    if outlier_frac > 0:
        g2 = torch.Generator(device=device)
        g2.manual_seed(seed64(workload, TAG_OUTLIER, layer, matrix))
        mask = torch.rand((n, k), generator=g2, device=device) < outlier_frac
        w[mask] *= outlier_scale
    return w


def mixnmatch_pattern(n_layers: int = 32, edge: int = 8) -> list:
    """Per-layer slice precision of the Mistral stack: the first and last
    `edge` layers at r = 8, the middle at r = 4 with every third middle layer
    (middle index j with j % 3 == 2) at r = 2.  For 32 layers this is
    8 x r8, 4,4,2, 4,4,2, 4,4,2, 4,4,2, 4,4,2, 4, 8 x r8."""
    rs = []
    for layer in range(n_layers):
        if layer < edge or layer >= n_layers - edge:
            rs.append(8)
        else:
            j = layer - edge
            rs.append(2 if j % 3 == 2 else 4)
    return rs
