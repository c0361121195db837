"""Seeded synthetic inputs for the Q4 x Q8 matmul path.

This module only draws random numbers and describes shapes.  It holds none
of the method's arithmetic (no quantisation, no normalisation, no products),
so both the oracle tests and the GPU path can use it without sharing code.

Host draws use numpy's PCG64 seeded by ``SeedSequence([seed, a, b, kind])``
and ``standard_normal(dtype=float32)`` scaled with a single fp32 multiply (and
a single fp32 add for the norm weight).  Large throughput-only weights may be
drawn on the device with a seeded ``torch.Generator`` instead
(``weight_device``); the parity tests always use the host draws.

Shapes follow Llama-family decoder layers: a layer has the seven matrices
Q, K, V, O, gate, up, down; decode feeds B activation columns, prefill T
token rows; the MoE workload routes each of T tokens to top_k of E experts.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

KIND_WEIGHT = 0
KIND_ACT = 1
KIND_NORM = 2
KIND_IDS = 3
KIND_ROUTE_W = 4

WEIGHT_SIGMA = 0.02
NORM_SIGMA = 0.1
RMS_EPS = 1e-5


def rng(seed: int, a: int, b: int, kind: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, a, b, kind])))


def weight(seed: int, layer: int, matrix: int, M: int, K: int, sigma: float = WEIGHT_SIGMA) -> np.ndarray:
    """W ~ N(0, sigma^2), f32 [M][K]."""
    z = rng(seed, layer, matrix, KIND_WEIGHT).standard_normal((M, K), dtype=np.float32)
    return z * np.float32(sigma)


def activation(seed: int, layer: int, slot: int, B: int, K: int) -> np.ndarray:
    """x ~ N(0, 1), f32 [B][K]."""
    return rng(seed, layer, slot, KIND_ACT).standard_normal((B, K), dtype=np.float32)


def norm_weight(seed: int, layer: int, slot: int, K: int, sigma: float = NORM_SIGMA) -> np.ndarray:
    """g ~ N(1, sigma^2), f32 [K]."""
    z = rng(seed, layer, slot, KIND_NORM).standard_normal(K, dtype=np.float32)
    return np.float32(1.0) + z * np.float32(sigma)


def expert_ids(seed: int, T: int, E: int, top_k: int) -> np.ndarray:
    """Per token, the first top_k entries of a seeded permutation of range(E):
    top_k distinct experts, uniform without replacement.  int32 [T][top_k]."""
    g = rng(seed, 0, 0, KIND_IDS)
    return np.stack([g.permutation(E)[:top_k] for _ in range(T)]).astype(np.int32)


def expert_weights(seed: int, T: int, top_k: int) -> np.ndarray:
    """Routing weights of the selected experts: per token, a softmax of
    top_k standard-normal logits (drawn in float32, exponentiated and
    normalised in float64, stored as float32).  f32 [T][top_k]."""
    z = rng(seed, 0, 0, KIND_ROUTE_W).standard_normal((T, top_k), dtype=np.float32).astype(np.float64)
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def weight_device(seed: int, layer: int, matrix: int, M: int, K: int, device, sigma: float = WEIGHT_SIGMA):
    """Device-drawn W ~ N(0, sigma^2), f32 [M][K] (throughput runs only)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed((seed * 1_000_003 + layer * 1009 + matrix * 17 + 7) & 0x7FFF_FFFF_FFFF)
    w = torch.empty((M, K), dtype=torch.float32, device=device)
    w.normal_(0.0, 1.0, generator=gen)
    return w.mul_(sigma)


def activation_device(seed: int, layer: int, slot: int, B: int, K: int, device):
    """Device-drawn x ~ N(0, 1), f32 [B][K] (throughput runs only)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed((seed * 1_000_003 + layer * 1009 + slot * 17 + 3) & 0x7FFF_FFFF_FFFF)
    x = torch.empty((B, K), dtype=torch.float32, device=device)
    return x.normal_(0.0, 1.0, generator=gen)


def norm_weight_device(seed: int, layer: int, slot: int, K: int, device, sigma: float = NORM_SIGMA):
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed((seed * 1_000_003 + layer * 1009 + slot * 17 + 5) & 0x7FFF_FFFF_FFFF)
    g = torch.empty(K, dtype=torch.float32, device=device)
    return g.normal_(0.0, 1.0, generator=gen).mul_(sigma).add_(1.0)


# ---------------------------------------------------------------------------
# Workload shapes
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Matrix:
    name: str
    M: int          # output rows
    K: int          # reduction length
    slot: int       # which activation row of the layer feeds it


# Activation slots of one decoder layer: 0 = attention-norm row (feeds Q, K,
# V), 1 = attention output (feeds O), 2 = FFN-norm row (feeds gate, up),
# 3 = FFN inner activation (feeds down).  Each slot is drawn as its own
# x ~ N(0,1) and goes through RMSNorm * g -> Q8.
def llama_layer(hidden: int, kv: int, ffn: int) -> tuple[Matrix, ...]:
    return (
        Matrix("q", hidden, hidden, 0),
        Matrix("k", kv, hidden, 0),
        Matrix("v", kv, hidden, 0),
        Matrix("o", hidden, hidden, 1),
        Matrix("gate", ffn, hidden, 2),
        Matrix("up", ffn, hidden, 2),
        Matrix("down", hidden, ffn, 3),
    )


LLAMA_3_2_1B = llama_layer(2048, 512, 8192)      # 16 layers
LLAMA_3_8B = llama_layer(4096, 1024, 14336)      # 32 layers


def slot_k(layer: tuple[Matrix, ...]) -> dict[int, int]:
    out: dict[int, int] = {}
    for m in layer:
        out[m.slot] = m.K
    return out


@dataclass(frozen=True)
class MoeShape:
    E: int = 64
    hidden: int = 2048
    ffn: int = 1408
    T: int = 16
    top_k: int = 8


MOE = MoeShape()

# The tiny single product: RMSNorm(x[K=512]) -> Q8; W[256 x 512] -> Q4; y[256].
TINY = Matrix("tiny", 256, 512, 0)


def layer_weight_bytes(layer: tuple[Matrix, ...]) -> int:
    """Q4 bytes (18 per 32 weights) of one layer's matrices."""
    return sum(m.M * m.K * 9 // 16 for m in layer)
