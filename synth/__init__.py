"""Seeded synthetic inputs for the W3G128 kernels and their oracle.

This module only draws numbers; it holds none of the format's arithmetic (no
packing, unpacking, dequantization or products).  Both the GPU tests/benchmark
and the oracle-based checks take their inputs from here, so the two sides see
the same values without sharing any of the computation.

Inputs are returned as plain numpy arrays:
  codes  uint8  [N, K]   values 0..7 (code = 4 + q)
  scales uint16 [N, K/128]  bf16 bit patterns
  x      uint16 [M, K]   bf16 bit patterns

Recipes (the workloads are Llama-3.1-70B layer shapes, with weights drawn like
the symmetric 5-level codebook of the GSQ model card):
  codes:  q in {-2,-1,0,1,2} with probabilities p, code = q + 4;
  scales: |N(0, sigma)| + eps drawn in fp32, rounded once to bf16 (nearest-even);
  x:      N(0, 1) drawn in fp32, rounded once to bf16 (nearest-even).
"""
from __future__ import annotations

import numpy as np

UNIFORM5 = (0.2, 0.2, 0.2, 0.2, 0.2)
PEAKED5 = (0.1, 0.2, 0.4, 0.2, 0.1)

# name -> (N = out_features, K = in_features, weight seed) for one decoder layer
LAYER_70B = {
    "q_proj": (8192, 8192, 4),
    "k_proj": (1024, 8192, 5),
    "v_proj": (1024, 8192, 6),
    "o_proj": (8192, 8192, 7),
    "gate_proj": (28672, 8192, 1),
    "up_proj": (28672, 8192, 2),
    "down_proj": (8192, 28672, 3),
}

_ROW_CHUNK = 2048


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even) and return the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7F800000) == 0x7F800000
    nan &= (u & 0x007FFFFF) != 0
    r = (u + (np.uint32(0x7FFF) + ((u >> 16) & 1))) >> 16
    r = np.where(nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _codes_from(rng: np.random.Generator, n: int, k: int, p) -> np.ndarray:
    cum = np.cumsum(np.asarray(p, dtype=np.float64))
    cum = (cum / cum[-1]).astype(np.float32)
    out = np.empty((n, k), dtype=np.uint8)
    for r0 in range(0, n, _ROW_CHUNK):
        r1 = min(n, r0 + _ROW_CHUNK)
        u = rng.random((r1 - r0, k), dtype=np.float32)
        q = np.zeros(u.shape, dtype=np.uint8)
        for t in cum[:-1]:
            q += u >= t
        out[r0:r1] = q + np.uint8(2)  # q index 0..4 -> code 2..6
    return out


def codes(seed: int, n: int, k: int, p=PEAKED5) -> np.ndarray:
    """Codes 4 + q with q in {-2..2} drawn with probabilities p."""
    return _codes_from(np.random.default_rng(seed), n, k, p)


def codes_all8(seed: int, n: int, k: int) -> np.ndarray:
    """Codes uniform over all eight 3-bit values (wider than the 5-level grid)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 8, size=(n, k), dtype=np.uint8)


def _scales_from(rng, n: int, g: int, sigma: float, eps: float) -> np.ndarray:
    s = np.abs(rng.standard_normal((n, g), dtype=np.float32)) * np.float32(sigma)
    s = s + np.float32(eps)
    return f32_to_bf16_bits(s)


def scales(seed: int, n: int, g: int, sigma: float = 0.01, eps: float = 1e-4) -> np.ndarray:
    return _scales_from(np.random.default_rng(seed), n, g, sigma, eps)


def _x_from(rng, m: int, k: int) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))


def activations(seed: int, m: int, k: int) -> np.ndarray:
    return _x_from(np.random.default_rng(seed), m, k)


def tiny_case():
    """W [256, 1024], uniform q in {-2..2}, scales |N(0,0.02)|+1e-3, x [1,1024].

    One generator, seed 0, drawing codes, then scales, then x.
    """
    rng = np.random.default_rng(0)
    c = _codes_from(rng, 256, 1024, UNIFORM5)
    s = _scales_from(rng, 256, 1024 // 128, 0.02, 1e-3)
    x = _x_from(rng, 1, 1024)
    return c, s, x


def layer_weights(name: str):
    """(codes, scales) of one 70B-layer projection; the same tensor every call."""
    n, k, seed = LAYER_70B[name]
    return codes(seed, n, k, PEAKED5), scales(1000 + seed, n, k // 128, 0.01, 1e-4)


def layer_x(m: int, k: int) -> np.ndarray:
    """Activations for an M-token batch with K inputs (seed 100 + M, +10000 at K=28672)."""
    seed = 100 + m + (10000 if k == 28672 else 0)
    return activations(seed, m, k)
