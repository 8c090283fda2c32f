"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds none of the method's arithmetic: it only draws random
numbers with the distributions of the workloads and casts them to the storage
types (int8 codes and signs, binary16 scales and activations).  Both the CPU
oracle and the HIP library consume the same bytes produced here.

Distributions (workload descriptions of the ternary g128 layer):
  codes   iid, P(-1) = 0.3, P(0) = 0.4, P(+1) = 0.3; with ``binary`` (weights
          of the 1-bit format) iid, P(-1) = P(+1) = 0.5
  scales  |N(0, 0.02)| rounded to binary16, one per 128 weights along K
  signs   Rademacher, one per column of K
  x       N(0, 1) rounded to binary16; with ``outliers`` a Bernoulli(0.01)
          mask of elements is multiplied by 20 before the rounding
Every tensor comes from its own PCG64 stream seeded with
SeedSequence([seed, cfg, layer, linear]), drawn in the order signs, codes,
scales, x.
"""
from __future__ import annotations

import dataclasses

import numpy as np

GROUP = 128


@dataclasses.dataclass
class LinearInputs:
    signs: np.ndarray    # int8 [K], +-1
    codes: np.ndarray    # int8 [N, K], {-1, 0, 1} ({-1, 1} when binary)
    scales: np.ndarray   # float16 [N, K/128]
    x: np.ndarray        # float16 [M, K]


def rng_for(seed: int, cfg: int, layer: int, linear: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg, layer, linear]))


def draw_signs(rng: np.random.Generator, k: int) -> np.ndarray:
    return (rng.integers(0, 2, k) * 2 - 1).astype(np.int8)


def draw_codes(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    u = rng.random((n, k), dtype=np.float32)
    c = (u >= 0.3).astype(np.int8)
    c += (u >= 0.7).astype(np.int8)
    c -= 1
    return c


def draw_binary_codes(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    return (rng.integers(0, 2, (n, k), dtype=np.int8) * 2 - 1).astype(np.int8)


def draw_scales(rng: np.random.Generator, n: int, k: int, group: int = GROUP) -> np.ndarray:
    return np.abs(0.02 * rng.standard_normal((n, k // group))).astype(np.float16)


def draw_x(rng: np.random.Generator, m: int, k: int, outliers: bool = False) -> np.ndarray:
    x = rng.standard_normal((m, k))
    if outliers:
        mask = rng.random((m, k)) < 0.01
        x[mask] *= 20.0
    return x.astype(np.float16)


def linear_inputs(n: int, k: int, m: int, *, seed: int = 0, cfg: int = 1, layer: int = 0,
                  linear: int = 0, outliers: bool = False, group: int = GROUP,
                  binary: bool = False) -> LinearInputs:
    rng = rng_for(seed, cfg, layer, linear)
    signs = draw_signs(rng, k)
    codes = draw_binary_codes(rng, n, k) if binary else draw_codes(rng, n, k)
    scales = draw_scales(rng, n, k, group)
    x = draw_x(rng, m, k, outliers)
    return LinearInputs(signs=signs, codes=codes, scales=scales, x=x)


# Shapes of the workloads (27B-class linear layers; K along the input dim).
# name -> (K, N)
SHAPES = {
    "cfg1": (1024, 1024),
    "gate": (5120, 17408),
    "up": (5120, 17408),
    "down": (17408, 5120),
    "q": (5120, 6144),
    "k": (5120, 1024),
    "v": (5120, 1024),
    "o": (6144, 5120),
}
# linear ids used in the seed so that every projection has its own draw
LINEAR_ID = {"cfg1": 0, "q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6}
LAYER_LINEARS = ("q", "k", "v", "o", "gate", "up", "down")
BATCHED_M = (1, 2, 4, 8, 16)
PREFILL_M = (512, 2048, 4096)
N_LAYERS = 64
