"""Seeded random draws of weights and activations.

Every draw takes a seed tuple and builds its own ``numpy.random.Generator``
from ``SeedSequence(seed)``, so a case is reproducible from its name alone and
independent of call order.

Distributions follow the workloads' recipes:

- ``normal``: N(0, sigma^2), fp32 (the plain Llama-shaped weight model).
- ``normal_outliers``: N(0, sigma^2) where each weight independently, with
  probability ``p``, is replaced by +-``mult``*sigma with a random sign
  (heavy outliers that a per-group absmax must absorb).
- ``student_t``: ``scale`` * t(nu) (heavy tails, for the 3-bit Lloyd-Max
  table).
- ``laplace``: Laplace(0, b) (many small weights plus rare large ones, the
  case logarithmic tables are designed for).
- activations: N(0, 1) rounded to fp16.
"""

from __future__ import annotations

import numpy as np

ROW_CHUNK = 2048  # rows drawn per generator call for large matrices


def _rng(seed) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(list(seed)))


def weights(kind: str, N: int, K: int, seed, **kw) -> np.ndarray:
    """fp32 weight matrix [N, K] (out x in) of distribution ``kind``."""
    rng = _rng(seed)
    out = np.empty((N, K), dtype=np.float32)
    for n0 in range(0, N, ROW_CHUNK):
        n1 = min(N, n0 + ROW_CHUNK)
        shape = (n1 - n0, K)
        if kind == "normal":
            blk = rng.standard_normal(shape, dtype=np.float32) * np.float32(kw.get("sigma", 0.02))
        elif kind == "normal_outliers":
            sigma = np.float32(kw.get("sigma", 0.02))
            blk = rng.standard_normal(shape, dtype=np.float32) * sigma
            hit = rng.random(shape, dtype=np.float32) < kw.get("p", 1e-3)
            sign = np.where(rng.random(shape, dtype=np.float32) < 0.5, -1.0, 1.0).astype(np.float32)
            blk = np.where(hit, sign * np.float32(kw.get("mult", 10.0)) * sigma, blk)
        elif kind == "student_t":
            blk = (rng.standard_t(kw.get("nu", 4.0), size=shape) * kw.get("scale", 0.02)).astype(np.float32)
        elif kind == "laplace":
            blk = rng.laplace(0.0, kw.get("b", 0.015), size=shape).astype(np.float32)
        else:
            raise ValueError(f"unknown weight distribution {kind!r}")
        out[n0:n1] = blk
    return out


def activations(M: int, K: int, seed) -> np.ndarray:
    """fp16 activations x [M, K], N(0, 1) rounded to nearest-even fp16."""
    rng = _rng(seed)
    return rng.standard_normal((M, K), dtype=np.float32).astype(np.float16)


def integers(shape, high: int, seed) -> np.ndarray:
    """Uniform integers in [0, high) as uint8 (raw codes for layout tests)."""
    rng = _rng(seed)
    return rng.integers(0, high, size=shape, dtype=np.uint8)
