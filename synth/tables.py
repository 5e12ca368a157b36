"""Lookup tables (2^b fp16 entries) that quantized weights index.

Four table families appear in the source pages:

- ``int_uniform``: asymmetric linear / uniform INT levels ``T[i] = i - z``
  with integer zero point ``z = 2^(b-1)`` (the tensor-wise asymmetric linear
  baseline that LogbQuant compares against; page 1, LogbQuant abstract). A
  uniform table turns LUT dequantization into plain INT dequantization.
- ``normal_float``: NormalFloat-style levels, the quantiles of N(0, 1) at the
  midpoints ``(i + 1/2) / 2^b`` scaled so the outermost level is 1 (page 2,
  FLUTE abstract, names LUT-based NormalFloat; the midpoint-quantile
  construction is the plainest reading of "quantiles of N(0,1) scaled to
  [-1,1]").
- ``lloyd_max``: the 2^b-level minimum-MSE quantizer of N(0, 1), found by
  the Lloyd-Max alternation (page 3, the TurboQuant/EDEN note, names the
  Lloyd-Max algorithm): thresholds are midpoints of neighbouring levels and
  each level is the conditional mean of its cell.
- ``log``: logarithmic levels with an adjustable base (page 1, LogbQuant
  abstract): 4-bit code = sign bit (MSB) + 3-bit exponent k, value
  ``(-1)^sign * base^(-k)``; no zero code.

All tables are computed in fp64 and rounded once to fp16 (round to nearest
even). The GPU receives the fp16 values as data.
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import ndtri
from scipy.stats import norm


def int_uniform(bits: int, zero_point: int | None = None) -> np.ndarray:
    z = (1 << (bits - 1)) if zero_point is None else zero_point
    return (np.arange(1 << bits, dtype=np.float64) - z).astype(np.float16)


def normal_float(bits: int) -> np.ndarray:
    L = 1 << bits
    p = (np.arange(L, dtype=np.float64) + 0.5) / L
    q = ndtri(p)
    return (q / ndtri((L - 0.5) / L)).astype(np.float16)


def lloyd_max_fp64(bits: int, tol: float = 1e-14, max_iter: int = 100000) -> np.ndarray:
    """Lloyd-Max levels for N(0, 1) in fp64, started from midpoint quantiles."""
    L = 1 << bits
    T = ndtri((np.arange(L, dtype=np.float64) + 0.5) / L)
    for _ in range(max_iter):
        t = 0.5 * (T[:-1] + T[1:])  # cell boundaries: midpoints of levels
        lo = np.concatenate(([-np.inf], t))
        hi = np.concatenate((t, [np.inf]))
        # centroid of N(0,1) on [lo, hi): (phi(lo) - phi(hi)) / (Phi(hi) - Phi(lo))
        Tn = (norm.pdf(lo) - norm.pdf(hi)) / (norm.cdf(hi) - norm.cdf(lo))
        delta = float(np.max(np.abs(Tn - T)))
        T = Tn
        if delta < tol:
            break
    return T


def lloyd_max(bits: int) -> np.ndarray:
    return lloyd_max_fp64(bits).astype(np.float16)


def log_table(bits: int = 4, base: float = math.sqrt(2.0)) -> np.ndarray:
    """Code c = (sign << (bits-1)) | k; value (-1)^sign * base^(-k)."""
    half = 1 << (bits - 1)
    mags = np.array([base ** (-k) for k in range(half)], dtype=np.float64)
    return np.concatenate((mags, -mags)).astype(np.float16)


def make(kind: str, bits: int, **kw) -> np.ndarray:
    if kind == "int":
        return int_uniform(bits, kw.get("zero_point"))
    if kind == "nf":
        return normal_float(bits)
    if kind == "lloyd_max":
        return lloyd_max(bits)
    if kind == "log":
        return log_table(bits, kw.get("base", math.sqrt(2.0)))
    raise ValueError(f"unknown table kind {kind!r}")
