"""The oracle for the quantizer: round-to-nearest onto a lookup table.

TEST INFRASTRUCTURE (see the package docstring): only the tests, the smoke
check and the benchmark's CPU-baseline leg use it.

What it computes (page 2, the PTQ-damage abstract: round-to-nearest
quantization at group-128 granularity; page 2, FLUTE abstract: the grid is an
arbitrary lookup table, uniform or not; page 1, LogbQuant abstract:
tensor-wise granularity and logarithmic tables whose base is adjustable):

- one fp16 scale per group of ``group`` consecutive weights along K, or one
  per tensor (``group == 0``), computed in fp64 and rounded once to fp16
  (nearest even), a zero scale replaced by 1 and a scale above the largest
  finite fp16 clamped to it;
    * rule ``absmax``: ``s = max|w| / max|T|`` (the largest-magnitude weight
      lands on the outermost table entry);
    * rule ``range``:  ``s = max(max(w) / max(T), min(w) / min(T))``, for a
      table with ``min(T) < 0 < max(T)``; for the uniform table
      ``T[i] = i - z`` this is the smallest scale whose level range covers the
      group, i.e. asymmetric INT round-to-nearest;
- codes ``c = argmin_i |w / s - T[i]|`` with ``w / s`` in fp64 (weights taken
  at their fp32 value) and the distance compared exactly; an exact tie goes
  to the lower code index;
- the weight error ``sum (w - s * T[c])^2`` in fp64, the objective of the
  table search;
- the logarithmic table ``T[sign, k] = (-1)^sign * base^(-k)`` (sign = the top
  code bit, k = the remaining bits) and the base search: the candidate base
  with the smallest weight error;
- table tuning on the weight error (page 2, FLUTE abstract: NormalFloat
  tables; page 3, TurboQuant/EDEN note: the Lloyd-Max algorithm): with the
  scales fixed from the initial table, alternate round-to-nearest codes and
  the least-squares entry T[i] = sum w s / sum s^2 over the weights coded i.

Parity status: every function here is pinned by tests/test_oracle_quantize.py
(closed forms, brute force with exact rationals, invariants).
"""

from __future__ import annotations

import numpy as np

ROW_CHUNK = 512
FP16_MAX = 65504.0


def _groups(w: np.ndarray, group: int) -> np.ndarray:
    """View of w as [n_groups, group_size] (one group per tensor if group == 0)."""
    N, K = w.shape
    if group == 0:
        return w.reshape(1, N * K)
    if group <= 0 or K % group:
        raise ValueError(f"group {group} does not divide K = {K}")
    return w.reshape(N * (K // group), group)


def scales(w: np.ndarray, lut: np.ndarray, group: int, rule: str) -> np.ndarray:
    """fp16 scales, [N, K/group] row-major or [1] for group == 0."""
    T = lut.astype(np.float64)
    g = _groups(np.asarray(w, np.float32), group).astype(np.float64)
    if rule == "absmax":
        s = np.abs(g).max(axis=1) / np.abs(T).max()
    elif rule == "range":
        if not (T.min() < 0 < T.max()):
            raise ValueError("rule 'range' needs a table with negative and positive entries")
        s = np.maximum(g.max(axis=1) / T.max(), g.min(axis=1) / T.min())
    else:
        raise ValueError(f"unknown rule {rule!r}")
    s = np.minimum(s, FP16_MAX)          # clamp before rounding: stays finite
    s16 = s.astype(np.float16)           # fp64 -> fp16, round to nearest even
    s16[s16 == 0] = np.float16(1.0)
    return s16.reshape(1) if group == 0 else s16.reshape(w.shape[0], -1)


def nearest(r: np.ndarray, lut: np.ndarray) -> np.ndarray:
    """Index of the table entry nearest to each r (fp64), ties to the lower index.

    Entry a is nearer than entry b (T[a] < T[b]) exactly when r is below
    their midpoint, which is exact in fp64 for fp16 entries; walking the
    sorted table, the answer for r is the first entry whose upper midpoint
    is not below r, and on equality the lower of the two indices.
    """
    T = lut.astype(np.float64)
    if np.unique(T).size != T.size:
        raise ValueError("table entries must be distinct")
    order = np.argsort(T, kind="stable")
    Ts = T[order]
    mids = (Ts[:-1] + Ts[1:]) / 2
    pos = (r[..., None] > mids).sum(axis=-1)          # midpoints strictly below r
    code = order[pos]
    at_mid = np.zeros(r.shape, bool)
    inner = pos < mids.size
    at_mid[inner] = r[inner] == mids[pos[inner]]
    if at_mid.any():
        p = pos[at_mid]
        code[at_mid] = np.minimum(order[p], order[p + 1])
    return code.astype(np.uint8)


def _ratio(w: np.ndarray, s16: np.ndarray, group: int) -> np.ndarray:
    """w / s in fp64, w at its fp32 value and s at its fp16 value."""
    N, K = w.shape
    w64 = np.asarray(w, np.float32).astype(np.float64)
    s64 = s16.astype(np.float64)
    if group == 0:
        return w64 / s64[0]
    return (w64.reshape(N, K // group, group) / s64.reshape(N, K // group, 1)).reshape(N, K)


def codes(w: np.ndarray, lut: np.ndarray, s16: np.ndarray, group: int) -> np.ndarray:
    out = np.empty(w.shape, np.uint8)
    for n0 in range(0, w.shape[0], ROW_CHUNK):
        n1 = min(w.shape[0], n0 + ROW_CHUNK)
        s_blk = s16 if group == 0 else s16[n0:n1]
        out[n0:n1] = nearest(_ratio(w[n0:n1], s_blk, group), lut)
    return out


def quantize(w: np.ndarray, lut: np.ndarray, group: int, rule: str):
    """(codes u8 [N, K], scales fp16): round-to-nearest onto the table."""
    s16 = scales(w, lut, group, rule)
    return codes(w, lut, s16, group), s16


def sq_error(w: np.ndarray, lut: np.ndarray, c: np.ndarray, s16: np.ndarray, group: int) -> float:
    """sum (w - s * T[c])^2 in fp64 (w at fp32, s and T at fp16)."""
    N, K = w.shape
    T = lut.astype(np.float64)
    total = 0.0
    for n0 in range(0, N, ROW_CHUNK):
        n1 = min(N, n0 + ROW_CHUNK)
        w64 = np.asarray(w[n0:n1], np.float32).astype(np.float64)
        v = T[c[n0:n1]]
        if group == 0:
            v = v * s16.astype(np.float64)[0]
        else:
            v = (v.reshape(n1 - n0, K // group, group)
                 * s16[n0:n1].astype(np.float64)[:, :, None]).reshape(n1 - n0, K)
        total += float(np.sum((w64 - v) ** 2))
    return total


def log_table(bits: int, base: float) -> np.ndarray:
    """fp16 table: code = sign bit (top) | k (low bits), value (-1)^sign * base^-k."""
    half = 1 << (bits - 1)
    k = np.arange(1 << bits) % half
    sign = np.where(np.arange(1 << bits) >= half, -1.0, 1.0)
    return (sign * np.power(float(base), -k.astype(np.float64))).astype(np.float16)


def log_base_search(w: np.ndarray, bits: int, group: int, bases) -> tuple[int, list[float]]:
    """Index of the base whose log table gives the smallest weight error
    (absmax scales), and the error of every candidate."""
    errs = []
    for b in bases:
        T = log_table(bits, b)
        c, s16 = quantize(w, T, group, "absmax")
        errs.append(sq_error(w, T, c, s16, group))
    return int(np.argmin(errs)), errs


def tune_table(w: np.ndarray, lut: np.ndarray, group: int, rule: str, iters: int):
    """Lloyd iterations on the weight error with fixed scales.

    The scales come from ``lut`` under ``rule`` and stay fixed. Each
    iteration codes the weights by round-to-nearest and replaces every used
    entry by the fp16 (nearest even) value of sum(w * s) / sum(s^2) over the
    weights holding that code, both sums in fp64 (exact products); an unused
    entry keeps its value. An update that would repeat an fp16 value stops
    the iterations. Returns (table, scales, errors): errors[k] is the weight
    error of the k-th table (errors[0] that of ``lut``), one more than the
    updates made.
    """
    s16 = scales(w, lut, group, rule)
    T = np.asarray(lut, np.float16).copy()
    N, K = w.shape
    w64 = np.asarray(w, np.float32).astype(np.float64)
    sfull = (np.full((N, K), s16.astype(np.float64)[0]) if group == 0
             else np.repeat(s16.astype(np.float64), group, axis=1))
    errors = []
    for k in range(iters + 1):
        c = codes(w, T, s16, group)
        errors.append(sq_error(w, T, c, s16, group))
        if k == iters:
            break
        num = np.bincount(c.ravel(), weights=(w64 * sfull).ravel(), minlength=T.size)
        den = np.bincount(c.ravel(), weights=(sfull * sfull).ravel(), minlength=T.size)
        T_new = T.copy()
        used = den > 0
        T_new[used] = (num[used] / den[used]).astype(np.float16)
        if np.unique(T_new.astype(np.float64)).size != T_new.size:
            break
        T = T_new
    return T, s16, errors
