"""Scales and round-to-nearest (RTN) codes for a given lookup table.

Group-wise granularity with groups of ``group`` consecutive weights along K
(128 in the workloads; page 2 names group-128 quantization and RTN), or one
scale for the whole tensor when ``group == 0`` (tensor-wise granularity,
page 1, LogbQuant abstract).

Scale rules (the value is rounded once to fp16, nearest even):

- ``absmax``: ``s = absmax(group) / max|T|`` so the largest-magnitude weight
  maps onto the outermost table entry (NormalFloat, Lloyd-Max and log tables).
- ``int``: for the uniform table ``T[i] = i - z`` with levels ``[-z, L-1-z]``,
  ``s = max(max(group) / (L-1-z), -min(group) / z)``, the smallest scale
  whose level range covers the group.
- A scale that comes out as 0 (an all-zero group) is replaced by 1.

Codes: ``r = w / s`` in fp64 (w and s taken as their fp32 / fp16 values) and
``c = argmin_i |r - T[i]|`` over the fp16 table entries, compared exactly;
an exact tie goes to the lower code index.
"""

from __future__ import annotations

import numpy as np

ROW_CHUNK = 1024


def _group_view(w: np.ndarray, group: int) -> np.ndarray:
    N, K = w.shape
    if group == 0:
        return w.reshape(1, 1, N * K)
    if K % group:
        raise ValueError(f"K={K} is not a multiple of group={group}")
    return w.reshape(N, K // group, group)


def scales(w: np.ndarray, lut: np.ndarray, group: int, rule: str) -> np.ndarray:
    """fp16 scales: [N, K/group] row-major, or [1] when group == 0."""
    T = lut.astype(np.float64)
    g = _group_view(w, group)
    if rule == "absmax":
        s = np.abs(g).max(axis=-1).astype(np.float64) / np.abs(T).max()
    elif rule == "int":
        L = T.size
        z = -T.min()  # T = i - z, so the smallest level is -z
        top = L - 1 - z
        mx = g.max(axis=-1).astype(np.float64)
        mn = g.min(axis=-1).astype(np.float64)
        s = np.maximum(mx / top, -mn / z)
    else:
        raise ValueError(f"unknown scale rule {rule!r}")
    s16 = s.astype(np.float16)
    s16[s16 == 0] = np.float16(1.0)
    if not np.all(np.isfinite(s16)) or np.any(s16 < 0):
        raise ValueError("scale out of fp16 range")
    return s16.reshape(1) if group == 0 else s16.reshape(w.shape[0], -1)


def nearest_codes(r: np.ndarray, lut: np.ndarray) -> np.ndarray:
    """Index of the table entry nearest to each r (exact compare, ties -> lower index)."""
    T = lut.astype(np.float64)
    order = np.argsort(T, kind="stable")
    Ts = T[order]
    if np.any(np.diff(Ts) <= 0):
        raise ValueError("table entries must be distinct")
    mids = 0.5 * (Ts[:-1] + Ts[1:])  # exact: fp16 values sum exactly in fp64
    j = np.searchsorted(mids, r, side="left")  # number of midpoints strictly below r
    tie = np.zeros(r.shape, dtype=bool)
    inner = j < mids.size
    tie[inner] = r[inner] == mids[j[inner]]
    pick = order[j]
    if np.any(tie):
        jt = j[tie]
        pick[tie] = np.minimum(order[jt], order[jt + 1])
    return pick.astype(np.uint8)


def codes(w: np.ndarray, lut: np.ndarray, s: np.ndarray, group: int) -> np.ndarray:
    """uint8 codes [N, K] (low ``log2(len(lut))`` bits used)."""
    N, K = w.shape
    out = np.empty((N, K), dtype=np.uint8)
    s64 = s.astype(np.float64)
    for n0 in range(0, N, ROW_CHUNK):
        n1 = min(N, n0 + ROW_CHUNK)
        blk = w[n0:n1].astype(np.float64)
        if group == 0:
            r = blk / s64[0]
        else:
            r = (blk.reshape(n1 - n0, K // group, group) / s64[n0:n1, :, None]).reshape(n1 - n0, K)
        out[n0:n1] = nearest_codes(r, lut)
    return out


def quantize(w: np.ndarray, lut: np.ndarray, group: int, rule: str):
    """(codes u8 [N,K], scales fp16) for weights w under table ``lut``."""
    s = scales(w, lut, group, rule)
    return codes(w, lut, s, group), s
