"""The oracle's arithmetic. See the package docstring for scope and status.

Readings taken where the pages leave a step open:

- codes are b-bit integers, b in {2, 3, 4} (page 2, FLUTE abstract: packed
  codes including the non-evenly-divisible 3 bits);
- the table has 2^b fp16 entries and the scales are fp16, one per ``group``
  consecutive weights along K, or one per tensor (``group == 0``; page 1,
  LogbQuant abstract, tensor-wise granularity);
- dequantization is one fp32 multiply (round to nearest even) of the table
  entry by its scale; the product is accumulated in fp64.
"""

from __future__ import annotations

import numpy as np

ROW_CHUNK = 2048


# -- canonical packing (the oracle's own format; page 2, FLUTE abstract:
#    weights are stored as packed b-bit codes) --------------------------------

def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Row-wise LSB-first bit stream: code k of a row occupies bits [k*b, k*b+b).

    Returns uint8 [N, ceil(K*b/8)]. Codes must already be < 2^bits.
    Pinned: hand-derived byte fixture + exhaustive round trip.
    """
    N, K = codes.shape
    if np.any(codes >> bits):
        raise ValueError("code out of range")
    # bit j of code k lands at stream bit k*bits + j
    bitmat = ((codes[:, :, None] >> np.arange(bits, dtype=np.uint8)) & 1).astype(np.uint8)
    stream = bitmat.reshape(N, K * bits)
    nbytes = (K * bits + 7) // 8
    pad = nbytes * 8 - K * bits
    if pad:
        stream = np.concatenate([stream, np.zeros((N, pad), np.uint8)], axis=1)
    return np.packbits(stream.reshape(N, nbytes, 8), axis=2, bitorder="little").reshape(N, nbytes)


def unpack_codes(packed: np.ndarray, N: int, K: int, bits: int) -> np.ndarray:
    """Inverse of ``pack_codes``: uint8 codes [N, K]."""
    stream = np.unpackbits(packed.reshape(N, -1, 1), axis=2, bitorder="little").reshape(N, -1)
    stream = stream[:, : K * bits].reshape(N, K, bits).astype(np.uint8)
    return (stream << np.arange(bits, dtype=np.uint8)).sum(axis=2, dtype=np.uint8)


# -- dequantization (page 2, FLUTE abstract: LUT-quantized weights; scale per
#    group of 128 along K; page 1: one scale per tensor) ----------------------

def dequant(codes: np.ndarray, lut: np.ndarray, scales: np.ndarray, group: int,
            zeros: np.ndarray | None = None, types: np.ndarray | None = None) -> np.ndarray:
    """W_hat = fp32(T[c]) * fp32(s[n, k // group]), one RNE fp32 multiply. [N, K] fp32.

    With per-group zero points ``zeros`` (fp16, shaped like the grouped
    scales; page 1, LogbQuant abstract: asymmetric linear quantization;
    page 2, BitMoD abstract: per-group quantization parameters):
    W_hat = s * (T[c] - z[n, k // group]) in fp64, which is exact for fp16
    operands. [N, K] fp64.

    With per-group data types ``types`` (uint8, shaped like the grouped
    scales; page 2, BitMoD abstract: a data type chosen per group), ``lut``
    holds one table per type, [n_types, 2^b], and group g of row n reads
    table types[n, g]: W_hat = s * (T[types[n, g]][c] - z) (z = 0 without
    zero points), in fp64. [N, K] fp64.

    Pinned: the uniform table reproduces INT RTN dequantization bit-exactly;
    one-hot products decode single weights; zero points against exact
    rationals, a shift invariance and integer asymmetric RTN; data types
    against exact rationals and a relabelling invariance.
    """
    N, K = codes.shape
    if types is not None:
        if group == 0:
            raise ValueError("data types need grouped scales")
        if K % group:
            raise ValueError("K must be a multiple of group")
        g = K // group
        tables = np.asarray(lut).astype(np.float64).reshape(-1, np.asarray(lut).shape[-1])
        ty = np.repeat(np.asarray(types).astype(np.int64).reshape(N, g), group, axis=1)
        t = tables[ty, codes].reshape(N, g, group)
        z = 0.0 if zeros is None else zeros.astype(np.float64).reshape(N, g, 1)
        sc = scales.astype(np.float64).reshape(N, g, 1)
        return (sc * (t - z)).reshape(N, K)
    if zeros is not None:
        if group == 0:
            raise ValueError("zero points need grouped scales")
        if K % group:
            raise ValueError("K must be a multiple of group")
        g = K // group
        t = lut.astype(np.float64)[codes].reshape(N, g, group)
        z = zeros.astype(np.float64).reshape(N, g, 1)
        sc = scales.astype(np.float64).reshape(N, g, 1)
        return (sc * (t - z)).reshape(N, K)
    t = lut.astype(np.float32)[codes]
    if group == 0:
        return t * np.float32(scales.reshape(-1)[0])
    if K % group:
        raise ValueError("K must be a multiple of group")
    s = scales.astype(np.float32).reshape(N, K // group)
    return (t.reshape(N, K // group, group) * s[:, :, None]).reshape(N, K)


# -- binary-coding quantization (page 4, AlphaTuning abstract: weights
#    factorized into binary parameters and separate scaling factors) -------

def dequant_bcq(codes: np.ndarray, alphas: np.ndarray, group: int) -> np.ndarray:
    """W_hat[n, k] = sum_i alphas[i, n, g] * (2 * bit_i(c[n, k]) - 1), g = k // group, in fp64.

    ``codes`` hold the q binary planes as the bits of a q-bit code (plane i
    in bit i); ``alphas`` are fp16 [q, N, K / group]. Every weight is a sum of
    q signed fp16 values, exact in fp64. [N, K] fp64.

    Pinned: exact rationals; q = 1 is a signed binary matrix; power-of-two
    plane factors (alpha_i = a 2^i) give the uniform table 2c - (2^q - 1)
    with scale a through ``dequant``; the same weights from the 2^q-entry
    table of each group.
    """
    N, K = codes.shape
    q = alphas.shape[0]
    if group <= 0 or K % group:
        raise ValueError("binary coding needs a group that divides K")
    g = K // group
    a = alphas.astype(np.float64).reshape(q, N, g, 1)
    c = codes.astype(np.int64).reshape(N, g, group)
    w = np.zeros((N, g, group))
    for i in range(q):
        w += a[i] * (2.0 * ((c >> i) & 1) - 1.0)
    return w.reshape(N, K)


def reference_bcq(x: np.ndarray, codes: np.ndarray, alphas: np.ndarray, group: int,
                  rows=None):
    """(y_ref, B) as ``reference``, for binary-coded weights (optionally only
    output columns ``rows``)."""
    if rows is not None:
        rows = np.asarray(rows)
        codes, alphas = codes[rows], alphas[:, rows]
    x64 = x.astype(np.float64)
    ax = np.abs(x64)
    N = codes.shape[0]
    y = np.empty((x.shape[0], N))
    B = np.empty((x.shape[0], N))
    for n0 in range(0, N, ROW_CHUNK):
        n1 = min(N, n0 + ROW_CHUNK)
        w = dequant_bcq(codes[n0:n1], alphas[:, n0:n1], group)
        y[:, n0:n1] = x64 @ w.T
        B[:, n0:n1] = ax @ np.abs(w).T
    return y, B


# -- the product (fp64 accumulation) ------------------------------------------

def _rows(codes, lut, scales, group, rows, zeros=None, types=None):
    if group == 0:
        return dequant(codes[rows], lut, scales, 0)
    return dequant(codes[rows], lut, scales[rows], group,
                   None if zeros is None else zeros[rows],
                   None if types is None else types[rows])


def reference(x: np.ndarray, codes: np.ndarray, lut: np.ndarray, scales: np.ndarray,
              group: int, zeros: np.ndarray | None = None, types: np.ndarray | None = None):
    """(y_ref, B): y_ref = fp64(x) @ fp64(W_hat).T and B = |x| @ |W_hat|.T, both [M, N] fp64.

    Chunked over N to bound memory. Pinned: exact rational brute force on
    tiny shapes, linearity in the scale, one-hot x.
    """
    N, K = codes.shape
    x64 = x.astype(np.float64)
    ax = np.abs(x64)
    M = x.shape[0]
    y = np.empty((M, N), np.float64)
    B = np.empty((M, N), np.float64)
    for n0 in range(0, N, ROW_CHUNK):
        n1 = min(N, n0 + ROW_CHUNK)
        w = _rows(codes, lut, scales, group, slice(n0, n1), zeros, types).astype(np.float64)
        y[:, n0:n1] = x64 @ w.T
        B[:, n0:n1] = ax @ np.abs(w).T
    return y, B


def reference_rows(x, codes, lut, scales, group, rows, zeros=None, types=None):
    """``reference`` restricted to output columns ``rows`` (indices into N)."""
    rows = np.asarray(rows)
    w = _rows(codes, lut, scales, group, rows, zeros, types).astype(np.float64)
    x64 = x.astype(np.float64)
    return x64 @ w.T, np.abs(x64) @ np.abs(w).T


# -- acceptance ---------------------------------------------------------------

REL_TOL = 1e-3
ABS_TOL = 1e-5


def error_bound(B: np.ndarray) -> np.ndarray:
    """Per-output tolerance 1e-3 * sum_k |x_k * w_k| + 1e-5."""
    return REL_TOL * B + ABS_TOL


BF16_UNIT_ROUNDOFF = 2.0 ** -8


def error_bound_bf16(B: np.ndarray, y_ref: np.ndarray) -> np.ndarray:
    """Tolerance for bf16 outputs: the fp16-output bound plus the rounding of
    the fp32 result to bf16 (8 significand bits: at most 2^-8 |y| relative,
    applied to |y_ref| plus the accumulation bound)."""
    acc = REL_TOL * B + ABS_TOL
    return acc + BF16_UNIT_ROUNDOFF * (np.abs(y_ref) + acc)


def check(y: np.ndarray, y_ref: np.ndarray, B: np.ndarray, out: str = "fp16"):
    """(ok, worst): ok when every |y - y_ref| <= the bound (error_bound(B), or
    error_bound_bf16 for bf16 outputs); worst is max(err / bound)."""
    err = np.abs(y.astype(np.float64) - y_ref)
    bound = error_bound(B) if out == "fp16" else error_bound_bf16(B, y_ref)
    ratio = err / bound
    worst = float(ratio.max()) if ratio.size else 0.0
    return bool(np.all(np.isfinite(y)) and worst <= 1.0), worst
