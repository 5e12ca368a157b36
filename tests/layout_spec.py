"""An independent numpy reading of the packed "wave-block" layout.

Written from the layout description in include/lutq.h only (it shares no code
with the HIP repack/unpack kernels): rows in tiles of 16, K in chunks of 128,
block (t, c) at byte offset (t * K/128 + c) * 256 * bits, lane slot
L = 16 q + r holding row 16 t + r at k = 128 c + 32 j + 8 q + e.
"""

from __future__ import annotations

import numpy as np

HI_OFFSET = (4, 6, 0, 2)  # bit offset of the 3-bit high pair in byte e/2, by k-step j


def _slot_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes [N, K] -> [ntiles, nchunks, 64 slots, 4 (j), 8 (e)] with zero padding rows."""
    N, K = codes.shape
    nt = -(-N // 16)
    padded = np.zeros((nt * 16, K), np.uint8)
    padded[:N] = codes & ((1 << bits) - 1)
    # [t, r, c, j, q, e]
    v = padded.reshape(nt, 16, K // 128, 4, 4, 8)
    # slot L = 16 q + r  -> [t, c, q, r, j, e]
    v = v.transpose(0, 2, 4, 1, 3, 5)
    return v.reshape(nt, K // 128, 64, 4, 8).astype(np.uint32)


def encode(codes: np.ndarray, bits: int) -> np.ndarray:
    """Bytes of the wave-block layout for uint8 codes [N, K] (K % 128 == 0)."""
    s = _slot_codes(codes, bits)
    ev, od = s[..., 0::2], s[..., 1::2]          # [.., j, i] even/odd codes of pair i
    sh = (8 * np.arange(4, dtype=np.uint32))     # byte i
    if bits == 4:
        words = ((ev | (od << 4)) << sh).sum(-1, dtype=np.uint32)            # [.., j]
    else:
        nib = (ev & 3) | ((od & 3) << 2)                                     # [.., j, i]
        lo = np.zeros(s.shape[:-2] + (2,), np.uint32)
        for j in range(4):
            lo[..., j >> 1] |= ((nib[..., j, :] << (4 * (j & 1))) << sh).sum(-1, dtype=np.uint32)
        if bits == 2:
            words = lo
        else:
            hb = (ev >> 2) | ((od >> 2) << 1)
            hi = np.zeros(s.shape[:-2], np.uint32)
            for j in range(4):
                hi |= (hb[..., j, :] << (sh + HI_OFFSET[j])).sum(-1, dtype=np.uint32)
            words = np.concatenate([lo, hi[..., None]], axis=-1)
    return words.astype("<u4").reshape(-1).view(np.uint8)


def decode(packed: np.ndarray, N: int, K: int, bits: int) -> np.ndarray:
    """uint8 codes [N, K] from wave-block bytes."""
    nt = -(-N // 16)
    w = np.ascontiguousarray(packed[: nt * 16 * K * bits // 8]).view("<u4").astype(np.uint32)
    w = w.reshape(nt, K // 128, 64, bits)
    sh = 8 * np.arange(4, dtype=np.uint32)
    out = np.zeros((nt, K // 128, 64, 4, 8), np.uint32)
    for j in range(4):
        for i in range(4):
            if bits == 4:
                byte = (w[..., j] >> sh[i]) & 0xFF
                c0, c1 = byte & 15, byte >> 4
            else:
                nib = (w[..., j >> 1] >> (sh[i] + 4 * (j & 1))) & 15
                c0, c1 = nib & 3, nib >> 2
                if bits == 3:
                    hb = (w[..., 2] >> (sh[i] + HI_OFFSET[j])) & 3
                    c0 = c0 | ((hb & 1) << 2)
                    c1 = c1 | ((hb >> 1) << 2)
            out[..., j, 2 * i] = c0
            out[..., j, 2 * i + 1] = c1
    # [t, c, q, r, j, e] -> [t, r, c, j, q, e]
    v = out.reshape(nt, K // 128, 4, 16, 4, 8).transpose(0, 3, 1, 4, 2, 5)
    return v.reshape(nt * 16, K)[:N].astype(np.uint8)
