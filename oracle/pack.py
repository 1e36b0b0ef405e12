"""Plain oracle of the packing helpers for the packed layout.

TEST INFRASTRUCTURE ONLY (as the rest of ``oracle/``).

What is computed (the DisentangledFlash 1.1.1 page, "Packed unpadded
inference and training": right-padded ``[B, L, ...]`` input is converted to
the FlashAttention-style ``[total_tokens, ...]`` layout with ``cu_seqlens``,
and the packed output is converted back). Reading used here: sequence b's
length is the number of valid tokens in row b of the mask; its valid tokens,
in order, become rows ``cu_seqlens[b] .. cu_seqlens[b+1]-1`` of the packed
tensor (for a right-padded mask these are its first tokens);
``cu_seqlens[0] = 0`` and ``cu_seqlens[b+1] = cu_seqlens[b] + length_b``;
``max_seqlen`` is the largest length. Unpacking writes the rows back to their
positions and zeros everywhere else.
"""
from __future__ import annotations

import numpy as np


def pack_padded(padded, mask):
    """``padded`` ``[B, L, ...]``, ``mask`` ``[B, L]`` (nonzero = valid).
    Returns (packed ``[T, ...]``, cu_seqlens int32 ``[B+1]``, max_seqlen)."""
    padded = np.asarray(padded)
    mask = np.asarray(mask) != 0
    B = mask.shape[0]
    rows, lengths = [], []
    for b in range(B):
        idx = [l for l in range(mask.shape[1]) if mask[b, l]]
        lengths.append(len(idx))
        rows.extend(padded[b, l] for l in idx)
    cu = np.zeros(B + 1, dtype=np.int32)
    for b in range(B):
        cu[b + 1] = cu[b] + lengths[b]
    packed = np.stack(rows) if rows else np.zeros((0,) + padded.shape[2:], dtype=padded.dtype)
    return packed, cu, (max(lengths) if lengths else 0)


def unpack_packed(packed, cu_seqlens, max_len: int, mask):
    """Inverse of :func:`pack_padded` for the same mask: ``[B, max_len, ...]``
    with the packed rows at the valid positions and zeros elsewhere."""
    packed = np.asarray(packed)
    mask = np.asarray(mask) != 0
    B = len(cu_seqlens) - 1
    out = np.zeros((B, max_len) + packed.shape[1:], dtype=packed.dtype)
    for b in range(B):
        t = int(cu_seqlens[b])
        for l in range(max_len):
            if mask[b, l]:
                out[b, l] = packed[t]
                t += 1
    return out
