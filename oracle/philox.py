"""Philox4x32-10 and the attention-dropout mask, for the oracle.

TEST INFRASTRUCTURE ONLY (see ``df_oracle``).

Philox4x32 is the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel random numbers: as easy as 1, 2, 3" (SC 2011). One round maps the
counter (c0, c1, c2, c3) and key (k0, k1) to
    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))
with M0 = 0xD2511F53, M1 = 0xCD9E8D57 (32 x 32 -> 64-bit products); the key is
bumped by the Weyl constants W0 = 0x9E3779B9, W1 = 0xBB67AE85 before every
round after the first; 10 rounds.

Attention dropout (DisentangledFlash 1.1.1 page, "Status": the fused kernels
apply dropout to the attention probabilities, and the backward recomputes the
mask from the Philox counter rather than saving it). The pages do not
fix the counter layout or how many random bits a pair takes; the reading
used here (and by the kernels): for sequence n of the batch, head h, local
query i and local key j, one call covers the eight keys 8m .. 8m+7 of a query,
    counter = (j // 8, i, n * H + h, offset),  key = (seed mod 2^32, seed >> 32),
and key j takes 16 bits of it: word (j % 8) // 2 of the output, its low half
for even j and its high half for odd j. The pair is kept iff those 16 bits,
read as an unsigned number, are >= floor(p * 2^16); kept probabilities are
scaled by 1 / (1 - p).
"""
from __future__ import annotations

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
_U32 = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox4x32 rounds on arrays of 32-bit counters (any broadcastable
    shapes); returns the four output words as uint64 arrays holding 32-bit values."""
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & np.uint64(_U32) for x in (c0, c1, c2, c3))
    k0 = np.uint64(int(k0) & _U32)
    k1 = np.uint64(int(k1) & _U32)
    m0, m1, u32 = np.uint64(M0), np.uint64(M1), np.uint64(_U32)
    for r in range(10):
        if r:
            k0 = np.uint64((int(k0) + W0) & _U32)
            k1 = np.uint64((int(k1) + W1) & _U32)
        p0 = m0 * c0
        p1 = m1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & u32
        hi1, lo1 = p1 >> np.uint64(32), p1 & u32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def keep_threshold(p: float) -> int:
    """16-bit values >= this keep their pair (p in [0, 1))."""
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return int(np.floor(p * 65536.0))


def keep_mask(p: float, seed: int, offset: int, n: int, h: int, H: int, L: int) -> np.ndarray:
    """Boolean [L, L] keep mask of sequence n, head h (rows: queries i, columns: keys j)."""
    thr = keep_threshold(p)
    if L == 0:  # an empty sequence has no pairs
        return np.zeros((0, 0), dtype=bool)
    i = np.arange(L, dtype=np.uint64)[:, None]
    jb = np.arange((L + 7) // 8, dtype=np.uint64)[None, :]
    words = philox4x32_10(jb, i, np.uint64(n * H + h), np.uint64(offset & _U32), seed & _U32,
                          (seed >> 32) & _U32)
    w = np.stack(words, axis=-1)  # [L, blocks, 4]
    halves = np.stack([w & np.uint64(0xFFFF), w >> np.uint64(16)], axis=-1)  # [L, blocks, 4, 2]
    bits16 = halves.reshape(L, -1)[:, :L]  # key j: half j % 2 of word (j % 8) // 2 of block j // 8
    return bits16 >= np.uint64(thr)
