"""Plain, slow, float64 oracle for exact DeBERTa-v2/v3 disentangled attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s CPU-baseline leg, never by the product path.

What is computed (the DisentangledFlash 1.1.1 page, "Status": exact,
bidirectional DeBERTa-v2/v3-style C2P/P2C attention without the [B,H,L,L]
matrix on the GPU; "Hugging Face usage": the LSE-producing forward and the
relative-projection gradients; "Performance": which score products exist).
The page never writes the formula out; the readings used here are:

* scores, per sequence and head, with local positions i (query), j (key)::

      S[i,j] = s * ( Q_i.K_j + Q_i.K_r[delta(i,j)] + K_j.Q_r[delta(j,i)] )
      s = 1 / sqrt(3 D)

* ``delta(a, b) = clamp(bucket(a - b) + att, 0, R - 1)``, ``att = buckets`` if
  ``buckets > 0`` else ``span``, ``R = 2 att`` (DeBERTa-v2/v3 relative index);
* ``bucket(d) = d`` if ``buckets == 0`` or ``|d| <= mid`` (``mid = buckets // 2``),
  otherwise ``sign(d) * (mid + ceil((mid - 1) ln(|d|/mid) / ln((span-1)/mid)))``
  with the ceiling taken in exact arithmetic;
* factorized padding mask ("Status": factorized 2-D padding masks): pair (i,j)
  is scored iff both tokens are valid; a masked query row has output 0 and
  LSE = -inf; pairs from different packed sequences are never scored
  ("Packed unpadded inference and training": cu_seqlens layout);
* LSE is the natural log of the row's sum of exp(S); q_r and k_r are
  ``[H, R, D]`` and shared by every sequence, so their gradients sum over all
  sequences.

Every array here is float64 and is materialised in full; nothing is blocked,
fused or reordered beyond the definition.
"""
from __future__ import annotations

import functools
import math
from typing import Optional

import numpy as np


# ----------------------------------------------------------------------------
# relative-position index

def att_and_rows(span: int, buckets: int) -> tuple:
    """``(att, R)``: the half-width and the number of relative-position rows."""
    att = buckets if buckets > 0 else span
    return att, 2 * att


def bucket_exact(d: int, span: int, buckets: int) -> int:
    """DeBERTa-v2/v3 log-bucketed relative position, ceiling taken exactly.

    For ``|d| > mid`` the bucket is ``mid + k`` with ``k`` the least integer
    ``>= (mid-1) ln(a/mid) / ln(b/mid)`` (a = |d|, b = span - 1). Because
    ``ln(b/mid) > 0`` this is the least ``k`` with
    ``b^k * mid^(mid-1) >= a^(mid-1) * mid^k``, decided here with Python's
    unbounded integers.
    """
    d = int(d)
    if buckets <= 0:
        return d
    mid = buckets // 2
    a = abs(d)
    if a <= mid:
        return d
    b = span - 1
    if b <= mid:
        raise ValueError("log buckets need span - 1 > buckets / 2")
    lhs = a ** (mid - 1)
    mid_pow = mid ** (mid - 1)

    def holds(k: int) -> bool:
        return b ** k * mid_pow >= lhs * mid ** k

    # start from a floating estimate, then settle it with exact comparisons
    k = max(0, int(math.floor((mid - 1) * math.log(a / mid) / math.log(b / mid))) - 1)
    while holds(k) and k > 0 and holds(k - 1):
        k -= 1
    while not holds(k):
        k += 1
    return int(math.copysign(mid + k, d))


@functools.lru_cache(maxsize=16)
def _bucket_range(lim: int, span: int, buckets: int) -> np.ndarray:
    """``bucket(d)`` for d in [-lim, lim] (cached; index d + lim)."""
    return np.array([bucket_exact(x, span, buckets) for x in range(-lim, lim + 1)],
                    dtype=np.int64)


def _delta_table(lo: int, hi: int, span: int, buckets: int) -> np.ndarray:
    """``clamp(bucket(d) + att, 0, R - 1)`` for every integer d in [lo, hi]."""
    att, R = att_and_rows(span, buckets)
    lim = max(abs(lo), abs(hi))
    lim = 1 << max(4, (lim - 1).bit_length())  # a few cached sizes cover every call
    b = _bucket_range(lim, span, buckets)[lo + lim: hi + lim + 1]
    return np.clip(b + att, 0, R - 1)


def delta(rel: np.ndarray, span: int, buckets: int) -> np.ndarray:
    """``clamp(bucket(rel) + att, 0, R - 1)`` elementwise, for an int array."""
    rel = np.asarray(rel, dtype=np.int64)
    if rel.size == 0:
        return rel.copy()
    lo, hi = int(rel.min()), int(rel.max())
    return _delta_table(lo, hi, span, buckets)[rel - lo]


P2C_CONVENTIONS = ("literal", "shared")


def p2c_rows(rel: np.ndarray, span: int, buckets: int, p2c: str = "literal") -> np.ndarray:
    """Row of Q_r that pair (i, j) uses, for ``rel = i - j``.

    ``"literal"``: ``delta(j, i)``, the P2C index as the method's score formula
    writes it. ``"shared"``: ``delta(i, j)``, the same row as C2P, which is
    how deployed DeBERTa-v2/v3 code indexes P2C in self-attention (only this
    index changes between the two)."""
    if p2c == "literal":
        return delta(-np.asarray(rel), span, buckets)
    if p2c == "shared":
        return delta(np.asarray(rel), span, buckets)
    raise ValueError(f"unknown P2C convention {p2c!r}")


def rel_luts(max_seqlen: int, span: int, buckets: int) -> tuple:
    """The two relative-index tables over ``d = i - j``.

    Index ``d + max_seqlen - 1`` for ``d`` in ``[-(max_seqlen-1), max_seqlen-1]``.
    ``c2p[d] = delta(i, j)`` (row of K_r seen by query i against key j) and
    ``p2c[d] = delta(j, i)`` (row of Q_r seen by key j against query i).
    """
    d = np.arange(-(max_seqlen - 1), max_seqlen, dtype=np.int64)
    return (delta(d, span, buckets).astype(np.int32),
            delta(-d, span, buckets).astype(np.int32))


# ----------------------------------------------------------------------------
# sequences and scores

def sequences(total_tokens: int, cu_seqlens=None, batch: Optional[int] = None,
              seqlen: Optional[int] = None) -> list:
    """``[(start, end), ...]`` token ranges of the sequences."""
    if cu_seqlens is not None:
        cu = [int(x) for x in np.asarray(cu_seqlens)]
        return [(cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    if batch is None:
        batch = 1
    if seqlen is None:
        seqlen = total_tokens // batch
    assert batch * seqlen == total_tokens
    return [(b * seqlen, (b + 1) * seqlen) for b in range(batch)]


def _valid(key_mask, st: int, en: int) -> np.ndarray:
    if key_mask is None:
        return np.ones(en - st, dtype=bool)
    return np.asarray(key_mask[st:en]).astype(bool)


def scores(Q, K, q_r_h, k_r_h, span: int, buckets: int, p2c: str = "literal") -> np.ndarray:
    """Unmasked score matrix ``S[i, j]`` for one sequence and one head.

    ``Q, K`` are ``[L, D]``; ``q_r_h, k_r_h`` are ``[R, D]``. The two L x R
    products are formed first and then gathered with explicit index arrays.
    """
    L, D = Q.shape
    s = 1.0 / math.sqrt(3.0 * D)
    idx = np.arange(L)
    rel = idx[:, None] - idx[None, :]
    ci = delta(rel, span, buckets)          # delta(i, j)
    pi = p2c_rows(rel, span, buckets, p2c)  # delta(j, i) (literal) or delta(i, j) (shared)
    c2p_full = Q @ k_r_h.T                  # [L, R]: Q_i . K_r[r]
    p2c_full = K @ q_r_h.T                  # [L, R]: K_j . Q_r[r]
    c2p = np.take_along_axis(c2p_full, ci, axis=1)          # [i, j] -> row i
    p2c_term = p2c_full[idx[None, :], pi]                    # [i, j] -> row j
    return s * (Q @ K.T + c2p + p2c_term)


def _probs(S: np.ndarray, valid: np.ndarray) -> tuple:
    """Masked softmax of one score matrix: ``(P, lse)``; masked rows give 0/-inf."""
    L = S.shape[0]
    pair = valid[:, None] & valid[None, :]
    Sm = np.where(pair, S, -np.inf)
    lse = np.full(L, -np.inf)
    P = np.zeros_like(S)
    rows = np.nonzero(valid)[0]
    if rows.size:
        mx = Sm[rows].max(axis=1)
        lse[rows] = mx + np.log(np.exp(Sm[rows] - mx[:, None]).sum(axis=1))
        P[rows] = np.exp(Sm[rows] - lse[rows][:, None])
    return P, lse


# ----------------------------------------------------------------------------
# forward

def _dropout_factor(dropout, n, h, H, L):
    """[L, L] factor keep / (1 - p) of attention dropout (1 where none), the
    mask from ``philox.keep_mask`` (the DisentangledFlash page, "Status":
    attention-probability dropout inside the fused kernels)."""
    if dropout is None:
        return 1.0
    from . import philox
    p, seed, offset = dropout
    return philox.keep_mask(p, seed, offset, n, h, H, L) * (1.0 / (1.0 - p))


def forward(q, k, v, q_r, k_r, span: int, buckets: int, key_mask=None,
            cu_seqlens=None, batch=None, seqlen=None, return_probs: bool = False,
            heads=None, dropout=None, p2c: str = "literal"):
    """Output ``[T, H, D]`` and LSE ``[H, T]`` (natural log), float64.

    ``q, k, v`` are ``[T, H, D]``; ``q_r, k_r`` are ``[H, R, D]``.
    ``heads`` restricts the work to a subset of heads (other heads are left
    0 / -inf). With ``return_probs`` also returns ``{(seq, head): P}``.
    ``dropout = (p, seed, offset)`` applies attention-probability dropout
    after the softmax: out = (P * keep / (1 - p)) V; the LSE is that of the
    undropped scores. ``p2c`` selects the P2C row convention (:func:`p2c_rows`).
    """
    q, k, v, q_r, k_r = (np.asarray(x, dtype=np.float64) for x in (q, k, v, q_r, k_r))
    T, H, D = q.shape
    _, R = att_and_rows(span, buckets)
    assert q_r.shape == (H, R, D) and k_r.shape == (H, R, D)
    out = np.zeros((T, H, D))
    lse = np.full((H, T), -np.inf)
    probs = {}
    hs = range(H) if heads is None else heads
    for n, (st, en) in enumerate(sequences(T, cu_seqlens, batch, seqlen)):
        valid = _valid(key_mask, st, en)
        for h in hs:
            S = scores(q[st:en, h], k[st:en, h], q_r[h], k_r[h], span, buckets, p2c)
            P, l = _probs(S, valid)
            out[st:en, h] = (P * _dropout_factor(dropout, n, h, H, en - st)) @ v[st:en, h]
            lse[h, st:en] = l
            if return_probs:
                probs[(n, h)] = P
    if return_probs:
        return out, lse, probs
    return out, lse


# ----------------------------------------------------------------------------
# backward

def backward(q, k, v, q_r, k_r, dout, span: int, buckets: int, key_mask=None,
             cu_seqlens=None, batch=None, seqlen=None, heads=None,
             return_strips: bool = False, dropout=None, p2c: str = "literal"):
    """Gradients of ``sum(out * dout)``: ``dq, dk, dv, dq_r, dk_r``, float64.

    Follows the chain rule of the forward step by step: dV = P^T dO,
    dP = dO V^T, Delta_i = sum_j P_ij dP_ij, dS = P (dP - Delta), then the
    segmented sums of dS into the two relative strips
    ``dC2P[i, r] = sum_{j: delta(i,j) = r} dS[i, j]`` and
    ``dP2C[j, r] = sum_{i: delta(j,i) = r} dS[i, j]``, and finally
    ``dQ = s (dS K + dC2P K_r)``, ``dK = s (dS^T Q + dP2C Q_r)``,
    ``dK_r = s sum dC2P^T Q``, ``dQ_r = s sum dP2C^T K`` (sums over all
    sequences). ``heads`` restricts the work to a subset of heads (other heads
    are left zero). With ``return_strips`` also returns
    ``{(seq, head): (dC2P, dP2C)}``. With ``dropout`` (see ``forward``) the
    factor F = keep / (1 - p) enters as dV = (P F)^T dO and
    dS = P (F dP - Delta), Delta_i = sum_j P_ij F_ij dP_ij (= dO_i . O_i).
    """
    q, k, v, q_r, k_r, dout = (np.asarray(x, dtype=np.float64)
                               for x in (q, k, v, q_r, k_r, dout))
    T, H, D = q.shape
    _, R = att_and_rows(span, buckets)
    s = 1.0 / math.sqrt(3.0 * D)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dq_r = np.zeros_like(q_r)
    dk_r = np.zeros_like(k_r)
    strips = {}
    hs = range(H) if heads is None else heads
    for n, (st, en) in enumerate(sequences(T, cu_seqlens, batch, seqlen)):
        L = en - st
        valid = _valid(key_mask, st, en)
        idx = np.arange(L)
        rel = idx[:, None] - idx[None, :]
        ci = delta(rel, span, buckets)
        pi = p2c_rows(rel, span, buckets, p2c)
        for h in hs:
            Q, K, V, dO = q[st:en, h], k[st:en, h], v[st:en, h], dout[st:en, h]
            S = scores(Q, K, q_r[h], k_r[h], span, buckets, p2c)
            P, _ = _probs(S, valid)
            F = _dropout_factor(dropout, n, h, H, L)
            dV = (P * F).T @ dO
            dP = (dO @ V.T) * F
            Delta = (P * dP).sum(axis=1)
            dS = P * (dP - Delta[:, None])
            # segmented sums (a scatter-add written with bincount)
            rows_i = np.broadcast_to(idx[:, None], (L, L))
            cols_j = np.broadcast_to(idx[None, :], (L, L))
            dC2P = np.bincount((rows_i * R + ci).ravel(), weights=dS.ravel(),
                               minlength=L * R).reshape(L, R)
            dP2C = np.bincount((cols_j * R + pi).ravel(), weights=dS.ravel(),
                               minlength=L * R).reshape(L, R)
            dq[st:en, h] = s * (dS @ K + dC2P @ k_r[h])
            dk[st:en, h] = s * (dS.T @ Q + dP2C @ q_r[h])
            dv[st:en, h] = dV
            dk_r[h] += s * (dC2P.T @ Q)
            dq_r[h] += s * (dP2C.T @ K)
            if return_strips:
                strips[(n, h)] = (dC2P, dP2C)
    if return_strips:
        return dq, dk, dv, dq_r, dk_r, strips
    return dq, dk, dv, dq_r, dk_r


# ----------------------------------------------------------------------------
# row-sampled evaluation (large workloads)

def _row_scores(Q, K, q_r_h, k_r_h, rows, span, buckets, p2c="literal"):
    """``S[rows, :]`` for one sequence and head, without the full L x L matrix."""
    L, D = K.shape
    s = 1.0 / math.sqrt(3.0 * D)
    rows = np.asarray(rows, dtype=np.int64)
    jdx = np.arange(L)
    rel = rows[:, None] - jdx[None, :]
    ci = delta(rel, span, buckets)
    pi = p2c_rows(rel, span, buckets, p2c)
    c2p_full = Q[rows] @ k_r_h.T
    p2c_full = K @ q_r_h.T
    c2p = np.take_along_axis(c2p_full, ci, axis=1)
    p2c_term = p2c_full[jdx[None, :], pi]
    return s * (Q[rows] @ K.T + c2p + p2c_term), ci


def forward_rows(q, k, v, q_r, k_r, span, buckets, seq: tuple, head: int,
                 rows, key_mask=None, p2c="literal"):
    """Output and LSE of the given local query ``rows`` of one sequence/head."""
    st, en = seq
    Q, K, V = (np.asarray(x[st:en, head], dtype=np.float64) for x in (q, k, v))
    S, _ = _row_scores(Q, K, np.asarray(q_r[head], np.float64),
                       np.asarray(k_r[head], np.float64), rows, span, buckets, p2c)
    valid = _valid(key_mask, st, en)
    rows = np.asarray(rows)
    Sm = np.where(valid[rows][:, None] & valid[None, :], S, -np.inf)
    out = np.zeros((len(rows), Q.shape[1]))
    lse = np.full(len(rows), -np.inf)
    for n in range(len(rows)):
        if not valid[rows[n]]:
            continue
        mx = Sm[n].max()
        lse[n] = mx + math.log(np.exp(Sm[n] - mx).sum())
        out[n] = np.exp(Sm[n] - lse[n]) @ V
    return out, lse


def dq_rows(q, k, v, q_r, k_r, dout, span, buckets, seq: tuple, head: int,
            rows, key_mask=None, p2c="literal"):
    """dQ of the given local query ``rows`` of one sequence/head.

    A row of dQ needs only its own rows of S, P, dP and dS, and its own row
    of dC2P: ``dQ_i = s (dS_i K + dC2P_i K_r)``.
    """
    st, en = seq
    Q, K, V, dO = (np.asarray(x[st:en, head], dtype=np.float64)
                   for x in (q, k, v, dout))
    k_r_h = np.asarray(k_r[head], np.float64)
    L, D = Q.shape
    R = k_r_h.shape[0]
    s = 1.0 / math.sqrt(3.0 * D)
    S, ci = _row_scores(Q, K, np.asarray(q_r[head], np.float64), k_r_h, rows,
                        span, buckets, p2c)
    valid = _valid(key_mask, st, en)
    rows = np.asarray(rows)
    out = np.zeros((len(rows), D))
    for n in range(len(rows)):
        if not valid[rows[n]]:
            continue
        Sm = np.where(valid, S[n], -np.inf)
        mx = Sm.max()
        P = np.exp(Sm - (mx + math.log(np.exp(Sm - mx).sum())))
        dP = dO[rows[n]] @ V.T
        dS = P * (dP - (P * dP).sum())
        dC2P = np.bincount(ci[n], weights=dS, minlength=R)
        out[n] = s * (dS @ K + dC2P @ k_r_h)
    return out
