"""Plain float64 oracle of the fused Q/K/V and relative-position projections.

TEST INFRASTRUCTURE ONLY (as the rest of ``oracle/``): imported by ``tests/``
and never by the product path.

What is computed (the DisentangledFlash 1.1.1 page, "Status": the fused QKV
projection is always enabled; "Hugging Face usage": the Q/K/V and
relative-position projections stay in the model's graph). The page does not
write the projections out; the reading used here is the DeBERTa-v2/v3 one
with a shared attention key: three linear maps of the hidden states with
weights stacked as one ``[3 H D, E]`` matrix (rows ``W_q``, ``W_k``, ``W_v``)
and one bias ``[3 H D]``, and the relative-position embedding rows projected
by the same query and key maps::

    q[t, h, d]   = sum_e x[t, e]   W[h D + d, e]         + b[h D + d]
    k[t, h, d]   = sum_e x[t, e]   W[H D + h D + d, e]   + b[H D + h D + d]
    v[t, h, d]   = sum_e x[t, e]   W[2 H D + h D + d, e] + b[2 H D + h D + d]
    q_r[h, r, d] = sum_e rel[r, e] W[h D + d, e]         + b[h D + d]
    k_r[h, r, d] = sum_e rel[r, e] W[H D + h D + d, e]   + b[H D + h D + d]

The whole product is one matrix multiplication (a library primitive) followed
by the split into heads; nothing else is fused or reordered.
"""
from __future__ import annotations

import numpy as np


def qkv_projection(x, w, b, rel, H: int, D: int):
    """Returns q, k, v ``[T, H, D]`` and, when ``rel`` is given, q_r, k_r
    ``[H, R, D]`` (float64). ``x`` ``[T, E]``, ``w`` ``[3 H D, E]``, ``b``
    ``[3 H D]`` or None, ``rel`` ``[R, E]`` or None."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    HD = H * D
    assert w.shape == (3 * HD, x.shape[1])
    bias = np.zeros(3 * HD) if b is None else np.asarray(b, dtype=np.float64)
    y = x @ w.T + bias                                   # [T, 3 H D]
    q, k, v = (y[:, i * HD:(i + 1) * HD].reshape(-1, H, D) for i in range(3))
    if rel is None:
        return q, k, v, None, None
    rel = np.asarray(rel, dtype=np.float64)
    yr = rel @ w[:2 * HD].T + bias[:2 * HD]              # [R, 2 H D]
    q_r = yr[:, :HD].reshape(-1, H, D).transpose(1, 0, 2)   # [H, R, D]
    k_r = yr[:, HD:].reshape(-1, H, D).transpose(1, 0, 2)
    return q, k, v, q_r, k_r


def qkv_projection_backward(x, w, rel, dq, dk, dv, dq_r, dk_r, H: int, D: int):
    """Gradients of the projections above for output gradients dq, dk, dv
    ``[T, H, D]`` and (with ``rel``) dq_r, dk_r ``[H, R, D]``: returns
    (dx ``[T, E]``, dw ``[3 H D, E]``, db ``[3 H D]``, drel ``[R, E]`` or None),
    float64. Each map is linear, so with dY the output gradients laid out like
    the GEMM's output (``[T, 3 H D]``, and ``[R, 2 H D]`` for the relative
    rows): dx = dY W, drel = dY_r W[:2HD], dW = dY^T x + [dY_r^T rel; 0],
    db = column sums of dY and dY_r."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T = x.shape[0]
    HD = H * D
    dY = np.concatenate([np.asarray(g, dtype=np.float64).reshape(T, HD) for g in (dq, dk, dv)], axis=1)
    dx = dY @ w
    dw = dY.T @ x
    db = dY.sum(axis=0)
    drel = None
    if rel is not None:
        rel = np.asarray(rel, dtype=np.float64)
        R = rel.shape[0]
        dYr = np.concatenate([np.asarray(g, dtype=np.float64).transpose(1, 0, 2).reshape(R, HD)
                              for g in (dq_r, dk_r)], axis=1)                    # [R, 2 H D]
        drel = dYr @ w[:2 * HD]
        dw[:2 * HD] += dYr.T @ rel
        db[:2 * HD] += dYr.sum(axis=0)
    return dx, dw, db, drel
