"""Pins of the projection oracle (oracle/proj.py) against what does not
depend on it: per-element sums written as loops, identity and zero weights,
the bias alone, linearity, and the relative rows behaving as tokens."""
import numpy as np
import pytest

import oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("T,E,H,D,R", [(5, 6, 2, 3, 4), (3, 8, 1, 4, 2)])
def test_brute_force_loops(T, E, H, D, R):
    rng = np.random.default_rng(7)
    x, w, b, rel = _rand(rng, T, E), _rand(rng, 3 * H * D, E), _rand(rng, 3 * H * D), _rand(rng, R, E)
    q, k, v, q_r, k_r = oracle.qkv_projection(x, w, b, rel, H, D)
    for which, out in enumerate((q, k, v)):
        for t in range(T):
            for h in range(H):
                for d in range(D):
                    n = which * H * D + h * D + d
                    ref = b[n]
                    for e in range(E):
                        ref += x[t, e] * w[n, e]
                    assert abs(out[t, h, d] - ref) <= 1e-12 * (1 + abs(ref))
    for which, out in enumerate((q_r, k_r)):
        for h in range(H):
            for r in range(R):
                for d in range(D):
                    n = which * H * D + h * D + d
                    ref = b[n] + sum(rel[r, e] * w[n, e] for e in range(E))
                    assert abs(out[h, r, d] - ref) <= 1e-12 * (1 + abs(ref))


def test_identity_weights_split_heads():
    """W_q = I (E = H D): q is x cut into heads, in order."""
    rng = np.random.default_rng(1)
    H, D, T = 3, 4, 5
    x = _rand(rng, T, H * D)
    w = np.zeros((3 * H * D, H * D))
    w[:H * D] = np.eye(H * D)
    w[2 * H * D:] = 2 * np.eye(H * D)
    q, k, v, _, _ = oracle.qkv_projection(x, w, None, None, H, D)
    for h in range(H):
        np.testing.assert_array_equal(q[:, h, :], x[:, h * D:(h + 1) * D])
    np.testing.assert_array_equal(k, 0)
    np.testing.assert_array_equal(v, 2 * x.reshape(T, H, D))


def test_bias_only_and_linearity():
    rng = np.random.default_rng(2)
    H, D, E, T, R = 2, 4, 6, 3, 5
    w, b = _rand(rng, 3 * H * D, E), _rand(rng, 3 * H * D)
    q, k, v, q_r, k_r = oracle.qkv_projection(np.zeros((T, E)), w, b, np.zeros((R, E)), H, D)
    np.testing.assert_array_equal(v, np.broadcast_to(b[2 * H * D:].reshape(H, D), (T, H, D)))
    np.testing.assert_array_equal(q_r, np.broadcast_to(b[:H * D].reshape(H, 1, D), (H, R, D)))
    x1, x2 = _rand(rng, T, E), _rand(rng, T, E)
    a1 = oracle.qkv_projection(x1, w, None, None, H, D)
    a2 = oracle.qkv_projection(x2, w, None, None, H, D)
    a12 = oracle.qkv_projection(2 * x1 - 3 * x2, w, None, None, H, D)
    for i in range(3):
        np.testing.assert_allclose(a12[i], 2 * a1[i] - 3 * a2[i], rtol=1e-12, atol=1e-12)


def test_relative_rows_are_projected_like_tokens():
    """q_r[h, r] and k_r[h, r] equal the q and k of a token whose hidden state
    is rel[r] (shared attention key)."""
    rng = np.random.default_rng(3)
    H, D, E, R = 2, 3, 5, 4
    w, b, rel = _rand(rng, 3 * H * D, E), _rand(rng, 3 * H * D), _rand(rng, R, E)
    q, k, _, q_r, k_r = oracle.qkv_projection(rel, w, b, rel, H, D)
    np.testing.assert_allclose(q_r, q.transpose(1, 0, 2), rtol=0, atol=1e-13)
    np.testing.assert_allclose(k_r, k.transpose(1, 0, 2), rtol=0, atol=1e-13)


def test_backward_finite_differences():
    """The projection backward against central differences of the forward
    oracle (the maps are linear in each argument, so the differences are
    exact up to rounding)."""
    rng = np.random.default_rng(9)
    T, E, H, D, R = 4, 6, 2, 3, 5
    HD = H * D
    x, w, b, rel = _rand(rng, T, E), _rand(rng, 3 * HD, E), _rand(rng, 3 * HD), _rand(rng, R, E)
    G = [_rand(rng, T, H, D) for _ in range(3)] + [_rand(rng, H, R, D) for _ in range(2)]

    def loss(x_, w_, b_, rel_):
        outs = oracle.qkv_projection(x_, w_, b_, rel_, H, D)
        return sum(float((o * g).sum()) for o, g in zip(outs, G))

    dx, dw, db, drel = oracle.qkv_projection_backward(x, w, rel, *G, H, D)
    eps = 1e-6
    for arr, grad in ((x, dx), (w, dw), (b, db), (rel, drel)):
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            lp = loss(x, w, b, rel)
            arr[idx] = old - eps
            lm = loss(x, w, b, rel)
            arr[idx] = old
            assert abs((lp - lm) / (2 * eps) - grad[idx]) <= 1e-6 * (1 + abs(grad[idx]))


def test_backward_without_relative_rows():
    rng = np.random.default_rng(10)
    T, E, H, D = 3, 4, 1, 2
    x, w = _rand(rng, T, E), _rand(rng, 3 * H * D, E)
    G = [_rand(rng, T, H, D) for _ in range(3)]
    dx, dw, db, drel = oracle.qkv_projection_backward(x, w, None, *G, None, None, H, D)
    assert drel is None
    dY = np.concatenate([g.reshape(T, -1) for g in G], axis=1)
    for t in range(T):
        for e in range(E):
            assert abs(dx[t, e] - sum(dY[t, n] * w[n, e] for n in range(3 * H * D))) < 1e-12
    np.testing.assert_allclose(db, dY.sum(axis=0), rtol=0, atol=1e-12)
