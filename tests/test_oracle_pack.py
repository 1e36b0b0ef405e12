"""Pins of the packing oracle (oracle/pack.py): a hand-written example, the
round trip, and the link to the attention oracle (packed attention on the
packed rows equals padded attention with the same right-padding mask, on the
valid rows)."""
import numpy as np

import oracle


def test_hand_example():
    x = np.arange(2 * 4 * 3).reshape(2, 4, 3)
    m = np.array([[1, 1, 0, 0], [1, 1, 1, 0]])
    p, cu, L = oracle.pack_padded(x, m)
    np.testing.assert_array_equal(cu, [0, 2, 5])
    assert L == 3
    np.testing.assert_array_equal(p, [x[0, 0], x[0, 1], x[1, 0], x[1, 1], x[1, 2]])


def test_round_trip_and_empty_rows():
    rng = np.random.default_rng(0)
    B, L = 5, 9
    lens = [0, 9, 3, 1, 7]
    m = np.array([[1] * n + [0] * (L - n) for n in lens])
    x = rng.standard_normal((B, L, 2, 4))
    p, cu, mx = oracle.pack_padded(x, m)
    assert p.shape == (sum(lens), 2, 4) and mx == 9
    np.testing.assert_array_equal(np.diff(cu), lens)
    back = oracle.unpack_packed(p, cu, L, m)
    np.testing.assert_array_equal(back, x * m[:, :, None, None])


def test_packed_attention_matches_padded():
    rng = np.random.default_rng(1)
    B, L, H, D, span, buckets = 3, 24, 2, 8, 16, 8
    lens = [24, 10, 17]
    att, R = oracle.att_and_rows(span, buckets)
    m = np.array([[1] * n + [0] * (L - n) for n in lens], dtype=np.uint8)
    q, k, v = (rng.standard_normal((B, L, H, D)) for _ in range(3))
    q_r, k_r = rng.standard_normal((H, R, D)), rng.standard_normal((H, R, D))
    o_pad, _ = oracle.forward(q.reshape(B * L, H, D), k.reshape(B * L, H, D), v.reshape(B * L, H, D),
                              q_r, k_r, span, buckets, key_mask=m.reshape(-1), batch=B)
    (qp, cu, _), (kp, _, _), (vp, _, _) = (oracle.pack_padded(t, m) for t in (q, k, v))
    o_pk, _ = oracle.forward(qp, kp, vp, q_r, k_r, span, buckets, cu_seqlens=cu, batch=B)
    np.testing.assert_allclose(oracle.unpack_packed(o_pk, cu, L, m),
                               o_pad.reshape(B, L, H, D) * m[:, :, None, None], rtol=0, atol=1e-12)
