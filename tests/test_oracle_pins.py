"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test names what it fixes: a closed form, an invariant, a library routine
(torch's scaled_dot_product_attention and autograd on the CPU in float64),
brute force on tiny inputs, high-precision evaluation of the bucket formula,
or central finite differences. A plausible slip in the oracle (a dropped
term, a swapped index, a wrong sign, a transposed operand) fails at least one.
"""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle
from synth import make_inputs, WORKLOADS

getcontext().prec = 80


# ----------------------------------------------------------------------------
# an independent, high-precision evaluation of the log bucket

def bucket_decimal(d, span, buckets):
    """The v2/v3 log bucket evaluated with 80-digit decimals (independent of
    the oracle's integer comparison). A ceiling argument within 1e-60 of an
    integer is treated as that integer."""
    if buckets <= 0:
        return d
    mid = buckets // 2
    a = abs(d)
    if a <= mid:
        return d
    x = (Decimal(mid - 1) * (Decimal(a) / Decimal(mid)).ln()
         / (Decimal(span - 1) / Decimal(mid)).ln())
    n = x.to_integral_value()
    k = int(n) if abs(x - n) < Decimal("1e-60") else math.ceil(x)
    return int(math.copysign(mid + k, d))


PARAMS = [(512, 256), (32, 0), (512, 0), (12, 8), (81, 10), (300, 256), (8192, 32)]


@pytest.mark.parametrize("span,buckets", PARAMS)
def test_p9_bucket_exact_vs_decimal(span, buckets):
    lim = 8192 if (span, buckets) in ((512, 256), (512, 0), (32, 0)) else 3000
    for d in range(-lim + 1, lim):
        assert oracle.bucket_exact(d, span, buckets) == bucket_decimal(d, span, buckets), d


def test_p9_bucket_properties_metric_config():
    span, buckets = 512, 256
    c2p, p2c = oracle.rel_luts(8192, span, buckets)
    o = 8191
    b = [oracle.bucket_exact(d, span, buckets) for d in range(-8191, 8192)]
    # odd
    assert all(b[o + d] == -b[o - d] for d in range(8192))
    # identity up to mid
    assert all(b[o + d] == d for d in range(-128, 129))
    # monotone non-decreasing, with no skipped values (slope < 1 at mid)
    assert all(0 <= b[n + 1] - b[n] <= 1 for n in range(len(b) - 1))
    # exact tie at |d| = span - 1: (mid-1) ln((span-1)/mid) / ln((span-1)/mid) = 127
    assert oracle.bucket_exact(511, span, buckets) == 255
    assert oracle.bucket_exact(-511, span, buckets) == -255
    assert oracle.bucket_exact(510, span, buckets) == 255
    assert oracle.bucket_exact(512, span, buckets) == 256
    # saturation: row R-1 = 511 from d = 506, row 0 from d = -512
    assert c2p[o + 505] == 510 and all(c2p[o + d] == 511 for d in range(506, 8192))
    assert c2p[o - 511] == 1 and all(c2p[o - d] == 0 for d in range(512, 8192))
    # p2c is c2p mirrored in d (delta(j,i) with j - i = -(i - j))
    assert np.array_equal(p2c, c2p[::-1])
    # every row is reached at L = 8192, row 0 unreached at L = 512
    assert len(set(c2p.tolist())) == 512
    c512, _ = oracle.rel_luts(512, span, buckets)
    assert len(set(c512.tolist())) == 511 and 0 not in set(c512.tolist())


def test_p9_unbucketed_closed_form():
    # span 32, no buckets: delta(i, j) = clamp(i - j + 32, 0, 63)
    c2p, p2c = oracle.rel_luts(64, 32, 0)
    d = np.arange(-63, 64)
    assert np.array_equal(c2p, np.clip(d + 32, 0, 63))
    assert np.array_equal(p2c, np.clip(-d + 32, 0, 63))


def test_p9_tie_small_params():
    # span 81, buckets 10: (80/5) = 2^4 and mid - 1 = 4, so |d| = 10, 20, 40, 80
    # give exact integer ceiling arguments 1, 2, 3, 4
    for a, k in ((10, 1), (20, 2), (40, 3), (80, 4)):
        assert oracle.bucket_exact(a, 81, 10) == 5 + k
        assert oracle.bucket_exact(a + 1, 81, 10) == 5 + k + 1


# ----------------------------------------------------------------------------
# helpers

def _small(L=20, H=2, D=8, span=12, buckets=8, seed=7, mask_frac=0.0, lengths=None):
    att, R = oracle.att_and_rows(span, buckets)
    if lengths is not None:
        return make_inputs(H, D, "fp32", span, buckets, R, seed, lengths=lengths,
                           packed=True, mask_frac=mask_frac, std="unit")
    return make_inputs(H, D, "fp32", span, buckets, R, seed, batch=1, seqlen=L,
                       mask_frac=mask_frac, std="unit")


def _run_fwd(inp, **kw):
    f = inp.f64
    w = inp.workload
    return oracle.forward(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], w.span,
                          w.buckets, key_mask=inp.key_mask,
                          cu_seqlens=inp.cu_seqlens, batch=inp.nseq, **kw)


def _run_bwd(inp, **kw):
    f = inp.f64
    w = inp.workload
    return oracle.backward(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], f["dout"],
                           w.span, w.buckets, key_mask=inp.key_mask,
                           cu_seqlens=inp.cu_seqlens, batch=inp.nseq, **kw)


# ----------------------------------------------------------------------------
# P1: reduction to plain attention (library routine)

@pytest.mark.parametrize("mask_frac", [0.0, 0.25])
def test_p1_zero_relative_is_sdpa(mask_frac):
    inp = _small(L=24, H=3, D=8, mask_frac=mask_frac)
    f = inp.f64
    zr = np.zeros_like(f["q_r"])
    w = inp.workload
    out, lse = oracle.forward(f["q"], f["k"], f["v"], zr, zr, w.span, w.buckets,
                              key_mask=inp.key_mask)
    D = f["q"].shape[2]
    s = 1.0 / math.sqrt(3 * D)
    q = torch.tensor(f["q"]).permute(1, 0, 2)[None].requires_grad_()
    k = torch.tensor(f["k"]).permute(1, 0, 2)[None].requires_grad_()
    v = torch.tensor(f["v"]).permute(1, 0, 2)[None].requires_grad_()
    valid = np.ones(24, bool) if inp.key_mask is None else inp.key_mask.astype(bool)
    am = torch.tensor(np.broadcast_to(valid[None, :], (24, 24)).copy())
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=am, scale=s)
    ref_o = ref[0].permute(1, 0, 2).detach().numpy()
    rows = np.nonzero(valid)[0]
    assert np.abs(out[rows] - ref_o[rows]).max() < 1e-12
    assert np.all(out[~valid] == 0) and np.all(np.isneginf(lse[:, ~valid]))
    # textbook log-sum-exp with the masked keys removed
    for h in range(3):
        Sx = s * f["q"][:, h] @ f["k"][:, h].T
        for i in rows:
            row = Sx[i, valid]
            assert abs(lse[h, i] - (row.max() + math.log(np.exp(row - row.max()).sum()))) < 1e-12
    # backward against torch autograd (loss only over valid rows)
    dout = f["dout"].copy()
    dout[~valid] = 0.0
    (ref[0].permute(1, 0, 2)[torch.tensor(rows)] * torch.tensor(dout[rows])).sum().backward()
    dq, dk, dv, _, _ = oracle.backward(f["q"], f["k"], f["v"], zr, zr, dout, w.span,
                                       w.buckets, key_mask=inp.key_mask)
    for mine, t in ((dq, q), (dk, k), (dv, v)):
        g = t.grad[0].permute(1, 0, 2).numpy()
        assert np.abs(mine - g).max() < 1e-12


# ----------------------------------------------------------------------------
# P2: brute force per element

def _brute(Q, K, V, Qr, Kr, span, buckets):
    L, D = len(Q), len(Q[0])
    att, R = oracle.att_and_rows(span, buckets)
    s = 1.0 / math.sqrt(3 * D)

    def dl(a, b):
        return min(max(bucket_decimal(a - b, span, buckets) + att, 0), R - 1)

    S = [[0.0] * L for _ in range(L)]
    for i in range(L):
        for j in range(L):
            acc = 0.0
            ci, pj = dl(i, j), dl(j, i)
            for d in range(D):
                acc += Q[i][d] * K[j][d] + Q[i][d] * Kr[ci][d] + K[j][d] * Qr[pj][d]
            S[i][j] = s * acc
    O = [[0.0] * D for _ in range(L)]
    lse = [0.0] * L
    for i in range(L):
        m = max(S[i])
        z = sum(math.exp(x - m) for x in S[i])
        lse[i] = m + math.log(z)
        for j in range(L):
            p = math.exp(S[i][j] - lse[i])
            for d in range(D):
                O[i][d] += p * V[j][d]
    return np.array(S), np.array(O), np.array(lse)


@pytest.mark.parametrize("span,buckets,L", [(6, 0, 14), (12, 8, 16), (81, 10, 16)])
def test_p2_brute_force(span, buckets, L):
    inp = _small(L=L, H=2, D=4, span=span, buckets=buckets, seed=11)
    f = inp.f64
    out, lse = _run_fwd(inp)
    for h in range(2):
        args = [f[n][:, h].tolist() for n in ("q", "k", "v")] + [f[n][h].tolist() for n in ("q_r", "k_r")]
        S, O, l = _brute(*args, span, buckets)
        S2 = oracle.scores(f["q"][:, h], f["k"][:, h], f["q_r"][h], f["k_r"][h], span, buckets)
        assert np.abs(S - S2).max() < 1e-12
        assert np.abs(O - out[:, h]).max() < 1e-12
        assert np.abs(l - lse[h]).max() < 1e-12


# ----------------------------------------------------------------------------
# P3: normalisation

def test_p3_rows_sum_to_one():
    inp = _small(L=30, H=2, D=8, mask_frac=0.2, lengths=[30, 17])
    out, lse, probs = _run_fwd(inp, return_probs=True)
    for (n, h), P in probs.items():
        st, en = oracle.sequences(inp.total_tokens, inp.cu_seqlens)[n]
        valid = inp.key_mask[st:en].astype(bool)
        assert np.abs(P[valid].sum(axis=1) - 1).max() < 1e-12
        assert np.all(P[~valid] == 0) and np.all(P[:, ~valid] == 0)
        f = inp.f64
        S = oracle.scores(f["q"][st:en, h], f["k"][st:en, h], f["q_r"][h], f["k_r"][h],
                          inp.workload.span, inp.workload.buckets)
        for i in np.nonzero(valid)[0]:
            mx = S[i, valid].max()
            assert mx - 1e-12 <= lse[h, st + i] <= mx + math.log(valid.sum()) + 1e-12


# ----------------------------------------------------------------------------
# P4: backward vs central finite differences

@pytest.mark.parametrize("case", ["bucketed_packed_masked", "unbucketed"])
def test_p4_finite_differences(case):
    if case == "unbucketed":
        inp = _small(L=18, H=2, D=4, span=6, buckets=0, seed=3)
    else:
        inp = _small(H=2, D=4, span=12, buckets=8, seed=5, mask_frac=0.2, lengths=[13, 19])
    f = {k: v.copy() for k, v in inp.f64.items()}
    w = inp.workload
    W = f["dout"]

    def loss(ff):
        o, _ = oracle.forward(ff["q"], ff["k"], ff["v"], ff["q_r"], ff["k_r"], w.span,
                              w.buckets, key_mask=inp.key_mask, cu_seqlens=inp.cu_seqlens,
                              batch=inp.nseq)
        return float((o * W).sum())

    grads = oracle.backward(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], W, w.span, w.buckets,
                            key_mask=inp.key_mask, cu_seqlens=inp.cu_seqlens, batch=inp.nseq)
    rng = np.random.default_rng(0)
    eps = 1e-6
    for name, g in zip(("q", "k", "v", "q_r", "k_r"), grads):
        x = f[name]
        flat = rng.choice(x.size, size=min(60, x.size), replace=False)
        num = np.zeros(len(flat))
        for n, e in enumerate(flat):
            idx = np.unravel_index(e, x.shape)
            old = x[idx]
            x[idx] = old + eps
            lp = loss(f)
            x[idx] = old - eps
            lm = loss(f)
            x[idx] = old
            num[n] = (lp - lm) / (2 * eps)
        ana = g.ravel()[flat]
        assert np.linalg.norm(ana - num) <= 1e-6 * max(np.linalg.norm(num), 1e-30), name


# ----------------------------------------------------------------------------
# P5: zero-sum structure of the relative gradients

def test_p5_zero_sums():
    inp = _small(H=2, D=8, span=12, buckets=8, seed=9, mask_frac=0.2, lengths=[25, 14])
    dq, dk, dv, dq_r, dk_r, strips = _run_bwd(inp, return_strips=True)
    # every valid row of dS sums to zero, hence so do the rows of dC2P and the
    # r-sum of dK_r; the columns of dS do not, so dQ_r's r-sum is not zero
    assert np.abs(dk_r.sum(axis=1)).max() <= 1e-10 * np.abs(dk_r).max()
    assert np.abs(dq_r.sum(axis=1)).max() > 1e-3 * np.abs(dq_r).max()
    for (dC2P, dP2C) in strips.values():
        assert np.abs(dC2P.sum(axis=1)).max() <= 1e-12
        assert np.abs(dC2P).max() > 0 and np.abs(dP2C).max() > 0


def test_p5_dv_column_sum():
    # dV = P^T dO and every row of P with a valid query sums to one (rows of
    # masked queries are zero), so per sequence and head the dV rows add up
    # to the dO rows of the valid queries
    inp = _small(H=2, D=8, span=12, buckets=8, seed=11, mask_frac=0.2, lengths=[25, 14, 9])
    dv = _run_bwd(inp)[2]
    dout = inp.f64["dout"]
    valid = inp.key_mask.astype(bool)
    for b in range(inp.nseq):
        st, en = int(inp.cu_seqlens[b]), int(inp.cu_seqlens[b + 1])
        want = dout[st:en][valid[st:en]].sum(axis=0)
        np.testing.assert_allclose(dv[st:en].sum(axis=0), want, rtol=0, atol=1e-12 * (1 + np.abs(want).max()))
    # a key-masked row receives nothing
    assert np.abs(dv[~valid]).max() == 0.0


# ----------------------------------------------------------------------------
# P6: transposition identity of the literal delta(j, i) reading

@pytest.mark.parametrize("span,buckets", [(12, 8), (6, 0)])
def test_p6_transpose_identity(span, buckets):
    inp = _small(L=22, H=1, D=6, span=span, buckets=buckets, seed=13)
    f = inp.f64
    S = oracle.scores(f["q"][:, 0], f["k"][:, 0], f["q_r"][0], f["k_r"][0], span, buckets)
    St = oracle.scores(f["k"][:, 0], f["q"][:, 0], f["k_r"][0], f["q_r"][0], span, buckets)
    assert np.abs(S.T - St).max() < 1e-13
    # and the relative terms really are present
    zr = np.zeros_like(f["q_r"][0])
    S0 = oracle.scores(f["q"][:, 0], f["k"][:, 0], zr, zr, span, buckets)
    assert np.abs(S - S0).max() > 1e-2


# ----------------------------------------------------------------------------
# P7: C2P shift invariance (a per-row constant leaves softmax unchanged)

def test_p7_kr_shift_invariance():
    inp = _small(L=26, H=2, D=6, seed=17)
    f = inp.f64
    w = inp.workload
    out, _ = _run_fwd(inp)
    c = np.random.default_rng(1).standard_normal((2, 1, 6))
    out2, _ = oracle.forward(f["q"], f["k"], f["v"], f["q_r"], f["k_r"] + c, w.span, w.buckets)
    assert np.abs(out - out2).max() < 1e-13
    # the same shift of Q_r is a per-column term and does change the output
    out3, _ = oracle.forward(f["q"], f["k"], f["v"], f["q_r"] + c, f["k_r"], w.span, w.buckets)
    assert np.abs(out - out3).max() > 1e-3


# ----------------------------------------------------------------------------
# P8: mask semantics and packing

def test_p8_right_padding_is_truncation_and_packing():
    L, n_valid = 24, 17
    inp = _small(L=L, H=2, D=6, seed=19)
    f = inp.f64
    w = inp.workload
    mask = np.zeros(L, np.uint8)
    mask[:n_valid] = 1
    out, lse = oracle.forward(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], w.span, w.buckets,
                              key_mask=mask)
    sl = slice(0, n_valid)
    out_t, lse_t = oracle.forward(f["q"][sl], f["k"][sl], f["v"][sl], f["q_r"], f["k_r"],
                                  w.span, w.buckets)
    assert np.abs(out[sl] - out_t).max() < 1e-13 and np.abs(lse[:, sl] - lse_t).max() < 1e-13
    assert np.all(out[n_valid:] == 0)
    dq, dk, dv, dq_r, dk_r = oracle.backward(f["q"], f["k"], f["v"], f["q_r"], f["k_r"],
                                             f["dout"], w.span, w.buckets, key_mask=mask)
    g_t = oracle.backward(f["q"][sl], f["k"][sl], f["v"][sl], f["q_r"], f["k_r"],
                          f["dout"][sl], w.span, w.buckets)
    for a, b in zip((dq[sl], dk[sl], dv[sl], dq_r, dk_r), g_t):
        assert np.abs(a - b).max() < 1e-13
    assert np.all(dq[n_valid:] == 0) and np.all(dk[n_valid:] == 0) and np.all(dv[n_valid:] == 0)
    # packed = per-sequence runs concatenated
    pk = _small(H=2, D=6, seed=23, lengths=[9, 15, 4])
    pf = pk.f64
    out_p, lse_p = _run_fwd(pk)
    gp = _run_bwd(pk)
    acc = [np.zeros_like(pf["q_r"]), np.zeros_like(pf["k_r"])]
    for (st, en) in oracle.sequences(pk.total_tokens, pk.cu_seqlens):
        sl = slice(st, en)
        o1, l1 = oracle.forward(pf["q"][sl], pf["k"][sl], pf["v"][sl], pf["q_r"], pf["k_r"],
                                12, 8)
        assert np.abs(out_p[sl] - o1).max() < 1e-13 and np.abs(lse_p[:, sl] - l1).max() < 1e-13
        g1 = oracle.backward(pf["q"][sl], pf["k"][sl], pf["v"][sl], pf["q_r"], pf["k_r"],
                             pf["dout"][sl], 12, 8)
        for a, b in zip(gp[:3], g1[:3]):
            assert np.abs(a[sl] - b).max() < 1e-13
        acc[0] += g1[3]
        acc[1] += g1[4]
    assert np.abs(gp[3] - acc[0]).max() < 1e-13 and np.abs(gp[4] - acc[1]).max() < 1e-13


# ----------------------------------------------------------------------------
# P10: the unbucketed far field uses the end rows (closed form)

def test_p10_far_field_end_rows():
    span, L, D = 8, 40, 5
    att, R = oracle.att_and_rows(span, 0)
    rng = np.random.default_rng(29)
    Q = rng.standard_normal((L, D))
    Kr = rng.standard_normal((R, D))
    Qr = rng.standard_normal((R, D))
    K = np.zeros((L, D))          # isolates the C2P term: S = s Q_i . K_r[delta(i,j)]
    S = oracle.scores(Q, K, Qr, Kr, span, 0)
    s = 1 / math.sqrt(3 * D)
    for i in range(L):
        for j in range(L):
            if i - j >= span:
                assert abs(S[i, j] - s * Q[i] @ Kr[R - 1]) < 1e-13
            elif j - i >= span:
                assert abs(S[i, j] - s * Q[i] @ Kr[0]) < 1e-13
            else:
                assert abs(S[i, j] - s * Q[i] @ Kr[i - j + att]) < 1e-13
    # fraction of pairs on the end rows for the long unbucketed workload:
    # pairs with |i - j| >= 512 over L^2 at L = 8192
    Lb = 8192
    far = sum(2 * (Lb - d) for d in range(512, Lb))
    assert abs(far / Lb ** 2 - 0.879) < 5e-4


# ----------------------------------------------------------------------------
# row-sampled helpers agree with the full evaluation

def test_row_sampling_helpers():
    inp = _small(H=2, D=6, seed=31, mask_frac=0.2, lengths=[21, 30])
    f = inp.f64
    w = inp.workload
    out, lse = _run_fwd(inp)
    dq, *_ = _run_bwd(inp)
    seqs = oracle.sequences(inp.total_tokens, inp.cu_seqlens)
    rows = np.array([0, 3, 7, 20, 29])
    o, l = oracle.forward_rows(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], w.span, w.buckets,
                               seqs[1], 1, rows, key_mask=inp.key_mask)
    st = seqs[1][0]
    assert np.abs(o - out[st + rows, 1]).max() < 1e-13
    ref_l = lse[1, st + rows]
    fin = np.isfinite(ref_l)
    assert (~fin).any() and fin.any()  # the sample holds masked and valid rows
    assert np.array_equal(np.isneginf(l), ~fin)
    assert np.abs(l[fin] - ref_l[fin]).max() < 1e-13
    g = oracle.dq_rows(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], f["dout"], w.span, w.buckets,
                       seqs[1], 1, rows, key_mask=inp.key_mask)
    assert np.abs(g - dq[st + rows, 1]).max() < 1e-13


def test_workload_recipes():
    import synth
    rng = np.random.default_rng(WORKLOADS[4].seed)
    lens = synth.packed_lengths(rng, 16384, 64, 2048)
    assert sum(lens) == 16384 and all(n <= 2048 for n in lens[:-1]) and all(n >= 64 for n in lens[:-1])
    assert WORKLOADS[3].batch * WORKLOADS[3].seqlen == 16384


# ----------------------------------------------------------------------------
# P11: the shared P2C convention (the row C2P uses, as deployed DeBERTa code
# indexes P2C in self-attention), pinned like the literal one: per-element
# loops, finite differences, and the reflection that links the two index
# functions where no clamp is reached.

def _brute_shared_scores(Q, K, Qr, Kr, span, buckets):
    L, D = len(Q), len(Q[0])
    att, R = oracle.att_and_rows(span, buckets)
    s = 1.0 / math.sqrt(3 * D)

    def dl(a, b):
        return min(max(bucket_decimal(a - b, span, buckets) + att, 0), R - 1)

    S = np.zeros((L, L))
    for i in range(L):
        for j in range(L):
            c = dl(i, j)   # both terms use delta(i, j)
            S[i, j] = s * sum(Q[i][d] * K[j][d] + Q[i][d] * Kr[c][d] + K[j][d] * Qr[c][d] for d in range(D))
    return S


@pytest.mark.parametrize("span,buckets,L", [(6, 0, 14), (12, 8, 16), (81, 10, 16)])
def test_p11_shared_brute_force(span, buckets, L):
    inp = _small(L=L, H=1, D=4, span=span, buckets=buckets, seed=21)
    f = inp.f64
    args = [f["q"][:, 0].tolist(), f["k"][:, 0].tolist(), f["q_r"][0].tolist(), f["k_r"][0].tolist()]
    S = _brute_shared_scores(*args, span, buckets)
    S2 = oracle.scores(f["q"][:, 0], f["k"][:, 0], f["q_r"][0], f["k_r"][0], span, buckets, "shared")
    assert np.abs(S - S2).max() < 1e-12
    S3 = oracle.scores(f["q"][:, 0], f["k"][:, 0], f["q_r"][0], f["k_r"][0], span, buckets, "literal")
    assert np.abs(S - S3).max() > 1e-3   # the conventions differ


def test_p11_shared_reflection():
    """Unbucketed, L <= span: no clamp is reached, the literal row is
    att - d and the shared row att + d = R - (att - d); so the shared scores
    with Q_r equal the literal scores with Q_r'[r] = Q_r[R - r]."""
    span, L, D = 20, 16, 4
    att, R = oracle.att_and_rows(span, 0)
    rng = np.random.default_rng(4)
    Q, K = rng.standard_normal((L, D)), rng.standard_normal((L, D))
    Qr, Kr = rng.standard_normal((R, D)), rng.standard_normal((R, D))
    Qr2 = np.zeros_like(Qr)
    Qr2[1:] = Qr[R - np.arange(1, R)]
    S_sh = oracle.scores(Q, K, Qr, Kr, span, 0, "shared")
    S_li = oracle.scores(Q, K, Qr2, Kr, span, 0, "literal")
    assert np.abs(S_sh - S_li).max() < 1e-13


def test_p11_shared_finite_differences():
    inp = _small(H=2, D=4, span=12, buckets=8, seed=6, mask_frac=0.2, lengths=[13, 19])
    f = {k: v.copy() for k, v in inp.f64.items()}
    w = inp.workload
    W = f["dout"]
    kw = dict(key_mask=inp.key_mask, cu_seqlens=inp.cu_seqlens, batch=inp.nseq, p2c="shared")

    def loss(ff):
        o, _ = oracle.forward(ff["q"], ff["k"], ff["v"], ff["q_r"], ff["k_r"], w.span, w.buckets, **kw)
        return float((o * W).sum())

    grads = oracle.backward(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], W, w.span, w.buckets, **kw)
    rng = np.random.default_rng(1)
    eps = 1e-6
    for name, g in zip(("q", "k", "v", "q_r", "k_r"), grads):
        x = f[name]
        flat = rng.choice(x.size, size=min(40, x.size), replace=False)
        num = np.zeros(len(flat))
        for n, e in enumerate(flat):
            idx = np.unravel_index(e, x.shape)
            old = x[idx]
            x[idx] = old + eps
            lp = loss(f)
            x[idx] = old - eps
            lm = loss(f)
            x[idx] = old
            num[n] = (lp - lm) / (2 * eps)
        assert np.linalg.norm(g.ravel()[flat] - num) <= 1e-6 * max(np.linalg.norm(num), 1e-30), name
