"""Pins for the oracle's attention dropout (DisentangledFlash 1.1.1 page,
"Status": dropout of the attention probabilities inside the fused kernels,
the mask recomputed from its counter in the backward).

* Philox4x32-10 against two known-answer vectors of the generator's reference
  implementation (Salmon et al., SC 2011; counter / key all zero, and the
  counter / key made of the hexadecimal digits of pi);
* p = 0 reduces exactly to the oracle without dropout;
* the kept fraction is 1 - p within a binomial bound, and the mask changes
  with the seed, the offset, the head and the sequence;
* the dropout backward matches central finite differences of the forward with
  the same (fixed) mask;
* averaged over many seeds, the dropout output approaches the undropped one
  (dropout is unbiased).
"""
import numpy as np
import pytest

import oracle
from oracle import philox
from synth import make_inputs


def test_philox_known_answers():
    assert [int(x) for x in philox.philox4x32_10(0, 0, 0, 0, 0, 0)] == [
        0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    assert [int(x) for x in philox.philox4x32_10(0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344,
                                                  0xA4093822, 0x299F31D0)] == [
        0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


def _small(L=20, H=2, D=4, span=8, buckets=4, seed=0, lengths=None, mask_frac=0.0):
    att, R = oracle.att_and_rows(span, buckets)
    if lengths is not None:
        return make_inputs(H, D, "fp32", span, buckets, R, seed, lengths=lengths, packed=True,
                           mask_frac=mask_frac)
    return make_inputs(H, D, "fp32", span, buckets, R, seed, batch=1, seqlen=L, mask_frac=mask_frac)


def _run(inp, dropout, backward=True):
    f, w = inp.f64, inp.workload
    kw = dict(key_mask=inp.key_mask, cu_seqlens=inp.cu_seqlens, batch=inp.nseq)
    o, l = oracle.forward(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], w.span, w.buckets,
                          dropout=dropout, **kw)
    if not backward:
        return o, l
    g = oracle.backward(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], f["dout"], w.span, w.buckets,
                        dropout=dropout, **kw)
    return (o, l) + tuple(g)


def test_p_zero_is_no_dropout():
    inp = _small(lengths=[11, 17], mask_frac=0.2, seed=2)
    a = _run(inp, None)
    b = _run(inp, (0.0, 1234, 7))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_keep_fraction_and_stream_separation():
    p, L, H = 0.3, 200, 3
    m = philox.keep_mask(p, 42, 0, 0, 1, H, L)
    n = m.size
    frac = m.mean()
    assert abs(frac - (1 - p)) <= 5 * np.sqrt(p * (1 - p) / n)
    # every 8-key block uses one call, two keys per output word: each key
    # position of the block, and the low and high half of a word, keeps 1 - p
    for pos in range(8):
        assert abs(m[:, pos::8].mean() - (1 - p)) <= 6 * np.sqrt(p * (1 - p) / (n / 8)), pos
    # the two keys of one word decide independently: P(both kept) = (1 - p)^2
    both = (m[:, 0:L - 1:2] & m[:, 1::2]).mean()
    assert abs(both - (1 - p) ** 2) <= 6 * np.sqrt((1 - p) ** 2 * (1 - (1 - p) ** 2) / (n / 2))
    for other in (philox.keep_mask(p, 43, 0, 0, 1, H, L), philox.keep_mask(p, 42, 1, 0, 1, H, L),
                  philox.keep_mask(p, 42, 0, 0, 2, H, L), philox.keep_mask(p, 42, 0, 1, 1, H, L)):
        agree = (other == m).mean()
        assert abs(agree - (p * p + (1 - p) * (1 - p))) <= 0.02
    assert philox.keep_mask(0.0, 42, 0, 0, 0, H, L).all()
    assert philox.keep_mask(p, 42, 0, 0, 0, H, 0).shape == (0, 0)  # empty sequence
    with pytest.raises(ValueError):
        philox.keep_threshold(1.0)


@pytest.mark.parametrize("case", ["packed_masked", "unbucketed"])
def test_dropout_backward_finite_differences(case):
    if case == "unbucketed":
        inp = _small(L=18, H=2, D=4, span=6, buckets=0, seed=3)
    else:
        inp = _small(H=2, D=4, span=12, buckets=8, seed=5, mask_frac=0.2, lengths=[13, 19])
    drop = (0.25, 99, 3)
    f = {k: v.copy() for k, v in inp.f64.items()}
    w = inp.workload
    W = f["dout"]

    def loss(ff):
        o, _ = oracle.forward(ff["q"], ff["k"], ff["v"], ff["q_r"], ff["k_r"], w.span, w.buckets,
                              key_mask=inp.key_mask, cu_seqlens=inp.cu_seqlens, batch=inp.nseq,
                              dropout=drop)
        return float((o * W).sum())

    grads = oracle.backward(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], W, w.span, w.buckets,
                            key_mask=inp.key_mask, cu_seqlens=inp.cu_seqlens, batch=inp.nseq,
                            dropout=drop)
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
        ana = g.ravel()[flat]
        assert np.linalg.norm(ana - num) <= 1e-6 * max(np.linalg.norm(num), 1e-30), name


def test_dropout_is_unbiased():
    inp = _small(L=16, H=1, D=4, span=6, buckets=4, seed=4)
    ref, _ = _run(inp, None, backward=False)
    acc = np.zeros_like(ref)
    acc2 = np.zeros_like(ref)
    n = 1500
    for s in range(n):
        o, _ = _run(inp, (0.2, s, 0), backward=False)
        acc += o
        acc2 += o * o
    mean = acc / n
    se = np.sqrt(np.maximum(acc2 / n - mean * mean, 0) / n)  # standard error per element
    # the mean is within 5 standard errors of the undropped output everywhere
    assert np.all(np.abs(mean - ref) <= 5 * se + 1e-12)
