"""GPU parity of the HIP path against the float64 oracle (through the C ABI).

Sizes are chosen so that the oracle finishes in seconds while the kernels see
several query/key tiles, ragged tails, band and far-field tiles, empty and
masked sequences, every head dim and every dtype.
Tolerances (rel-L2 per tensor): bf16/fp16 forward 1e-2, gradients 2e-2;
fp32 1e-5. Relative-index tables must match bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import make_inputs, workload_inputs
from parity_util import run_gpu, run_oracle, compare, rel_l2

pytestmark = pytest.mark.gpu


def _inp(L=300, B=1, H=2, D=64, dtype="bf16", span=64, buckets=32, seed=0, lengths=None,
         mask_frac=0.0):
    att, R = oracle.att_and_rows(span, buckets)
    if lengths is not None:
        return make_inputs(H, D, dtype, span, buckets, R, seed, lengths=lengths, packed=True,
                           mask_frac=mask_frac)
    return make_inputs(H, D, dtype, span, buckets, R, seed, batch=B, seqlen=L, mask_frac=mask_frac)


# ----------------------------------------------------------------------------
# relative index tables: bit-exact

@pytest.mark.parametrize("L,span,buckets", [
    (64, 32, 0), (512, 512, 256), (8192, 512, 256), (8192, 512, 0), (2048, 512, 256),
    (300, 12, 8), (3000, 81, 10), (3000, 300, 256), (5000, 8192, 32), (40, 6, 0), (1, 4, 2),
])
def test_rel_index_bit_exact(L, span, buckets):
    import deberta_disentangled_attention_rel_amd as df
    print(f"rel index L={L} span={span} buckets={buckets}", flush=True)
    c2p, p2c = df.build_rel_index(L, span, buckets)
    torch.cuda.synchronize()
    rc, rp = oracle.rel_luts(L, span, buckets)
    assert np.array_equal(c2p.cpu().numpy(), rc)
    assert np.array_equal(p2c.cpu().numpy(), rp)


# ----------------------------------------------------------------------------
# forward + backward parity, small shapes

CASES = {
    # name: kwargs for _inp
    "tiny_fp32_L64": dict(L=64, H=2, D=32, dtype="fp32", span=32, buckets=0, seed=1001),
    "bf16_D64_bucketed_ragged": dict(L=300, B=2, H=2, D=64, span=64, buckets=32, seed=1),
    "bf16_D64_unbucketed_far": dict(L=520, H=2, D=64, span=48, buckets=0, seed=2),
    "bf16_D32": dict(L=200, H=3, D=32, span=40, buckets=16, seed=3),
    "bf16_D128": dict(L=260, H=2, D=128, span=64, buckets=32, seed=4),
    "fp16_D128_unbucketed": dict(L=333, H=2, D=128, dtype="fp16", span=64, buckets=0, seed=5),
    "fp16_D64": dict(L=130, H=2, D=64, dtype="fp16", span=20, buckets=8, seed=6),
    "fp32_D64": dict(L=190, H=2, D=64, dtype="fp32", span=64, buckets=32, seed=7),
    "fp32_D128": dict(L=150, H=1, D=128, dtype="fp32", span=40, buckets=0, seed=8),
    "bf16_packed_masked": dict(lengths=[100, 1, 257, 64, 0, 190], H=2, D=64, span=64, buckets=32,
                               seed=9, mask_frac=0.1),
    "fp16_packed_masked_D128": dict(lengths=[33, 300, 129], H=2, D=128, dtype="fp16", span=40,
                                    buckets=16, seed=10, mask_frac=0.25),
    "bf16_big_bucket_odd": dict(L=400, H=2, D=64, span=300, buckets=256, seed=11),
    "bf16_metric_index_L1024": dict(L=1024, H=1, D=64, span=512, buckets=256, seed=12),
    # tables that skip rows (mid - 1 > mid ln((span-1)/mid)): the general
    # kernel instantiations, which gather both relative terms from global
    # memory and walk with skipped rows, in other dtypes and head dims
    "fp32_D128_wide_bucket": dict(L=260, H=1, D=128, dtype="fp32", span=100, buckets=128, seed=13),
    "fp16_D32_wide_bucket": dict(L=180, H=2, D=32, dtype="fp16", span=100, buckets=128, seed=14),
    "bf16_D128_wide_bucket_masked": dict(lengths=[170, 41, 96], H=2, D=128, span=100, buckets=128, seed=15,
                                         mask_frac=0.2),
    # the tile ranges (far / band / far) at their edges: span beyond the
    # sequence (every tile a band tile, no far range), one row in the last
    # query block with 32-key tiles, and packed lengths on both sides of the
    # 32-, 64- and 128-row tile edges
    "bf16_all_band_span_gt_L": dict(L=200, H=2, D=64, span=256, buckets=128, seed=16),
    "fp16_D128_L129_far": dict(L=129, H=2, D=128, dtype="fp16", span=16, buckets=8, seed=17),
    "bf16_D128_packed_tile_edges": dict(lengths=[32, 33, 31, 64, 65, 128, 1, 127], H=2, D=128, span=24,
                                        buckets=8, seed=18, mask_frac=0.1),
}


@pytest.mark.parametrize("name", list(CASES))
def test_parity_small(name):
    kw = CASES[name]
    print(f"parity case {name}: {kw}", flush=True)
    inp = _inp(**kw)
    gpu = run_gpu(inp)
    ref = run_oracle(inp)
    errs, bad = compare(inp, gpu, ref)
    print(name, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert not bad, f"{name}: {bad}"


# the shared P2C convention (P2C takes the row C2P uses): the kernels run on
# a reversed q_r with a reversed-coordinate table; the oracle indexes directly
@pytest.mark.parametrize("name", ["bf16_D64_bucketed_ragged", "fp32_D64", "bf16_packed_masked",
                                  "fp16_D128_unbucketed", "bf16_big_bucket_odd", "bf16_metric_index_L1024"])
def test_parity_shared_p2c(name):
    kw = CASES[name]
    print(f"shared p2c case {name}: {kw}", flush=True)
    inp = _inp(**kw)
    gpu = run_gpu(inp, p2c="shared")
    ref = run_oracle(inp, p2c="shared")
    errs, bad = compare(inp, gpu, ref)
    print(name, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert not bad, f"{name}: {bad}"
    # the two conventions differ most in dk and dq_r (rel-L2 ~1 between the
    # oracle's two results on these inputs): the GPU must be far from the
    # literal ones
    lit = run_oracle(inp)
    for n in ("dk", "dq_r"):
        assert rel_l2(gpu[n], lit[n]) > 0.2, n


@pytest.mark.parametrize("name,p2c", [("bf16_D64_bucketed_ragged", "literal"), ("fp32_D64", "literal"),
                                      ("bf16_packed_masked", "shared")])
def test_bwd_reuses_forward_workspace(name, p2c):
    """DF_FLAG_BWD_REUSE_FWD: the backward on the forward's workspace (its
    index tables and strips kept) equals the recomputing backward bit for bit."""
    import deberta_disentangled_attention_rel_amd as df
    from parity_util import to_dev
    print(f"bwd reuse {name} {p2c}", flush=True)
    inp = _inp(**CASES[name])
    w = inp.workload
    t, km, cu = to_dev(inp)
    kw = dict(key_mask=km, cu_seqlens=cu, max_seqlen=inp.max_seqlen, p2c=p2c)
    args = (t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets)
    shape = df.make_shape(t["q"].view(-1, *t["q"].shape[-2:]), inp.nseq, inp.max_seqlen, p2c)
    ws = torch.empty(df.workspace_size(1, shape, w.span, w.buckets), dtype=torch.uint8, device="cuda")
    out, lse = df.fwd(*args, workspace=ws, **kw)
    g_reuse = df.bwd(*args, out, lse, t["dout"], workspace=ws, reuse_fwd_workspace=True, **kw)
    g_fresh = df.bwd(*args, out, lse, t["dout"], **kw)
    torch.cuda.synchronize()
    for n_, a, b in zip(("dq", "dk", "dv", "dq_r", "dk_r"), g_reuse, g_fresh):
        assert torch.equal(a, b), n_


def test_workload1_forward():
    inp = workload_inputs(1)
    gpu = run_gpu(inp, backward=False)
    ref = run_oracle(inp, backward=False)
    errs, bad = compare(inp, gpu, ref, backward=False)
    print("workload1", errs, flush=True)
    assert not bad, bad


def test_backward_deterministic():
    inp = _inp(L=700, H=2, D=64, dtype="fp16", span=64, buckets=0, seed=21)
    a = run_gpu(inp)
    b = run_gpu(inp)
    for n in ("out", "lse", "dq", "dk", "dv", "dq_r", "dk_r"):
        assert np.array_equal(a[n].view(np.uint32), b[n].view(np.uint32)), n


# ----------------------------------------------------------------------------
# inference forward: the training forward's output without LSE

@pytest.mark.parametrize("name", ["bf16_D64_bucketed_ragged", "fp16_D128_unbucketed", "fp32_D64",
                                  "bf16_packed_masked"])
def test_inference_forward(name):
    import deberta_disentangled_attention_rel_amd as df
    from parity_util import to_dev, rel_l2, TOL
    print(f"inference forward {name}", flush=True)
    inp = _inp(**CASES[name])
    w = inp.workload
    t, km, cu = to_dev(inp)
    kw = dict(key_mask=km, cu_seqlens=cu, max_seqlen=inp.max_seqlen)
    out_t, _ = df.fwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets, **kw)
    out_i = df.fwd_inference(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets, **kw)
    torch.cuda.synchronize()
    # the same kernel: bit-identical to the training forward's output
    assert torch.equal(out_i, out_t)
    ref = run_oracle(inp, backward=False)
    err = rel_l2(out_i.float().cpu().numpy(), ref["out"])
    assert np.isfinite(err) and err <= TOL[inp.dtype][0], err


# ----------------------------------------------------------------------------
# attention-probability dropout: the kernels regenerate the oracle's Philox
# mask (both sides implement the generator from its definition)

DROP_CASES = {
    "bf16_D64_bucketed_ragged": (0.1, 1234, 5),
    "fp32_D64": (0.3, 0xDEADBEEF12345, 0),
    "bf16_packed_masked": (0.2, 77, 9),
    "fp16_D128_unbucketed": (0.15, 3, 1),
    "tiny_fp32_L64": (0.5, 1, 2),
    "bf16_big_bucket_odd": (0.25, 99, 4),      # tables that skip rows
    "fp32_D128_wide_bucket": (0.1, 5, 0),
    # the 16-bit D=128 kernels run 32-key tiles: packed and masked, narrow
    # and row-skipping tables
    "fp16_packed_masked_D128": (0.2, 4321, 3),
    "bf16_D128_wide_bucket_masked": (0.1, 8, 6),
}


@pytest.mark.parametrize("name", list(DROP_CASES))
def test_dropout_parity(name):
    import deberta_disentangled_attention_rel_amd as df
    from parity_util import to_dev, rel_l2, TOL
    print(f"dropout {name}", flush=True)
    p, seed, offset = DROP_CASES[name]
    inp = _inp(**CASES[name])
    w = inp.workload
    t, km, cu = to_dev(inp)
    kw = dict(key_mask=km, cu_seqlens=cu, max_seqlen=inp.max_seqlen)
    dkw = dict(dropout_p=p, seed=seed, offset=offset)
    out, lse = df.fwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets, **kw, **dkw)
    g = df.bwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets, out, lse, t["dout"], **kw, **dkw)
    torch.cuda.synchronize()
    f = inp.f64
    okw = dict(key_mask=inp.key_mask, cu_seqlens=inp.cu_seqlens, batch=inp.nseq, dropout=(p, seed, offset))
    ref_o, ref_l = oracle.forward(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], w.span, w.buckets, **okw)
    ref_g = oracle.backward(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], f["dout"], w.span, w.buckets, **okw)
    tol_f, tol_b = TOL[inp.dtype]
    errs = {"out": rel_l2(out.float().cpu().numpy(), ref_o)}
    valid = np.isfinite(ref_l)
    errs["lse"] = rel_l2(lse.cpu().numpy()[valid], ref_l[valid])
    for n_, a, b in zip(("dq", "dk", "dv", "dq_r", "dk_r"), g, ref_g):
        errs[n_] = rel_l2(a.float().cpu().numpy(), b)
    bad = {n_: e for n_, e in errs.items()
           if not np.isfinite(e) or e > (tol_f if n_ in ("out", "lse") else tol_b)}
    assert not bad, (errs, bad)


@pytest.mark.parametrize("name,drop", [("bf16_packed_masked", None), ("fp16_packed_masked_D128", None),
                                       ("bf16_packed_masked", (0.2, 77, 9))])
def test_bwd_side_by_side_is_bitwise_serial(name, drop):
    """Packed batches of uneven sequences run the dK/dV and dQ kernels on two
    streams; every output must be bitwise the serial order's (the stage
    profiler forces that order), also twice in a row."""
    import deberta_disentangled_attention_rel_amd as df
    from parity_util import to_dev
    print(f"side by side vs serial {name} dropout={drop}", flush=True)
    inp = _inp(**CASES[name])
    w = inp.workload
    t, km, cu = to_dev(inp)
    kw = dict(key_mask=km, cu_seqlens=cu, max_seqlen=inp.max_seqlen)
    if drop:
        kw.update(dropout_p=drop[0], seed=drop[1], offset=drop[2])
    out, lse = df.fwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets, **kw)

    def bwd():
        g = df.bwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets, out, lse, t["dout"], **kw)
        torch.cuda.synchronize()
        return [x.clone() for x in g]

    a1, a2 = bwd(), bwd()
    df.profile_enable(True)
    try:
        b = bwd()
        df.profile_read()
    finally:
        df.profile_enable(False)
    for n_, x, y, z in zip(("dq", "dk", "dv", "dq_r", "dk_r"), a1, a2, b):
        assert torch.equal(x, y), n_
        assert torch.equal(x, z), n_


def _onehot_rows(lengths, H, D):
    """[T, H, D] float64 with row t = e_i, i = t's position in its sequence
    (every length <= D)."""
    x = np.zeros((sum(lengths), H, D))
    st = 0
    for n in lengths:
        i = np.arange(n)
        x[st + i, :, i] = 1.0
        st += n
    return x


@pytest.mark.parametrize("D,lengths", [(64, [64, 37, 1, 9, 16, 63, 8]), (128, [128, 77, 1, 33, 96, 8, 9])])
def test_dropout_mask_bits(D, lengths):
    """Each kernel's keep decisions against the oracle's mask, pair by pair
    (a rel-L2 over a whole tensor could hide a few wrong pairs).

    Forward and dK/dV: with V and dO one-hot by position in the sequence,
    O[i, j] = P_ij F_ij / (1 - p) and dV[j, i] = P_ij F_ij / (1 - p), so their
    zero patterns are the two kernels' masks. dQ: with K and V one-hot and
    the relative rows zero, dQ[i, j] = s dS_ij with dS_ij = P_ij (F_ij dP_ij /
    (1 - p) - Delta_i), dP_ij = dO_i[j]; each element lies next to the value
    for F = 1 or for F = 0, decided where the two differ well beyond bf16
    rounding."""
    import deberta_disentangled_attention_rel_amd as df
    from oracle import philox
    from parity_util import to_dev
    H, p, seed, offset = 2, 0.3, 20261203 + D, 5
    print(f"dropout mask bits D={D} lengths={lengths}", flush=True)
    inp = _inp(lengths=lengths, H=H, D=D, span=64, buckets=32, seed=21 + D)
    w = inp.workload
    oh = _onehot_rows(lengths, H, D)
    masks = []
    st = 0
    for n, L in enumerate(lengths):
        masks.append([philox.keep_mask(p, seed, offset, n, h, H, L) for h in range(H)])
    dkw = dict(dropout_p=p, seed=seed, offset=offset)

    # forward and dK/dV
    for nm in ("v", "dout"):
        inp.t[nm] = torch.from_numpy(oh).to(inp.t[nm].dtype)
    t, km, cu = to_dev(inp)
    kw = dict(key_mask=km, cu_seqlens=cu, max_seqlen=inp.max_seqlen)
    out, lse = df.fwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets, **kw, **dkw)
    g = df.bwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets, out, lse, t["dout"], **kw, **dkw)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    dv = g[2].float().cpu().numpy()
    st = 0
    for n, L in enumerate(lengths):
        for h in range(H):
            m = masks[n][h]
            assert np.array_equal(o[st:st + L, h, :L] != 0, m), ("forward", n, h)
            assert np.array_equal(dv[st:st + L, h, :L].T != 0, m), ("dK/dV", n, h)
        st += L

    # dQ
    inp = _inp(lengths=lengths, H=H, D=D, span=64, buckets=32, seed=21 + D)
    for nm in ("k", "v"):
        inp.t[nm] = torch.from_numpy(oh).to(inp.t[nm].dtype)
    for nm in ("q_r", "k_r"):
        inp.t[nm] = torch.zeros_like(inp.t[nm])
    t, km, cu = to_dev(inp)
    out, lse = df.fwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets, **kw, **dkw)
    g = df.bwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets, out, lse, t["dout"], **kw, **dkw)
    torch.cuda.synchronize()
    s = 1.0 / np.sqrt(3.0 * D)
    q = inp.t["q"].double().numpy()
    do = inp.t["dout"].double().numpy()
    o = out.double().cpu().numpy()
    dq = g[0].double().cpu().numpy()
    st, decided, total = 0, 0, 0
    for n, L in enumerate(lengths):
        for h in range(H):
            S = s * q[st:st + L, h, :L]  # S_ij = s q_i . e_j
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            dP = do[st:st + L, h, :L]  # dO_i . e_j
            dlt = (do[st:st + L, h, :] * o[st:st + L, h, :]).sum(axis=1, keepdims=True)
            ds1, ds0 = P * (dP / (1.0 - p) - dlt), P * (-dlt)
            gq = dq[st:st + L, h, :L] / s
            ok = np.abs(ds1 - ds0) > 0.1 * (np.abs(ds1) + np.abs(ds0))
            implied = np.abs(gq - ds1) < np.abs(gq - ds0)
            assert np.array_equal(implied[ok], masks[n][h][ok]), ("dQ", n, h)
            decided += int(ok.sum())
            total += L * L
        st += L
    assert decided >= 0.8 * total, (decided, total)


# ----------------------------------------------------------------------------
# structure the method fixes, checked on the GPU's own output: every valid row
# of dS sums to zero, so sum_r dK_r[h, r, :] = 0 (up to the rounding of the
# stored dC2P strip and of dk_r); sum_r dQ_r is not zero

@pytest.mark.parametrize("name", ["bf16_D64_bucketed_ragged", "fp32_D64", "bf16_packed_masked"])
def test_gpu_dk_r_rows_sum_to_zero(name):
    inp = _inp(**CASES[name])
    print(f"zero sums {name}", flush=True)
    gpu = run_gpu(inp)
    for h in range(gpu["dk_r"].shape[0]):
        s_k = np.linalg.norm(gpu["dk_r"][h].astype(np.float64).sum(axis=0))
        s_q = np.linalg.norm(gpu["dq_r"][h].astype(np.float64).sum(axis=0))
        n_k = np.linalg.norm(gpu["dk_r"][h].astype(np.float64))
        tol = 1e-5 if inp.dtype == "fp32" else 2e-2
        assert s_k <= tol * n_k, (h, s_k, n_k)
        assert s_q > 10 * tol * np.linalg.norm(gpu["dq_r"][h].astype(np.float64))
