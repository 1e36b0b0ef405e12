"""GPU parity at the full sizes of the five workloads, through the C ABI, in
the launch configuration the benchmark times.

The oracle cannot evaluate every head of the large workloads in seconds, so
(per workload) two seeded heads are compared in full (every sequence, every
output tensor, including dq_r / dk_r, which sum over all sequences) and the
other heads on 64 seeded query rows (O, LSE and dQ need only their own row).
Tolerances (rel-L2 per tensor): bf16/fp16 forward 1e-2, gradients 2e-2;
fp32 1e-5; every compared row also on its own, within ROW_MULT times the
tensor tolerance (parity_util.max_row_err), so that a few wrong rows cannot
hide in a tensor-wide figure. The long unbucketed stress workload also checks that two backward
runs are bitwise identical.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import workload_inputs, WORKLOADS
from parity_util import rel_l2, TOL, to_dev, max_row_err, ROW_MULT

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _gpu(inp, backward, p2c="literal"):
    import deberta_disentangled_attention_rel_amd as df
    w = inp.workload
    t, km, cu = to_dev(inp)
    kw = dict(key_mask=km, cu_seqlens=cu, max_seqlen=inp.max_seqlen, p2c=p2c)
    out, lse = df.fwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets, **kw)
    res = {"out": out, "lse": lse}
    if backward:
        g = df.bwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets, out, lse,
                   t["dout"], **kw)
        res.update(dict(zip(("dq", "dk", "dv", "dq_r", "dk_r"), g)))
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy() for k, v in res.items()}


def _check(n, dtype=None, backward=True, p2c="literal"):
    inp = workload_inputs(n, dtype=dtype, with_dout=backward)
    w = inp.workload
    print(f"workload {n} ({w.name}, {inp.dtype}, p2c {p2c}): T={inp.total_tokens} nseq={inp.nseq}", flush=True)
    gpu = _gpu(inp, backward, p2c)
    f = inp.f64
    H = w.heads
    rng = np.random.default_rng(w.seed + 1)
    full = sorted(rng.choice(H, size=min(2, H), replace=False).tolist())
    tol_f, tol_b = TOL[inp.dtype]
    kw = dict(key_mask=inp.key_mask, cu_seqlens=inp.cu_seqlens, batch=inp.nseq, p2c=p2c)
    out, lse = oracle.forward(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], w.span, w.buckets,
                              heads=full, **kw)
    errs = {}
    for h in full:
        valid = np.isfinite(lse[h])
        assert np.array_equal(np.isfinite(gpu["lse"][h]), valid)
        errs[f"out[h{h}]"] = (rel_l2(gpu["out"][:, h], out[:, h]), tol_f)
        errs[f"out rows[h{h}]"] = (max_row_err(gpu["out"][:, h], out[:, h]), ROW_MULT * tol_f)
        errs[f"lse[h{h}]"] = (rel_l2(gpu["lse"][h][valid], lse[h][valid]), tol_f)
        # each valid row's LSE to the same relative bound
        errs[f"lse rows[h{h}]"] = (float(np.max(np.abs(gpu["lse"][h][valid] - lse[h][valid]) /
                                                np.maximum(np.abs(lse[h][valid]), 1.0))) if valid.any() else 0.0,
                                   ROW_MULT * tol_f)
    if backward:
        g = oracle.backward(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], f["dout"], w.span,
                            w.buckets, heads=full, **kw)
        for name, ref in zip(("dq", "dk", "dv", "dq_r", "dk_r"), g):
            for h in full:
                a = gpu[name][:, h] if name in ("dq", "dk", "dv") else gpu[name][h]
                b = ref[:, h] if name in ("dq", "dk", "dv") else ref[h]
                errs[f"{name}[h{h}]"] = (rel_l2(a, b), tol_b)
                errs[f"{name} rows[h{h}]"] = (max_row_err(a, b), ROW_MULT * tol_b)
    # other heads: sampled query rows
    seqs = oracle.sequences(inp.total_tokens, inp.cu_seqlens, inp.nseq)
    rest = [h for h in range(H) if h not in full]
    go, gl, gq, ro, rl, rq = [], [], [], [], [], []
    for h in rest:
        for _ in range(64 // max(1, len(rest)) + 1):
            s = int(rng.integers(len(seqs)))
            st, en = seqs[s]
            if en == st:
                continue
            rows = np.array([int(rng.integers(en - st))])
            o, l = oracle.forward_rows(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], w.span,
                                       w.buckets, (st, en), h, rows, key_mask=inp.key_mask, p2c=p2c)
            go.append(gpu["out"][st + rows, h]); ro.append(o)
            gl.append(gpu["lse"][h, st + rows]); rl.append(l)
            if backward:
                d = oracle.dq_rows(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], f["dout"], w.span,
                                   w.buckets, (st, en), h, rows, key_mask=inp.key_mask, p2c=p2c)
                gq.append(gpu["dq"][st + rows, h]); rq.append(d)
    if rest:
        gl_, rl_ = np.concatenate(gl), np.concatenate(rl)
        assert np.array_equal(np.isfinite(gl_), np.isfinite(rl_))
        v = np.isfinite(rl_)
        errs["out[sampled rows]"] = (rel_l2(np.concatenate(go), np.concatenate(ro)), tol_f)
        errs["out[each sampled row]"] = (max_row_err(np.concatenate(go), np.concatenate(ro)), ROW_MULT * tol_f)
        errs["lse[sampled rows]"] = (rel_l2(gl_[v], rl_[v]), tol_f)
        if backward:
            errs["dq[sampled rows]"] = (rel_l2(np.concatenate(gq), np.concatenate(rq)), tol_b)
            errs["dq[each sampled row]"] = (max_row_err(np.concatenate(gq), np.concatenate(rq)), ROW_MULT * tol_b)
    print({k: f"{e:.2e}" for k, (e, _) in errs.items()}, flush=True)
    bad = {k: e for k, (e, t) in errs.items() if not (e <= t)}
    assert not bad, bad
    return gpu


def test_workload2_bf16_L512_forward():
    _check(2, backward=False)


def test_workload3_bf16_L8192_fwd_bwd():
    _check(3)


def test_workload4_packed_varlen_masked():
    _check(4)


@pytest.mark.parametrize("n", [3, 4])
def test_shared_p2c_full_size(n):
    """The shared P2C convention at the L=8192 and packed workloads."""
    _check(n, p2c="shared")


@pytest.mark.parametrize("dtype", ["fp16", "fp32"])
def test_workload5_unbucketed_deterministic(dtype):
    gpu = _check(5, dtype=dtype)
    inp = workload_inputs(5, dtype=dtype)
    again = _gpu(inp, True)
    for n in ("dq_r", "dk_r", "dq", "dk", "dv", "out", "lse"):
        assert np.array_equal(gpu[n].view(np.uint32), again[n].view(np.uint32)), n


@pytest.mark.parametrize("n", [3, 4])
def test_inference_forward_full_size(n):
    """The inference forward at full size equals the training forward's output
    bit for bit (the same kernel without the LSE store); the training forward
    is compared with the oracle by the tests above."""
    import deberta_disentangled_attention_rel_amd as df
    inp = workload_inputs(n, with_dout=False)
    w = inp.workload
    print(f"inference forward, workload {n}", flush=True)
    t, km, cu = to_dev(inp)
    kw = dict(key_mask=km, cu_seqlens=cu, max_seqlen=inp.max_seqlen)
    out_t, _ = df.fwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets, **kw)
    out_i = df.fwd_inference(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out_i, out_t)


def test_dropout_full_size_one_head():
    """Attention dropout (p = 0.1) at the L=8192 workload: one seeded head in
    full (both sequences, every output including that head's dq_r / dk_r),
    which exercises the Philox counters at large query and key indices."""
    import deberta_disentangled_attention_rel_amd as df
    inp = workload_inputs(3)
    w = inp.workload
    p, seed, offset = 0.1, 20261203, 7
    print(f"dropout full size p={p}", flush=True)
    t, km, cu = to_dev(inp)
    kw = dict(key_mask=km, cu_seqlens=cu, max_seqlen=inp.max_seqlen, dropout_p=p, seed=seed, offset=offset)
    args = (t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets)
    out, lse = df.fwd(*args, **kw)
    g = df.bwd(*args, out, lse, t["dout"], **kw)
    torch.cuda.synchronize()
    h = int(np.random.default_rng(w.seed + 3).integers(w.heads))
    f = inp.f64
    okw = dict(key_mask=inp.key_mask, cu_seqlens=inp.cu_seqlens, batch=inp.nseq, heads=[h],
               dropout=(p, seed, offset))
    ro, rl = oracle.forward(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], w.span, w.buckets, **okw)
    rg = oracle.backward(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], f["dout"], w.span, w.buckets, **okw)
    tol_f, tol_b = TOL[inp.dtype]
    errs = {"out": (rel_l2(out.float().cpu().numpy()[:, h], ro[:, h]), tol_f),
            "lse": (rel_l2(lse.cpu().numpy()[h], rl[h]), tol_f)}
    for name, a, b in zip(("dq", "dk", "dv", "dq_r", "dk_r"), g, rg):
        a = a.float().cpu().numpy()
        errs[name] = (rel_l2(a[:, h] if name in ("dq", "dk", "dv") else a[h],
                             b[:, h] if name in ("dq", "dk", "dv") else b[h]), tol_b)
    print({k: f"{e:.2e}" for k, (e, _) in errs.items()}, flush=True)
    bad = {k: e for k, (e, t_) in errs.items() if not (e <= t_)}
    assert not bad, bad


def test_long_sequence_L65519_sampled_rows_and_sums():
    """One sequence eight times the benchmark's length, ending in a ragged
    47-row tile: O, LSE and dQ on seeded rows against the oracle's row
    functions, sum_j dV_j = sum_i dO_i (every row of P sums to one, so this
    holds at any size), and a bitwise-repeatable backward."""
    import deberta_disentangled_attention_rel_amd as df
    from synth import make_inputs
    L, H, D, span, buckets, R = 65519, 2, 64, 512, 256, 512
    inp = make_inputs(H, D, "bf16", span, buckets, R, seed=4242, batch=1, seqlen=L)
    print(f"long sequence: L={L} H={H} D={D} bf16", flush=True)
    t, km, cu = to_dev(inp)
    out, lse = df.fwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], span, buckets, max_seqlen=L)
    g1 = df.bwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], span, buckets, out, lse, t["dout"], max_seqlen=L)
    g2 = df.bwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], span, buckets, out, lse, t["dout"], max_seqlen=L)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    out_h, lse_h, dq_h, dv_h = (x.float().cpu().numpy() for x in (out, lse, g1[0], g1[2]))
    f = inp.f64
    tol_f, tol_b = TOL["bf16"]
    rng = np.random.default_rng(4243)
    # the first and last rows, the ragged tail, and seeded rows in between
    rows = np.unique(np.concatenate([[0, L - 1], L - 1 - np.arange(47),
                                     rng.integers(0, L, size=32)]))[::2]
    rows = np.union1d(rows, [L - 1])
    errs = {}
    for h in range(H):
        o, l = oracle.forward_rows(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], span, buckets,
                                   (0, L), h, rows)
        d = oracle.dq_rows(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], f["dout"], span, buckets,
                           (0, L), h, rows)
        errs[f"out[h{h}]"] = (rel_l2(out_h[rows, h], o), tol_f)
        errs[f"lse[h{h}]"] = (rel_l2(lse_h[h, rows], l), tol_f)
        errs[f"dq[h{h}]"] = (rel_l2(dq_h[rows, h], d), tol_b)
        # every dV_j is near the same vector (P is nearly uniform at this
        # length), so their bf16 roundings (at most 2^-9 relative each) can
        # add up coherently: the bound is 2^-9 plus the fp32 accumulation
        errs[f"sum dv[h{h}]"] = (rel_l2(dv_h[:, h].astype(np.float64).sum(0), f["dout"][:, h].sum(0)), 4e-3)
    print({k: f"{e:.2e}" for k, (e, _) in errs.items()}, flush=True)
    bad = {k: e for k, (e, t_) in errs.items() if not (e <= t_)}
    assert not bad, bad


def test_workload3_bwd_reusing_forward_workspace():
    """The benchmark's launch configuration at full size: the backward runs on
    the forward's workspace (index tables and strips kept) and must equal,
    bit for bit, the recomputing backward that the workload-3 test compares
    with the oracle on the same seeded inputs."""
    import deberta_disentangled_attention_rel_amd as df
    inp = workload_inputs(3)
    w = inp.workload
    print(f"workload 3 ({w.name}): backward reusing the forward's workspace", flush=True)
    t, km, cu = to_dev(inp)
    kw = dict(key_mask=km, cu_seqlens=cu, max_seqlen=inp.max_seqlen)
    args = (t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets)
    shape = df.make_shape(t["q"].view(-1, *t["q"].shape[-2:]), inp.nseq, inp.max_seqlen)
    ws = torch.empty(df.workspace_size(1, shape, w.span, w.buckets), dtype=torch.uint8, device="cuda")
    out, lse = df.fwd(*args, workspace=ws, **kw)
    g_reuse = df.bwd(*args, out, lse, t["dout"], workspace=ws, reuse_fwd_workspace=True, **kw)
    g_fresh = df.bwd(*args, out, lse, t["dout"], **kw)
    torch.cuda.synchronize()
    for n_, a, b in zip(("dq", "dk", "dv", "dq_r", "dk_r"), g_reuse, g_fresh):
        assert torch.equal(a, b), n_
    # the timed dropout step (p = 0.1) the same way
    dk = dict(kw, dropout_p=0.1, seed=1234, offset=0)
    out, lse = df.fwd(*args, workspace=ws, **dk)
    g_reuse = df.bwd(*args, out, lse, t["dout"], workspace=ws, reuse_fwd_workspace=True, **dk)
    g_fresh = df.bwd(*args, out, lse, t["dout"], **dk)
    torch.cuda.synchronize()
    for n_, a, b in zip(("dq", "dk", "dv", "dq_r", "dk_r"), g_reuse, g_fresh):
        assert torch.equal(a, b), "dropout " + n_
