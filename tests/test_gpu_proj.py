"""GPU parity of the fused Q/K/V and relative-position projections
(df_qkv_proj, through the C ABI binding) against the float64 oracle.

Cases span ragged row and column tiles (tokens, relative rows and 3*H*D not
multiples of 128), a hidden size that is not a multiple of the 64-wide
contraction step, no bias, no relative rows, no tokens, both 16-bit dtypes,
and the metric workload's projection shape (tokens 16384, hidden 768, 12
heads of 64, 512 relative rows) on a seeded sample of token rows. Tolerance:
rel-L2 <= 1e-2 per output (the forward tolerance for 16-bit outputs); a
second call must give bitwise-identical outputs.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import make_proj_inputs
from parity_util import rel_l2

pytestmark = pytest.mark.gpu
NAMES = ("q", "k", "v", "q_r", "k_r")


def _run(inp):
    import deberta_disentangled_attention_rel_amd as df
    t = {k: v.cuda() for k, v in inp.t.items()}
    outs = df.qkv_proj(t["x"], t["w"], t.get("bias"), t.get("rel"), inp.heads, inp.head_dim)
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("T,E,H,D,R,dtype,bias,rel", [
    (300, 64, 2, 32, 64, "bf16", True, True),
    (1000, 768, 12, 64, 512, "bf16", True, True),
    (1000, 768, 12, 64, 512, "fp16", True, True),
    (257, 136, 3, 32, 10, "bf16", True, True),
    (129, 256, 2, 128, 1, "fp16", False, True),
    (77, 64, 1, 64, 0, "bf16", True, False),
    (0, 64, 2, 32, 33, "bf16", True, True),
])
def test_proj_parity(T, E, H, D, R, dtype, bias, rel):
    print(f"proj T={T} E={E} H={H} D={D} R={R} {dtype} bias={bias} rel={rel}", flush=True)
    inp = make_proj_inputs(T, E, H, D, R, dtype, seed=T + E + H, bias=bias, rel=rel)
    f = inp.f64
    ref = oracle.qkv_projection(f["x"], f["w"], f.get("bias"), f.get("rel"), H, D)
    got = _run(inp)
    for nm, g, r in zip(NAMES, got, ref):
        if r is None:
            assert g is None
            continue
        if r.size == 0:
            continue
        e = rel_l2(g.float().cpu().numpy(), r)
        print(f"  {nm} rel-L2 {e:.2e}", flush=True)
        assert e <= 1e-2, (nm, e)
    again = _run(inp)
    for g, h in zip(got, again):
        if g is not None:
            assert torch.equal(g, h)


def test_proj_metric_shape_sampled_rows():
    """Tokens 16384, hidden 768, 12 heads of 64, 512 relative rows: every
    relative output in full, 256 seeded token rows of q, k, v."""
    T, E, H, D, R = 16384, 768, 12, 64, 512
    print(f"proj full size T={T} E={E} H={H} D={D} R={R}", flush=True)
    inp = make_proj_inputs(T, E, H, D, R, "bf16", seed=11)
    got = _run(inp)
    f = inp.f64
    rows = np.sort(np.random.default_rng(12).choice(T, 256, replace=False))
    ref = oracle.qkv_projection(f["x"][rows], f["w"], f["bias"], f["rel"], H, D)
    for nm, g, r in zip(NAMES, got, ref):
        g = g.float().cpu().numpy()
        if nm in ("q", "k", "v"):
            g = g[rows]
        e = rel_l2(g, r)
        print(f"  {nm} rel-L2 {e:.2e}", flush=True)
        assert e <= 1e-2, (nm, e)


# ----------------------------------------------------------------------------
# backward of the projections (df_qkv_proj_bwd)

def _grads(T, H, D, R, dtype, seed):
    from synth import DTYPES
    rng = np.random.default_rng(seed)
    dt = DTYPES[dtype]
    dqkv = torch.from_numpy(rng.standard_normal((T, 3, H, D))).to(dt)
    dq_r = torch.from_numpy(rng.standard_normal((H, R, D))).to(dt)
    dk_r = torch.from_numpy(rng.standard_normal((H, R, D))).to(dt)
    return dqkv, dq_r, dk_r


@pytest.mark.parametrize("T,E,H,D,R,dtype,rel", [
    (300, 64, 2, 32, 64, "bf16", True),
    (1000, 768, 12, 64, 512, "bf16", True),
    (1000, 768, 12, 64, 512, "fp16", True),
    (257, 136, 3, 32, 10, "bf16", True),
    (129, 256, 2, 128, 0, "fp16", False),
    (0, 64, 2, 32, 33, "bf16", True),
    (16384, 768, 12, 64, 512, "bf16", True),
])
def test_proj_bwd_parity(T, E, H, D, R, dtype, rel):
    import deberta_disentangled_attention_rel_amd as df
    print(f"proj bwd T={T} E={E} H={H} D={D} R={R} {dtype} rel={rel}", flush=True)
    inp = make_proj_inputs(T, E, H, D, R, dtype, seed=T + 3 * E + H, rel=rel)
    dqkv, dq_r, dk_r = _grads(T, H, D, R, dtype, seed=T + 7)
    f = inp.f64
    g64 = {n: t.to(torch.float64).numpy() for n, t in (("dqkv", dqkv), ("dq_r", dq_r), ("dk_r", dk_r))}
    ref = oracle.qkv_projection_backward(f["x"], f["w"], f.get("rel"), g64["dqkv"][:, 0], g64["dqkv"][:, 1],
                                         g64["dqkv"][:, 2], g64["dq_r"] if rel else None,
                                         g64["dk_r"] if rel else None, H, D)
    x, w = inp.t["x"].cuda(), inp.t["w"].cuda()
    rl = inp.t["rel"].cuda() if rel else None
    args = (x, w, rl, dqkv.cuda(), dq_r.cuda() if rel else None, dk_r.cuda() if rel else None)
    got = df.qkv_proj_bwd(*args, num_heads=H, head_dim=D)
    again = df.qkv_proj_bwd(*args, num_heads=H, head_dim=D)
    torch.cuda.synchronize()
    for name, g, r, h in zip(("dx", "dw", "db", "drel"), got, ref, again):
        if r is None:
            assert g is None
            continue
        assert torch.equal(g, h), name
        if r.size == 0:
            continue
        e = rel_l2(g.float().cpu().numpy(), r)
        print(f"  {name} rel-L2 {e:.2e}", flush=True)
        assert e <= 1e-2, (name, e)
