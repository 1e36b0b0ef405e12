"""End-to-end use of the library's pieces in the pages' order ("Packed
unpadded inference and training": pack right-padded hidden states, project
them, run packed attention, unpack): the fused projections on the packed
hidden states, the packed forward and backward, and the unpacked output,
against the oracle's composition of the same steps (packing, projection,
attention), on a seeded small configuration with ragged lengths."""
import numpy as np
import pytest
import torch

import oracle
from parity_util import rel_l2

pytestmark = pytest.mark.gpu


def test_pack_project_attend_unpack():
    import deberta_disentangled_attention_rel_amd as df
    rng = np.random.default_rng(31)
    B, L, H, D, span, buckets = 3, 160, 2, 64, 128, 64
    E = H * D
    att, R = oracle.att_and_rows(span, buckets)
    lens = [160, 37, 101]
    m = (np.arange(L)[None, :] < np.array(lens)[:, None]).astype(np.uint8)
    bf = torch.bfloat16
    x = torch.from_numpy(rng.standard_normal((B, L, E))).to(bf)
    w = torch.from_numpy(rng.standard_normal((3 * E, E)) / np.sqrt(E)).to(bf)
    b = torch.from_numpy(rng.standard_normal(3 * E) * 0.1).to(bf)
    rel = torch.from_numpy(rng.standard_normal((R, E))).to(bf)
    dout = torch.from_numpy(rng.standard_normal((B, L, H, D))).to(bf)

    # GPU: pack, project, attend (packed), unpack
    md = torch.from_numpy(m).cuda()
    xp, cu, mx = df.pack_padded(x.cuda(), md)
    q, k, v, q_r, k_r = df.qkv_proj(xp, w.cuda(), b.cuda(), rel.cuda(), H, D)
    out, lse = df.fwd(q, k, v, q_r, k_r, span, buckets, cu_seqlens=cu, max_seqlen=mx)
    dop, _, _ = df.pack_padded(dout.cuda(), md)
    dq, dk, dv, dq_r, dk_r = df.bwd(q, k, v, q_r, k_r, span, buckets, out, lse, dop, cu_seqlens=cu,
                                    max_seqlen=mx)
    o_pad = df.unpack_packed(out, cu, md)
    torch.cuda.synchronize()

    # oracle: the same composition in float64 on the rounded inputs (the
    # projections' outputs rounded to bf16 as the GPU stores them)
    f64 = lambda t: t.to(torch.float64).numpy()
    xp_o, cu_o, _ = oracle.pack_padded(f64(x), m)
    np.testing.assert_array_equal(cu.cpu().numpy(), cu_o)
    proj = oracle.qkv_projection(xp_o, f64(w), f64(b), f64(rel), H, D)
    for name, g, r in zip(("q", "k", "v", "q_r", "k_r"), (q, k, v, q_r, k_r), proj):
        e = rel_l2(g.float().cpu().numpy(), r)
        print(f"{name} rel-L2 {e:.2e}", flush=True)
        assert e <= 1e-2, name
    rq = [torch.from_numpy(a).to(bf).to(torch.float64).numpy() for a in proj]
    dop_o, _, _ = oracle.pack_padded(f64(dout), m)
    ref_o, _ = oracle.forward(*rq, span, buckets, cu_seqlens=cu_o, batch=B)
    ref_g = oracle.backward(*rq, dop_o, span, buckets, cu_seqlens=cu_o, batch=B)
    errs = {"out": rel_l2(o_pad.float().cpu().numpy(), oracle.unpack_packed(ref_o, cu_o, L, m))}
    for name, g, r in zip(("dq", "dk", "dv", "dq_r", "dk_r"), (dq, dk, dv, dq_r, dk_r), ref_g):
        errs[name] = rel_l2(g.float().cpu().numpy(), r)
    print({k_: f"{e:.2e}" for k_, e in errs.items()}, flush=True)
    assert errs["out"] <= 1e-2
    assert all(errs[n] <= 2e-2 for n in ("dq", "dk", "dv", "dq_r", "dk_r")), errs
