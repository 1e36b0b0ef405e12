"""Strided layouts through the raw C ABI (tok_stride / head_stride), which
the Python binding never produces (it passes contiguous [T, H, D] tensors):

* fused token-major: q, k, v are the three slices of one [T, 3, H, D]
  buffer (tok_stride 3*H*D, head_stride D) — the layout a fused QKV
  projection writes — and dq, dk, dv come back into one such buffer;
* head-major: every [T, H, D] tensor stored as [H, T, D] (tok_stride D,
  head_stride T*D).

Only the addressing changes, so forward and backward must equal the
contiguous run bit for bit (which the parity tests compare with the oracle).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from synth import make_inputs

pytestmark = pytest.mark.gpu


def _call(df, shape, q, k, v, q_r, k_r, span, buckets, out, lse, dout, dq, dk, dv, dq_r, dk_r, cu=None):
    L = df.lib()
    vp = ctypes.c_void_p
    ws_b = df.workspace_size(1, shape, span, buckets)
    ws = torch.empty(ws_b, dtype=torch.uint8, device="cuda")
    st = vp(torch.cuda.current_stream().cuda_stream)
    cu_p = vp(cu.data_ptr()) if cu is not None else None
    rc = L.df_attn_fwd(ctypes.byref(shape), vp(q), vp(k), vp(v), vp(q_r.data_ptr()), vp(k_r.data_ptr()),
                       span, buckets, None, cu_p, vp(out), vp(lse.data_ptr()), vp(ws.data_ptr()), ws_b, st)
    assert rc == 0, L.df_last_error().decode()
    rc = L.df_attn_bwd(ctypes.byref(shape), vp(q), vp(k), vp(v), vp(q_r.data_ptr()), vp(k_r.data_ptr()),
                       span, buckets, None, cu_p, vp(out), vp(lse.data_ptr()), vp(dout), vp(dq), vp(dk), vp(dv),
                       vp(dq_r.data_ptr()), vp(dk_r.data_ptr()), vp(ws.data_ptr()), ws_b, st)
    assert rc == 0, L.df_last_error().decode()
    torch.cuda.synchronize()


@pytest.mark.parametrize("layout", ["fused_qkv", "head_major"])
def test_strided_layouts_match_contiguous(layout):
    import deberta_disentangled_attention_rel_amd as df
    print(f"strided layout {layout}", flush=True)
    span, buckets = 64, 32
    att, R = oracle.att_and_rows(span, buckets)
    inp = make_inputs(2, 64, "bf16", span, buckets, R, seed=41, batch=2, seqlen=300)
    t = {k_: v_.cuda() for k_, v_ in inp.t.items()}
    T, H, D = t["q"].shape
    es = 2
    # the contiguous reference run, through the binding
    out_c, lse_c = df.fwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], span, buckets, max_seqlen=300)
    g_c = df.bwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], span, buckets, out_c, lse_c, t["dout"],
                 max_seqlen=300)
    torch.cuda.synchronize()
    lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
    dq_r, dk_r = torch.empty_like(t["q_r"]), torch.empty_like(t["k_r"])
    if layout == "fused_qkv":
        qkv = torch.stack([t["q"], t["k"], t["v"]], dim=1).contiguous()        # [T, 3, H, D]
        obuf = torch.zeros_like(qkv)                                             # out in slice 0
        dobuf = torch.zeros_like(qkv)
        dobuf[:, 0] = t["dout"]
        gbuf = torch.empty_like(qkv)                                             # dq, dk, dv
        shape = df.Shape(2, 300, T, H, D, 0, 3 * H * D, D, 0, 0)
        base, step = qkv.data_ptr(), H * D * es
        _call(df, shape, base, base + step, base + 2 * step, t["q_r"], t["k_r"], span, buckets,
              obuf.data_ptr(), lse, dobuf.data_ptr(), gbuf.data_ptr(), gbuf.data_ptr() + step,
              gbuf.data_ptr() + 2 * step, dq_r, dk_r)
        out, dq, dk, dv = obuf[:, 0], gbuf[:, 0], gbuf[:, 1], gbuf[:, 2]
    else:
        hm = {n: t[n].permute(1, 0, 2).contiguous() for n in ("q", "k", "v", "dout")}   # [H, T, D]
        out_h, dq_h, dk_h, dv_h = (torch.empty_like(hm["q"]) for _ in range(4))
        shape = df.Shape(2, 300, T, H, D, 0, D, T * D, 0, 0)
        _call(df, shape, hm["q"].data_ptr(), hm["k"].data_ptr(), hm["v"].data_ptr(), t["q_r"], t["k_r"],
              span, buckets, out_h.data_ptr(), lse, hm["dout"].data_ptr(), dq_h.data_ptr(), dk_h.data_ptr(),
              dv_h.data_ptr(), dq_r, dk_r)
        out, dq, dk, dv = (x.permute(1, 0, 2) for x in (out_h, dq_h, dk_h, dv_h))
    assert torch.equal(out.reshape(T, H, D), out_c.reshape(T, H, D))
    assert torch.equal(lse, lse_c)
    for name, a, b in zip(("dq", "dk", "dv", "dq_r", "dk_r"), (dq, dk, dv, dq_r, dk_r), g_c):
        assert torch.equal(a.reshape(b.shape), b), name
