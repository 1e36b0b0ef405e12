"""df_attn_fwd_noalloc (the forward whose workspace is the library's static
scratch array, for callers that cannot allocate) against df_attn_fwd with a
caller workspace on the same inputs: out and lse equal bit for bit, on two
calls in a row, the second with a smaller input (the scratch keeps the first
call's contents), and with lse = NULL against df_attn_fwd_inference."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from synth import make_inputs
from parity_util import to_dev

pytestmark = pytest.mark.gpu


def _noalloc(df, inp, t, km, cu, with_lse=True):
    w = inp.workload
    q3 = t["q"]
    shape = df.make_shape(q3, inp.nseq, inp.max_seqlen)
    out = torch.empty_like(q3)
    lse = torch.empty((q3.shape[1], q3.shape[0]), dtype=torch.float32, device=q3.device) if with_lse else None
    p = df._ptr
    rc = df.lib().df_attn_fwd_noalloc(ctypes.byref(shape), p(t["q"]), p(t["k"]), p(t["v"]), p(t["q_r"]),
                                      p(t["k_r"]), w.span, w.buckets, p(km), p(cu), p(out), p(lse),
                                      df._stream(q3.device))
    df._check(rc)
    return out, lse


@pytest.mark.parametrize("first,second", [
    # (T, H, D, dtype, span, buckets, lengths/padded, mask) of the two calls
    ((dict(batch=2, L=1300, dtype="bf16", H=12, D=64, span=512, buckets=256, packed=False, mask_frac=0.0)),
     (dict(batch=3, L=200, dtype="fp16", H=4, D=128, span=512, buckets=256, packed=True,
           lengths=[200, 37, 120], mask_frac=0.1))),
    ((dict(batch=2, L=256, dtype="fp32", H=2, D=32, span=64, buckets=0, packed=False, mask_frac=0.1)),
     (dict(batch=1, L=64, dtype="bf16", H=2, D=32, span=32, buckets=0, packed=False, mask_frac=0.0))),
])
def test_noalloc_matches_workspace_forward(first, second):
    import deberta_disentangled_attention_rel_amd as df
    for n, cfg in enumerate((first, second)):
        cfg = dict(cfg)
        batch, L, dtype, H, D = cfg.pop("batch"), cfg.pop("L"), cfg.pop("dtype"), cfg.pop("H"), cfg.pop("D")
        span, buckets = cfg.pop("span"), cfg.pop("buckets")
        att, R = oracle.att_and_rows(span, buckets)
        print(f"noalloc call {n}: B={batch} L={L} {dtype} H={H} D={D} span={span} buckets={buckets}", flush=True)
        if cfg.pop("packed"):
            inp = make_inputs(H, D, dtype, span, buckets, R, seed=900 + n, packed=True, **cfg)
        else:
            inp = make_inputs(H, D, dtype, span, buckets, R, seed=900 + n, batch=batch, seqlen=L, **cfg)
        t, km, cu = to_dev(inp)
        shape = df.make_shape(t["q"], inp.nseq, inp.max_seqlen)
        assert df.workspace_size(0, shape, span, buckets) <= (64 << 20)
        out_n, lse_n = _noalloc(df, inp, t, km, cu)
        out_r, lse_r = df.fwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], span, buckets, key_mask=km,
                              cu_seqlens=cu, max_seqlen=inp.max_seqlen)
        inf_n, _ = _noalloc(df, inp, t, km, cu, with_lse=False)
        inf_r = df.fwd_inference(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], span, buckets, key_mask=km,
                                 cu_seqlens=cu, max_seqlen=inp.max_seqlen)
        torch.cuda.synchronize()
        bits = torch.int32 if out_n.dtype == torch.float32 else torch.int16
        assert torch.equal(out_n.view(bits), out_r.view(bits))
        assert torch.equal(lse_n, lse_r)
        assert torch.equal(inf_n.view(bits), inf_r.view(bits))
        assert torch.isfinite(out_n.float()).all()
