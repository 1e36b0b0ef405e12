"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
binding and compare with the float64 oracle on identical seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = {"bf16": (1e-2, 2e-2), "fp16": (1e-2, 2e-2), "fp32": (1e-5, 1e-5)}  # (forward, gradients)


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return float(num / den) if den > 0 else float(num)


def to_dev(inp, dev="cuda"):
    t = {k: v.to(dev) for k, v in inp.t.items()}
    km = None if inp.key_mask is None else torch.from_numpy(inp.key_mask).to(dev)
    cu = None if inp.cu_seqlens is None else torch.from_numpy(inp.cu_seqlens).to(dev)
    return t, km, cu


def run_gpu(inp, backward=True, dev="cuda", p2c="literal"):
    import deberta_disentangled_attention_rel_amd as df
    w = inp.workload
    t, km, cu = to_dev(inp, dev)
    kw = dict(key_mask=km, cu_seqlens=cu, max_seqlen=inp.max_seqlen, p2c=p2c)
    out, lse = df.fwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets, **kw)
    res = {"out": out, "lse": lse}
    if backward:
        g = df.bwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets, out, lse,
                   t["dout"], **kw)
        res.update(dict(zip(("dq", "dk", "dv", "dq_r", "dk_r"), g)))
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy() for k, v in res.items()}


def run_oracle(inp, backward=True, p2c="literal"):
    f = inp.f64
    w = inp.workload
    kw = dict(key_mask=inp.key_mask, cu_seqlens=inp.cu_seqlens, batch=inp.nseq, p2c=p2c)
    out, lse = oracle.forward(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], w.span, w.buckets, **kw)
    res = {"out": out, "lse": lse}
    if backward:
        g = oracle.backward(f["q"], f["k"], f["v"], f["q_r"], f["k_r"], f["dout"], w.span,
                            w.buckets, **kw)
        res.update(dict(zip(("dq", "dk", "dv", "dq_r", "dk_r"), g)))
    return res


def compare(inp, gpu, ref, backward=True):
    """rel-L2 of every output; LSE over valid rows, masked rows must be -inf."""
    tol_f, tol_b = TOL[inp.dtype]
    errs = {}
    lse_g, lse_r = gpu["lse"], ref["lse"]
    valid = np.isfinite(lse_r)
    assert np.array_equal(np.isfinite(lse_g), valid), "LSE -inf pattern differs"
    errs["lse"] = rel_l2(lse_g[valid], lse_r[valid])
    errs["out"] = rel_l2(gpu["out"], ref["out"])
    names = ["out", "lse"]
    if backward:
        for n in ("dq", "dk", "dv", "dq_r", "dk_r"):
            errs[n] = rel_l2(gpu[n], ref[n])
        names += ["dq", "dk", "dv", "dq_r", "dk_r"]
    bad = {n: e for n, e in errs.items()
           if not np.isfinite(e) or e > (tol_f if n in ("out", "lse") else tol_b)}
    return errs, bad


# Per-row gate at the full sizes: a tensor-wide rel-L2 over 16,384 rows can
# hide a few wrong rows (one zeroed row adds only ~0.8%), so every compared
# row is also checked on its own. A row's error is its L2 error over its
# reference norm, the norm floored at ROW_FLOOR times the RMS row norm (a
# masked row, whose reference is exactly zero, must then come out near zero).
# The bound is ROW_MULT times the tensor tolerance: a zeroed or sign-flipped
# row scores 1 or 2, far above it, while bf16 rounding of a 32..128-element
# row stays well below it.
ROW_MULT = 4.0
ROW_FLOOR = 0.05


def max_row_err(x, ref) -> float:
    """Largest per-row relative L2 error of x against ref (rows = axis 0)."""
    x = np.asarray(x, dtype=np.float64).reshape(len(ref), -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(len(ref), -1)
    if ref.size == 0:
        return 0.0
    rn = np.linalg.norm(ref, axis=1)
    rms = float(np.sqrt(np.mean(rn ** 2)))
    den = np.maximum(rn, ROW_FLOOR * rms) if rms > 0 else np.ones_like(rn)
    return float(np.max(np.linalg.norm(x - ref, axis=1) / den))
