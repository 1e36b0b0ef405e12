#!/usr/bin/env python3
"""Forward+backward throughput of exact disentangled attention on one MI355X.

Workload (the DisentangledFlash 1.1.1 page, "Performance": BF16, 12 heads,
head dim 64, 16,384 active tokens, padded layout, all tokens active, no
dropout): B=2, L=8192, H=12, D=64, log-bucketed relative index with
position_buckets=256, max_relative_positions=512 (R=512), synthetic seeded
inputs N(0, 1/D), dout N(0, 1).

A step is one pass of the whole path: the forward (index tables, strips,
fused forward) and the backward (Delta, dK/dV and dQ with their
relative-gradient epilogues, the split-K relative-row gradients), which
reuses the forward's index tables and strips from the shared workspace
(DF_FLAG_BWD_REUSE_FWD; the line also reports the backward recomputing
them). FLOPs per step follow the page's convention,
B*H*(14 L^2 D + 16 L R D). Inputs, outputs and the workspace are resident in
HBM before timing; nothing is allocated inside the timed region.

Prints one JSON line. Per-kernel durations come from HIP events recorded by
the library around each of its launches during the timed steps.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+bwd TFLOP/s (BH(14L²D+16LRD)) L=8192 H=12 D=64 bf16; % MFMA peak"
WORKLOAD = 3
# MI355X dense bf16 MFMA peak: 256 CUs x 4096 FLOP/clk x 2.4 GHz
PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
# the pages' own latency for this exact workload (H200, DF Triton, fwd+bwd)
PAGES_H200_FWD_BWD_MS = 53.80


def flops_fwd_bwd(B, H, L, D, R):
    return B * H * (14.0 * L * L * D + 16.0 * L * R * D)


# MI355X dense fp32 MFMA peak (the strict-fp32 path's matrix products)
PEAK_FP32_TFLOPS = 157.3


def kernel_algorithmic_flops(stage, B, H, L, D, R):
    """Algorithmic FLOPs of one launch of a stage (matrix products it must run)."""
    per = B * H * L * L * D
    rel = B * H * L * R * D
    return {
        "fwd": 4.0 * per,                  # S = QK^T, O = PV
        "bwd_dkv": 8.0 * per + 2.0 * rel,  # S, dP = dO V^T, dV = P^T dO, dK = dS^T Q; dP2C Q_r
        "bwd_dq": 6.0 * per + 2.0 * rel,   # S, dP, dQ = dS K; dC2P K_r
        "strips": 2.0 * rel,               # one of Q K_r^T / K Q_r^T
        "relgrad_dw": 4.0 * rel,           # dC2P^T Q and dP2C^T K
    }.get(stage)


# Sources each stage's kernel is built from: the committed HBM-traffic figure
# of a kernel (profiles/hbm_traffic_<stage>_<workload>.md, from rocprofv3
# FETCH_SIZE / WRITE_SIZE runs) is reported only while these files hash to
# the value recorded with it.
_CSRC = os.path.join(ROOT, "deberta_disentangled_attention_rel_amd", "csrc")
_COMMON = ["common.hpp", "params.hpp", "pipe.hpp", "band.hpp", "walk.hpp", "tiles.hpp", "../build.py"]
STAGE_SOURCES = {
    "fwd": ["fwd.hip"] + _COMMON,
    "bwd_dkv": ["bwd_dkv.hip"] + _COMMON,
    "bwd_dq": ["bwd_dq.hip"] + _COMMON,
    "strips": ["strips.hip", "common.hpp", "params.hpp", "../build.py"],
}


def stage_source_sha(stage):
    import hashlib
    files = STAGE_SOURCES.get(stage)
    if not files:
        return None
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(_CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def recorded_traffic(stage, workload_name):
    """HBM bytes per launch recorded for `stage`, or None if absent or stale."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{stage}_{workload_name}.md")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            rec[k.strip()] = v.strip().strip("`")
    if rec.get("source_sha256") != stage_source_sha(stage):
        return None
    try:
        return int(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, slices=3):
    """The float64 oracle on a bounded sample of the same workload: the first
    ``slices`` heads of the first sequence, each one (sequence, head) slice."""
    import numpy as np
    from threadpoolctl import threadpool_info
    import oracle
    w = inp.workload
    L = inp.lengths[0]
    f = inp.f64
    sl = slice(0, L)
    n = min(slices, w.heads)
    t0 = time.perf_counter()
    for h in range(n):
        args = [f["q"][sl, h:h + 1], f["k"][sl, h:h + 1], f["v"][sl, h:h + 1], f["q_r"][h:h + 1],
                f["k_r"][h:h + 1]]
        oracle.forward(*args, w.span, w.buckets)
        oracle.backward(*args, f["dout"][sl, h:h + 1], w.span, w.buckets)
    dt = time.perf_counter() - t0
    threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    fl = n * flops_fwd_bwd(1, 1, L, w.head_dim, w.rows)
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "slices_timed": n, "slices_in_workload": inp.nseq * w.heads,
            "seconds_per_slice": round(dt / n, 3),
            "sample": f"float64 numpy oracle, forward then backward, {n} (sequence, head) slices "
                      f"of the workload (L={L}, D={w.head_dim}, R={w.rows}); {dt:.1f} s wall; "
                      f"scaled by the same FLOP convention"}


def dist(xs):
    """min / p10 / median / p90 of a list of per-call milliseconds."""
    xs = sorted(xs)

    def pct(q):
        return xs[min(len(xs) - 1, int(round(q * (len(xs) - 1))))]
    return {"n": len(xs), "min": round(xs[0], 4), "p10": round(pct(0.1), 4), "median": round(pct(0.5), 4),
            "p90": round(pct(0.9), 4)}


def per_call(fn, n):
    """Milliseconds of each of n calls, each between its own events."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(n):
        fn()
        evs[i + 1].record()
    torch.cuda.synchronize()
    return [evs[i].elapsed_time(evs[i + 1]) for i in range(n)]


def other_workload(df, n, dtype, backward, reps):
    """Throughput of the other workloads (parity cases of the same path): the
    L=512 bf16 forward, the packed varlen D=128 forward+backward and the
    L=8192 D=128 unbucketed stress forward+backward in fp16 and strict fp32.
    FLOPs by the same convention, per sequence with its own active row count;
    percent of the MFMA peak of the working dtype (bf16/fp16: 2516.6, fp32:
    157.3 TFLOP/s)."""
    import torch
    from synth import workload_inputs
    dev = torch.device("cuda", 0)
    inp = workload_inputs(n, dtype=dtype)
    w = inp.workload
    H, D = w.heads, w.head_dim
    t = {k_: v_.to(dev) for k_, v_ in inp.t.items()}
    km = None if inp.key_mask is None else torch.from_numpy(inp.key_mask).to(dev)
    cu = None if inp.cu_seqlens is None else torch.from_numpy(inp.cu_seqlens).to(dev)
    shape = df.make_shape(t["q"], inp.nseq, inp.max_seqlen)
    ws = torch.empty(max(df.workspace_size(0, shape, w.span, w.buckets),
                         df.workspace_size(1, shape, w.span, w.buckets)), dtype=torch.uint8, device=dev)
    out = torch.empty_like(t["q"])
    lse = torch.empty((H, t["q"].shape[0]), dtype=torch.float32, device=dev)
    grads = tuple(torch.empty_like(t[x]) for x in ("q", "k", "v", "q_r", "k_r"))
    kw = dict(key_mask=km, cu_seqlens=cu, max_seqlen=inp.max_seqlen, workspace=ws)

    def step():
        df.fwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets, out=out, lse=lse, **kw)
        if backward:
            df.bwd(t["q"], t["k"], t["v"], t["q_r"], t["k_r"], w.span, w.buckets, out, lse, t["dout"],
                   grads=grads, reuse_fwd_workspace=True, **kw)
    step()
    times = per_call(step, reps)
    fl = 0.0
    c2p, _ = df.build_rel_index(inp.max_seqlen, w.span, w.buckets, device=dev)
    for Lk in inp.lengths:
        # active rows at length Lk: distinct table values over |d| < Lk
        mid = inp.max_seqlen - 1
        r_k = int(torch.unique(c2p[mid - (Lk - 1): mid + Lk]).numel()) if Lk > 0 else 0
        per = 4.0 * Lk * Lk * D + 4.0 * Lk * r_k * D
        if backward:
            per += 10.0 * Lk * Lk * D + 12.0 * Lk * r_k * D
        fl += H * per
    d = dist(times)
    peak = PEAK_FP32_TFLOPS if (dtype or w.dtype) == "fp32" else PEAK_BF16_TFLOPS
    tf = fl / (d["median"] * 1e-3) / 1e12
    del ws, t, grads
    torch.cuda.empty_cache()
    return {"workload": w.name, "dtype": dtype or w.dtype, "passes": "fwd+bwd" if backward else "fwd",
            "tokens": int(inp.total_tokens), "sequences": int(inp.nseq), "heads": H, "head_dim": D,
            "rel_rows": w.rows, "ms": d, "tflops": round(tf, 2), "peak_tflops": round(peak, 1),
            "pct_peak": round(100.0 * tf / peak, 2)}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (for profiler runs)")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the other workloads' timings (for profiler runs)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB (3 times), "
                         "the reference for scaling memory counters to bytes")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(this path has no multi-GPU mode)", file=sys.stderr)
        return 2

    import torch
    import deberta_disentangled_attention_rel_amd as df
    from synth import workload_inputs

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda", 0)
    inp = workload_inputs(WORKLOAD)
    w = inp.workload
    B, L, H, D, R = inp.nseq, inp.max_seqlen, w.heads, w.head_dim, w.rows
    t = {k: v.to(dev) for k, v in inp.t.items()}
    q, k, v, dout = (t[n].view(B, L, H, D) for n in ("q", "k", "v", "dout"))
    q_r, k_r = t["q_r"], t["k_r"]
    shape = df.make_shape(q.view(B * L, H, D), B, L)
    ws_bytes = max(df.workspace_size(0, shape, w.span, w.buckets),
                   df.workspace_size(1, shape, w.span, w.buckets))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((H, B * L), dtype=torch.float32, device=dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
             torch.empty_like(q_r), torch.empty_like(k_r))

    # active relative rows (the page's R): distinct table entries reached at L
    c2p, _ = df.build_rel_index(L, w.span, w.buckets, device=dev)
    r_active = int(torch.unique(c2p).numel())

    def step():
        df.fwd(q, k, v, q_r, k_r, w.span, w.buckets, out=out, lse=lse, workspace=ws)
        # the backward reuses the forward's index tables and strips, which stay
        # in the shared workspace (DF_FLAG_BWD_REUSE_FWD)
        df.bwd(q, k, v, q_r, k_r, w.span, w.buckets, out, lse, dout, grads=grads, workspace=ws,
               reuse_fwd_workspace=True)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    df.profile_enable(True)
    df.profile_read()
    # one event per step boundary on the stream the library launches on
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record()
    for i in range(a.steps):
        step()
        marks[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stages = df.profile_read()
    df.profile_enable(False)
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(a.steps))

    def pct(xs, q):
        return xs[min(len(xs) - 1, int(round(q * (len(xs) - 1))))]

    # the two passes alone (outside the timed steps; the backward replays on
    # the last forward's output and LSE)
    def timed(fn, n):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # cold-cache steps: before each, a 512 MiB fill (twice the 256 MB MALL)
    # evicts L2 and MALL; each step is timed alone between its own events
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(min(a.steps, 10)):
        flush.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    cold.sort()
    del flush

    # the two passes alone, each call between its own events
    fwd_calls = per_call(lambda: df.fwd(q, k, v, q_r, k_r, w.span, w.buckets, out=out, lse=lse, workspace=ws),
                         a.steps)
    bwd_calls = per_call(lambda: df.bwd(q, k, v, q_r, k_r, w.span, w.buckets, out, lse, dout, grads=grads,
                                        workspace=ws, reuse_fwd_workspace=True), a.steps)
    fwd_ms = sum(fwd_calls) / len(fwd_calls)
    bwd_ms = sum(bwd_calls) / len(bwd_calls)
    # the backward on its own, recomputing the index tables and strips
    bwd_recompute_ms = timed(lambda: df.bwd(q, k, v, q_r, k_r, w.span, w.buckets, out, lse, dout,
                                            grads=grads, workspace=ws), a.steps)
    # the inference forward (no LSE), into its own output buffer
    out_inf = torch.empty_like(out)
    inf_ms = timed(lambda: df.fwd_inference(q, k, v, q_r, k_r, w.span, w.buckets, out=out_inf, workspace=ws),
                   a.steps)
    # a fwd+bwd step with attention dropout 0.1 (its own output buffers)
    lse_d = torch.empty_like(lse)

    def drop_step():
        df.fwd(q, k, v, q_r, k_r, w.span, w.buckets, out=out_inf, lse=lse_d, workspace=ws,
               dropout_p=0.1, seed=1234, offset=0)
        df.bwd(q, k, v, q_r, k_r, w.span, w.buckets, out_inf, lse_d, dout, grads=grads, workspace=ws,
               dropout_p=0.1, seed=1234, offset=0, reuse_fwd_workspace=True)
    drop_step()
    drop_ms = timed(drop_step, max(1, a.steps // 3))

    # the fused Q/K/V + relative projections that produce this workload's
    # inputs (hidden size H*D, relative rows R), timed on their own: not part
    # of the page's FLOP convention or of the step
    from synth import make_proj_inputs
    pin = make_proj_inputs(B * L, H * D, H, D, R, "bf16", seed=77)
    pt = {k_: v_.to(dev) for k_, v_ in pin.t.items()}
    pouts = df.qkv_proj(pt["x"], pt["w"], pt["bias"], pt["rel"], H, D)
    proj_ms = timed(lambda: df.qkv_proj(pt["x"], pt["w"], pt["bias"], pt["rel"], H, D, out=pouts), a.steps)
    proj_flops = 2.0 * B * L * (H * D) * 3 * H * D + 2.0 * R * (H * D) * 2 * H * D
    # and its backward (dx, dW, db, d_rel) for unit output gradients
    pg = torch.ones((B * L, 3, H, D), dtype=torch.bfloat16, device=dev)
    pr = torch.ones((H, R, D), dtype=torch.bfloat16, device=dev)
    pws = torch.empty(df.lib().df_qkv_proj_bwd_workspace_size(B * L, H * D, H, D, R, 0), dtype=torch.uint8,
                      device=dev)
    df.qkv_proj_bwd(pt["x"], pt["w"], pt["rel"], pg, pr, pr, H, D, workspace=pws)
    proj_bwd_ms = timed(lambda: df.qkv_proj_bwd(pt["x"], pt["w"], pt["rel"], pg, pr, pr, H, D, workspace=pws),
                        a.steps)
    del pt, pouts, pg, pr, pws

    # the other workloads, unless skipped (profiler runs)
    others = []
    if not a.headline_only:
        del ws, grads, out, out_inf, lse_d
        torch.cuda.empty_cache()
        for n_, dt_, bw_, reps in ((2, None, False, 20), (4, None, True, 10), (5, "fp16", True, 5),
                                   (5, "fp32", True, 3)):
            others.append(other_workload(df, n_, dt_, bw_, reps))

    ms = (t1 - t0) * 1e3 / a.steps
    fl = flops_fwd_bwd(B, H, L, D, r_active)
    tflops = fl / (ms * 1e-3) / 1e12
    kern = {n: {"ms_per_launch": round(tot / cnt, 4), "launches_per_step": cnt / a.steps}
            for n, (tot, cnt) in stages.items() if cnt > 0}
    dom = max((n for n in kern if kernel_algorithmic_flops(n, B, H, L, D, R) is not None),
              key=lambda n: stages[n][0])
    dom_ms = stages[dom][0] / stages[dom][1]
    dom_tf = kernel_algorithmic_flops(dom, B, H, L, D, R) / (dom_ms * 1e-3) / 1e12
    bound = "mfma"
    if a.calib_copy_mib > 0:
        nbytes = a.calib_copy_mib << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    line = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(PAGES_H200_FWD_BWD_MS / ms, 3),
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "seq_len": L, "heads": H, "head_dim": D,
                   "tokens": B * L, "layout": "padded", "position_buckets": w.buckets,
                   "max_relative_positions": w.span, "rel_rows": R, "rel_rows_active": r_active},
        "pct_mfma_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "step_ms": {"min": round(per_step[0], 4), "p10": round(pct(per_step, 0.1), 4),
                    "median": round(pct(per_step, 0.5), 4), "p90": round(pct(per_step, 0.9), 4)},
        "step_ms_cold_cache": {"n": len(cold), "min": round(cold[0], 4), "p10": round(pct(cold, 0.1), 4),
                               "median": round(pct(cold, 0.5), 4), "p90": round(pct(cold, 0.9), 4),
                               "max": round(cold[-1], 4)},
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        "fwd_ms_dist": dist(fwd_calls),
        "bwd_ms_dist": dist(bwd_calls),
        "bwd_recompute_ms": round(bwd_recompute_ms, 4),
        "bwd_reuses_fwd_strips": True,
        "inference_fwd_ms": round(inf_ms, 4),
        "dropout_0.1_step_ms": round(drop_ms, 4),
        "qkv_proj": {"ms": round(proj_ms, 4), "tflops": round(proj_flops / (proj_ms * 1e-3) / 1e12, 1),
                     "bwd_ms": round(proj_bwd_ms, 4),
                     "bwd_tflops": round(2 * proj_flops / (proj_bwd_ms * 1e-3) / 1e12, 1),
                     "shape": f"x [{B * L}, {H * D}] w [{3 * H * D}, {H * D}] rel [{R}, {H * D}]"},
        "roofline": {"kernel": dom, "bound": bound, "achieved": round(dom_tf, 2),
                     "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(dom_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(dom, w.name)},
        "kernels": kern,
        "other_workloads": others,
        "device": torch.cuda.get_device_properties(dev).name,
        "cus": torch.cuda.get_device_properties(dev).multi_processor_count,
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
