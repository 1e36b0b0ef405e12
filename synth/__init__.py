"""Seeded synthetic inputs for disentangled attention.

This module is shared by the tests, the benchmark and the smoke check. It
draws random tensors and builds the structure of a workload (sequence lengths,
padding masks); it holds none of the attention arithmetic. Both the GPU path
and the CPU oracle consume what it returns.

Recipe (each workload's shape follows the DisentangledFlash 1.1.1 page,
"Status" and "Performance" sections: head dims 32/64/128, bf16/fp16/fp32,
factorized padding masks, packed ``cu_seqlens`` layouts, and the 12-head,
head-dim-64, 16,384-token L=8192 measurement):

* one ``numpy.random.default_rng(seed)`` (PCG64) stream per workload;
* for packed workloads the sequence lengths are drawn first: integers uniform
  in ``[lo, hi]`` until their sum reaches the token budget, the last one cut
  to the remainder;
* then, in this order, q, k, v (each ``[T, H, D]``), q_r, k_r (each
  ``[H, R, D]``) and dout (``[T, H, D]``) are drawn in float64 from
  ``N(0, std^2)`` (``std = 1`` or ``1/sqrt(D)``; dout always ``N(0, 1)``);
* every tensor is rounded once to the working dtype with torch's
  round-to-nearest-even cast; the float64 copies handed to the oracle are the
  already-rounded values, so both sides see identical inputs;
* a padding mask, when present, is right padding: the trailing
  ``floor(frac * L_k)`` tokens of each sequence are marked invalid.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and structure of one synthetic workload.

    ``rows`` is the number of relative-position rows of q_r / k_r; it is
    stated here as data (it is twice ``buckets`` when bucketing is on, else
    twice ``span``) so that this module carries no index arithmetic.
    """

    name: str
    heads: int
    head_dim: int
    dtype: str
    span: int
    buckets: int
    rows: int
    seed: int
    batch: int = 1              # padded layout: number of sequences
    seqlen: int = 0             # padded layout: L
    packed_tokens: int = 0      # packed layout: total token budget (0 = padded)
    len_range: tuple = (0, 0)   # packed layout: inclusive length range
    mask_frac: float = 0.0      # trailing fraction of each sequence masked
    std: str = "inv_sqrt_d"     # "unit" or "inv_sqrt_d" for q, k, v, q_r, k_r
    passes: tuple = ("fwd", "bwd")

    @property
    def packed(self) -> bool:
        return self.packed_tokens > 0


# The five workloads the throughput and parity suites are built around.
WORKLOADS = {
    1: Workload("tiny_fp32_L64", heads=2, head_dim=32, dtype="fp32", span=32,
                buckets=0, rows=64, seed=1001, batch=1, seqlen=64, std="unit",
                passes=("fwd",)),
    2: Workload("bf16_fwd_L512", heads=12, head_dim=64, dtype="bf16", span=512,
                buckets=256, rows=512, seed=1002, batch=32, seqlen=512,
                passes=("fwd",)),
    3: Workload("bf16_fwdbwd_L8192_H12_D64", heads=12, head_dim=64, dtype="bf16",
                span=512, buckets=256, rows=512, seed=1003, batch=2,
                seqlen=8192),
    4: Workload("packed_varlen_H16_D128", heads=16, head_dim=128, dtype="bf16",
                span=512, buckets=256, rows=512, seed=1004,
                packed_tokens=16384, len_range=(64, 2048), mask_frac=0.1),
    5: Workload("det_stress_L8192_H16_D128", heads=16, head_dim=128,
                dtype="fp16", span=512, buckets=0, rows=1024, seed=1005,
                batch=2, seqlen=8192),
}


def packed_lengths(rng: np.random.Generator, total: int, lo: int, hi: int) -> list:
    """Uniform integer lengths in [lo, hi] until ``total`` tokens; last one cut."""
    lens = []
    acc = 0
    while acc < total:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, total - acc)
        lens.append(n)
        acc += n
    return lens


@dataclasses.dataclass
class Inputs:
    """One set of inputs, as working-dtype torch tensors and float64 copies."""

    workload: Workload
    dtype: str
    lengths: list               # per-sequence lengths
    cu_seqlens: Optional[np.ndarray]   # int32 [nseq+1] for packed, else None
    key_mask: Optional[np.ndarray]     # uint8 [T] (1 = valid) or None
    t: dict                     # name -> torch tensor (CPU, working dtype)
    f64: dict                   # name -> numpy float64 (rounded values)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lengths))

    @property
    def max_seqlen(self) -> int:
        return int(max(self.lengths))

    @property
    def nseq(self) -> int:
        return len(self.lengths)


def _round(x64: np.ndarray, dtype: str) -> tuple:
    t = torch.from_numpy(x64).to(DTYPES[dtype])
    return t, t.to(torch.float64).numpy()


def make_inputs(heads: int, head_dim: int, dtype: str, span: int, buckets: int,
                rows: int, seed: int, *, batch: int = 1, seqlen: int = 0,
                lengths: Optional[Sequence[int]] = None, packed: bool = False,
                mask_frac: float = 0.0, std: str = "inv_sqrt_d",
                with_dout: bool = True, name: str = "custom") -> Inputs:
    """Draw one input set.

    Padded layout: ``batch`` sequences of ``seqlen`` tokens (``lengths`` unused).
    Packed layout (``packed=True``): explicit ``lengths``.
    """
    rng = np.random.default_rng(seed)
    if packed:
        assert lengths is not None and len(lengths) > 0
        lens = [int(n) for n in lengths]
    else:
        lens = [int(seqlen)] * int(batch)
    T = int(sum(lens))
    H, D, R = int(heads), int(head_dim), int(rows)
    sd = 1.0 if std == "unit" else 1.0 / math.sqrt(D)
    t, f = {}, {}
    for nm, shape, scale in (("q", (T, H, D), sd), ("k", (T, H, D), sd),
                             ("v", (T, H, D), sd), ("q_r", (H, R, D), sd),
                             ("k_r", (H, R, D), sd)):
        t[nm], f[nm] = _round(rng.standard_normal(shape) * scale, dtype)
    if with_dout:
        t["dout"], f["dout"] = _round(rng.standard_normal((T, H, D)), dtype)
    key_mask = None
    if mask_frac > 0.0:
        key_mask = np.ones(T, dtype=np.uint8)
        st = 0
        for n in lens:
            nm = int(math.floor(mask_frac * n))
            if nm > 0:
                key_mask[st + n - nm: st + n] = 0
            st += n
    cu = None
    if packed:
        cu = np.zeros(len(lens) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lens)
    wl = Workload(name, heads=H, head_dim=D, dtype=dtype, span=span,
                  buckets=buckets, rows=R, seed=seed, batch=len(lens),
                  seqlen=(0 if packed else int(seqlen)),
                  packed_tokens=(T if packed else 0), mask_frac=mask_frac,
                  std=std)
    return Inputs(wl, dtype, lens, cu, key_mask, t, f)


def workload_inputs(n: int, dtype: Optional[str] = None,
                    with_dout: bool = True) -> Inputs:
    """Inputs for workload ``n`` of :data:`WORKLOADS` (dtype may be overridden)."""
    w = WORKLOADS[n]
    dt = dtype or w.dtype
    if w.packed:
        rng = np.random.default_rng(w.seed)
        lens = packed_lengths(rng, w.packed_tokens, *w.len_range)
        # tensors come from a second stream so that the lengths stay fixed
        # whatever the tensor shapes are
        return make_inputs(w.heads, w.head_dim, dt, w.span, w.buckets, w.rows,
                           w.seed + 100000, lengths=lens, packed=True,
                           mask_frac=w.mask_frac, std=w.std,
                           with_dout=with_dout, name=w.name)
    return make_inputs(w.heads, w.head_dim, dt, w.span, w.buckets, w.rows,
                       w.seed, batch=w.batch, seqlen=w.seqlen,
                       mask_frac=w.mask_frac, std=w.std, with_dout=with_dout,
                       name=w.name)


@dataclasses.dataclass
class ProjInputs:
    """Inputs of the fused projections, as working-dtype torch tensors (CPU)
    and float64 copies of the rounded values."""

    tokens: int
    hidden: int
    heads: int
    head_dim: int
    rows: int
    dtype: str
    t: dict
    f64: dict


def make_proj_inputs(tokens: int, hidden: int, heads: int, head_dim: int, rows: int, dtype: str,
                     seed: int, *, bias: bool = True, rel: bool = True) -> ProjInputs:
    """Hidden states x ~ N(0, 1) [tokens, hidden], stacked weights
    w ~ N(0, 1/hidden) [3*heads*head_dim, hidden] (outputs of unit scale),
    bias ~ N(0, 0.1^2) and relative-position embedding rows rel ~ N(0, 1)
    [rows, hidden], drawn in float64 in that order and rounded once."""
    rng = np.random.default_rng(seed)
    N = 3 * heads * head_dim
    t, f = {}, {}
    specs = [("x", (tokens, hidden), 1.0), ("w", (N, hidden), 1.0 / math.sqrt(hidden))]
    if bias:
        specs.append(("bias", (N,), 0.1))
    if rel:
        specs.append(("rel", (rows, hidden), 1.0))
    for nm, shape, scale in specs:
        t[nm], f[nm] = _round(rng.standard_normal(shape) * scale, dtype)
    return ProjInputs(tokens, hidden, heads, head_dim, rows if rel else 0, dtype, t, f)
