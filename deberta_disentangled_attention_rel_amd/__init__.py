"""Exact disentangled (C2P/P2C) self-attention on AMD gfx950.

A thin ctypes binding of ``libdf_attn.so`` (declared in ``include/df_attn.h``).
It only marshals arguments: every step of the computation runs in the HIP
kernels of the library. PyTorch supplies device memory and the current
stream. If the library is missing, every call raises; there is no fallback.

Layouts: ``q, k, v, out, dout`` and their gradients are ``[T, H, D]`` (packed,
with ``cu_seqlens``) or ``[B, L, H, D]`` (padded); ``q_r, k_r`` are
``[H, R, D]``; ``lse`` is float32 ``[H, T]``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["lib", "Shape", "build_rel_index", "workspace_size", "supported", "fwd", "fwd_inference", "bwd",
           "rel_rows",
           "qkv_proj", "qkv_proj_bwd", "pack_padded", "unpack_packed",
           "profile_enable", "profile_read", "DfError", "DTYPE_CODES", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdf_attn.so")
DTYPE_CODES = {torch.bfloat16: 0, torch.float16: 1, torch.float32: 2}

EXPORTED = ("df_attn_supported", "df_attn_workspace_size", "df_build_rel_index",
            "df_attn_fwd", "df_attn_fwd_inference", "df_attn_bwd", "df_attn_fwd_dropout",
            "df_attn_bwd_dropout", "df_strerror", "df_last_error",
            "df_attn_version",
            "df_attn_profile_enable", "df_attn_profile_read", "df_attn_stage_name", "df_qkv_proj",
            "df_pack_padded", "df_unpack_packed", "df_qkv_proj_bwd", "df_qkv_proj_bwd_workspace_size",
            "df_attn_fwd_noalloc")
NUM_STAGES = 9


class DfError(RuntimeError):
    """An error code returned by the library."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"df_attn error {code}: {msg}")
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("max_seqlen", ctypes.c_int32),
                ("total_tokens", ctypes.c_int64), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("tok_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
                ("p2c_convention", ctypes.c_int32), ("flags", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m deberta_disentangled_attention_rel_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sp = ctypes.POINTER(Shape)
    L.df_attn_supported.argtypes = [sp, i32, i32]
    L.df_attn_supported.restype = ctypes.c_int
    L.df_attn_workspace_size.argtypes = [ctypes.c_int, sp, i32, i32]
    L.df_attn_workspace_size.restype = sz
    L.df_build_rel_index.argtypes = [i32, i32, i32, vp, vp, vp]
    L.df_build_rel_index.restype = ctypes.c_int
    L.df_attn_fwd.argtypes = [sp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    L.df_attn_fwd.restype = ctypes.c_int
    L.df_attn_fwd_inference.argtypes = [sp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, sz, vp]
    L.df_attn_fwd_inference.restype = ctypes.c_int
    L.df_attn_fwd_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp]
    L.df_attn_fwd_noalloc.restype = ctypes.c_int
    f32, u64, u32 = ctypes.c_float, ctypes.c_uint64, ctypes.c_uint32
    L.df_attn_fwd_dropout.argtypes = [sp, vp, vp, vp, vp, vp, i32, i32, vp, vp, f32, u64, u32, vp, vp, vp, sz, vp]
    L.df_attn_fwd_dropout.restype = ctypes.c_int
    L.df_attn_bwd_dropout.argtypes = [sp, vp, vp, vp, vp, vp, i32, i32, vp, vp, f32, u64, u32, vp, vp, vp,
                                      vp, vp, vp, vp, vp, vp, sz, vp]
    L.df_attn_bwd_dropout.restype = ctypes.c_int
    L.df_attn_bwd.argtypes = [sp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp,
                              vp, vp, vp, vp, vp, vp, sz, vp]
    L.df_attn_bwd.restype = ctypes.c_int
    L.df_qkv_proj.argtypes = [ctypes.c_int64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.df_qkv_proj.restype = ctypes.c_int
    L.df_qkv_proj_bwd_workspace_size.argtypes = [ctypes.c_int64, i32, i32, i32, i32, i32]
    L.df_qkv_proj_bwd_workspace_size.restype = ctypes.c_size_t
    L.df_qkv_proj_bwd.argtypes = [ctypes.c_int64, i32, i32, i32, i32, i32] + [vp] * 10 + [vp, sz, vp]
    L.df_qkv_proj_bwd.restype = ctypes.c_int
    L.df_pack_padded.argtypes = [i32, i32, ctypes.c_int64, vp, vp, vp, vp, vp, vp]
    L.df_pack_padded.restype = ctypes.c_int
    L.df_unpack_packed.argtypes = [i32, i32, ctypes.c_int64, vp, vp, vp, vp, vp]
    L.df_unpack_packed.restype = ctypes.c_int
    L.df_strerror.argtypes = [ctypes.c_int]
    L.df_strerror.restype = ctypes.c_char_p
    L.df_last_error.argtypes = []
    L.df_last_error.restype = ctypes.c_char_p
    L.df_attn_version.argtypes = []
    L.df_attn_version.restype = ctypes.c_int
    L.df_attn_profile_enable.argtypes = [ctypes.c_int]
    L.df_attn_profile_enable.restype = ctypes.c_int
    L.df_attn_profile_read.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int),
                                       ctypes.c_int]
    L.df_attn_profile_read.restype = ctypes.c_int
    L.df_attn_stage_name.argtypes = [ctypes.c_int]
    L.df_attn_stage_name.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(rc: int) -> None:
    if rc != 0:
        L = lib()
        raise DfError(rc, f"{L.df_strerror(rc).decode()}: {L.df_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _as_thd(x: torch.Tensor) -> torch.Tensor:
    """View ``[B, L, H, D]`` as ``[B*L, H, D]`` (no copy when possible)."""
    if x.dim() == 4:
        return x.reshape(x.shape[0] * x.shape[1], x.shape[2], x.shape[3])
    if x.dim() != 3:
        raise ValueError(f"expected [T,H,D] or [B,L,H,D], got {tuple(x.shape)}")
    return x


P2C_CONVENTIONS = {"literal": 0, "shared": 1}


FLAG_BWD_REUSE_FWD = 1


def make_shape(q: torch.Tensor, batch: int, max_seqlen: int, p2c: str = "literal", flags: int = 0) -> Shape:
    T, H, D = q.shape
    if q.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if p2c not in P2C_CONVENTIONS:
        raise ValueError(f"p2c must be one of {sorted(P2C_CONVENTIONS)}")
    return Shape(int(batch), int(max_seqlen), int(T), int(H), int(D), DTYPE_CODES[q.dtype],
                 int(q.stride(0)), int(q.stride(1)), P2C_CONVENTIONS[p2c], int(flags))


def _layout(q, k, v, cu_seqlens, max_seqlen):
    """Common shape marshalling of fwd/bwd: returns ([T,H,D] views, batch, L)."""
    padded4 = q.dim() == 4
    if cu_seqlens is not None:
        if max_seqlen is None:
            raise ValueError("packed layout needs max_seqlen")
        batch, L = cu_seqlens.numel() - 1, int(max_seqlen)
    elif padded4:
        batch, L = q.shape[0], q.shape[1]
    else:
        if max_seqlen is None:
            raise ValueError("[T,H,D] without cu_seqlens needs max_seqlen (= L)")
        L = int(max_seqlen)
        batch = q.shape[0] // L
    q3, k3, v3 = (_as_thd(x).contiguous() for x in (q, k, v))
    return q3, k3, v3, batch, L


def rel_rows(span: int, buckets: int) -> int:
    """R = 2 * att, att = buckets if buckets > 0 else span: the row count that
    q_r, k_r, dq_r and dk_r must have."""
    return 2 * (int(buckets) if int(buckets) > 0 else int(span))


def _check_args(q3, k3, v3, q_r, k_r, span, buckets, key_mask, cu_seqlens):
    """Reject, before any library call, tensors whose raw pointers the
    kernels would read with a shape, dtype or device other than the one the
    shape block describes (the C ABI cannot see tensor metadata)."""
    if q3.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {q3.dtype}")
    for name, t in (("k", k3), ("v", v3)):
        if t.shape != q3.shape or t.dtype != q3.dtype or t.device != q3.device:
            raise ValueError(f"{name} must match q in shape, dtype and device "
                             f"({tuple(t.shape)} {t.dtype} {t.device} vs {tuple(q3.shape)} {q3.dtype} {q3.device})")
    T, H, D = q3.shape
    R = rel_rows(span, buckets)
    for name, t in (("q_r", q_r), ("k_r", k_r)):
        if t.shape != (H, R, D) or t.dtype != q3.dtype or t.device != q3.device:
            raise ValueError(f"{name} must be [H, R, D] = {(H, R, D)} (R = 2*att for span {span}, buckets {buckets})"
                             f" in q's dtype and device, got {tuple(t.shape)} {t.dtype} {t.device}")
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.device != q3.device:
            raise ValueError(f"cu_seqlens must be a 1-D int32 tensor on {q3.device}, got "
                             f"{cu_seqlens.dtype} {tuple(cu_seqlens.shape)} {cu_seqlens.device}")
        if not cu_seqlens.is_contiguous() or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be contiguous with batch + 1 >= 2 entries")
    if key_mask is not None:
        if key_mask.dtype not in (torch.uint8, torch.bool) or key_mask.device != q3.device:
            raise ValueError(f"key_mask must be uint8 or bool on {q3.device}, got {key_mask.dtype} {key_mask.device}")
        if key_mask.numel() != T or not key_mask.is_contiguous():
            raise ValueError(f"key_mask must be contiguous with T = {T} elements, got {key_mask.numel()}")


def _require_gpu(q3):
    if q3.device.type != "cuda":
        raise ValueError(f"q, k, v must be on a GPU device, got {q3.device}")


def _check_lse(lse, q3):
    T, H, _ = q3.shape
    if lse.dtype != torch.float32 or lse.shape != (H, T) or not lse.is_contiguous() or lse.device != q3.device:
        raise ValueError(f"lse must be a contiguous float32 [H, T] = {(H, T)} tensor on {q3.device}, got "
                         f"{lse.dtype} {tuple(lse.shape)} {lse.device}")


def profile_enable(on: bool) -> None:
    """Turn per-launch HIP event timing inside the library on or off."""
    _check(lib().df_attn_profile_enable(1 if on else 0))


def profile_read() -> dict:
    """``{stage_name: (total_ms, launches)}`` since the last read (waits for the events)."""
    ms = (ctypes.c_float * NUM_STAGES)()
    n = (ctypes.c_int * NUM_STAGES)()
    _check(lib().df_attn_profile_read(ms, n, NUM_STAGES))
    L = lib()
    return {L.df_attn_stage_name(i).decode(): (float(ms[i]), int(n[i])) for i in range(NUM_STAGES)}


def build_rel_index(max_seqlen: int, span: int, buckets: int, device="cuda"):
    """The two relative-index tables (int32, ``2*max_seqlen - 1`` entries)."""
    n = 2 * int(max_seqlen) - 1
    c2p = torch.empty(n, dtype=torch.int32, device=device)
    p2c = torch.empty(n, dtype=torch.int32, device=device)
    _check(lib().df_build_rel_index(int(max_seqlen), int(span), int(buckets), _ptr(c2p), _ptr(p2c),
                                    _stream(c2p.device)))
    return c2p, p2c


def workspace_size(pass_: int, shape: Shape, span: int, buckets: int) -> int:
    return int(lib().df_attn_workspace_size(int(pass_), ctypes.byref(shape), int(span), int(buckets)))


def supported(shape: Shape, span: int, buckets: int) -> int:
    """0 if the configuration is accepted, else the error code (non-raising)."""
    return int(lib().df_attn_supported(ctypes.byref(shape), int(span), int(buckets)))


def _workspace(pass_, shape, span, buckets, device, workspace):
    need = workspace_size(pass_, shape, span, buckets)
    if need == 0:
        _check(supported(shape, span, buckets))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace


def fwd(q, k, v, q_r, k_r, span: int, buckets: int, key_mask=None, cu_seqlens=None,
        max_seqlen: Optional[int] = None, out=None, lse=None, workspace=None,
        dropout_p: float = 0.0, seed: int = 0, offset: int = 0, p2c: str = "literal"):
    """Forward pass. Returns ``(out, lse)`` with ``out`` shaped like ``q``.
    ``dropout_p > 0`` applies attention-probability dropout (mask from
    ``(seed, offset)``; pass the same values to ``bwd``). ``p2c`` is the P2C
    row convention: "literal" (delta(j, i)) or "shared" (the C2P row)."""
    q3, k3, v3, batch, L = _layout(q, k, v, cu_seqlens, max_seqlen)
    _require_gpu(q3)
    _check_args(q3, k3, v3, q_r, k_r, span, buckets, key_mask, cu_seqlens)
    shape = make_shape(q3, batch, L, p2c)
    T, H, D = q3.shape
    if out is None:
        out = torch.empty_like(q3)
    out3 = _as_thd(out)
    if out3.shape != q3.shape or not out3.is_contiguous() or out3.dtype != q3.dtype or out3.device != q3.device:
        raise ValueError("out must be a contiguous tensor shaped like q, in q's dtype and device")
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    _check_lse(lse, q3)
    ws = _workspace(0, shape, span, buckets, q.device, workspace)
    q_r, k_r = q_r.contiguous(), k_r.contiguous()
    if dropout_p:
        _check(lib().df_attn_fwd_dropout(ctypes.byref(shape), _ptr(q3), _ptr(k3), _ptr(v3), _ptr(q_r),
                                         _ptr(k_r), int(span), int(buckets), _ptr(key_mask),
                                         _ptr(cu_seqlens), float(dropout_p), int(seed), int(offset),
                                         _ptr(out3), _ptr(lse), _ptr(ws), ws.numel(), _stream(q.device)))
    else:
        _check(lib().df_attn_fwd(ctypes.byref(shape), _ptr(q3), _ptr(k3), _ptr(v3), _ptr(q_r), _ptr(k_r),
                                 int(span), int(buckets), _ptr(key_mask), _ptr(cu_seqlens),
                                 _ptr(out3), _ptr(lse), _ptr(ws), ws.numel(), _stream(q.device)))
    return out.view(q.shape) if q.dim() == 4 else out, lse


def fwd_inference(q, k, v, q_r, k_r, span: int, buckets: int, key_mask=None, cu_seqlens=None,
                  max_seqlen: Optional[int] = None, out=None, workspace=None, p2c: str = "literal"):
    """Inference forward (no LSE, nothing kept for a backward). Returns ``out``."""
    q3, k3, v3, batch, L = _layout(q, k, v, cu_seqlens, max_seqlen)
    _require_gpu(q3)
    _check_args(q3, k3, v3, q_r, k_r, span, buckets, key_mask, cu_seqlens)
    shape = make_shape(q3, batch, L, p2c)
    if out is None:
        out = torch.empty_like(q3)
    out3 = _as_thd(out)
    if out3.shape != q3.shape or not out3.is_contiguous() or out3.dtype != q3.dtype or out3.device != q3.device:
        raise ValueError("out must be a contiguous tensor shaped like q, in q's dtype and device")
    ws = _workspace(0, shape, span, buckets, q.device, workspace)
    q_r, k_r = q_r.contiguous(), k_r.contiguous()
    _check(lib().df_attn_fwd_inference(ctypes.byref(shape), _ptr(q3), _ptr(k3), _ptr(v3), _ptr(q_r),
                                       _ptr(k_r), int(span), int(buckets), _ptr(key_mask),
                                       _ptr(cu_seqlens), _ptr(out3), _ptr(ws), ws.numel(),
                                       _stream(q.device)))
    return out.view(q.shape) if q.dim() == 4 else out


def bwd(q, k, v, q_r, k_r, span: int, buckets: int, out, lse, dout, key_mask=None,
        cu_seqlens=None, max_seqlen: Optional[int] = None, grads=None, workspace=None,
        dropout_p: float = 0.0, seed: int = 0, offset: int = 0, p2c: str = "literal",
        reuse_fwd_workspace: bool = False):
    """Backward pass. Returns ``(dq, dk, dv, dq_r, dk_r)``. The dropout
    arguments and ``p2c`` must be those of the forward that produced ``out``.
    ``reuse_fwd_workspace``: ``workspace`` is the buffer that forward used
    (sized for the backward) and still holds its index tables and strips
    (DF_FLAG_BWD_REUSE_FWD)."""
    q3, k3, v3, batch, L = _layout(q, k, v, cu_seqlens, max_seqlen)
    _require_gpu(q3)
    _check_args(q3, k3, v3, q_r, k_r, span, buckets, key_mask, cu_seqlens)
    _check_lse(lse, q3)
    if reuse_fwd_workspace and workspace is None:
        raise ValueError("reuse_fwd_workspace needs the forward's workspace")
    shape = make_shape(q3, batch, L, p2c, FLAG_BWD_REUSE_FWD if reuse_fwd_workspace else 0)
    out3, dout3 = _as_thd(out).contiguous(), _as_thd(dout).contiguous()
    for name, t in (("out", out3), ("dout", dout3)):
        if t.shape != q3.shape or t.dtype != q3.dtype or t.device != q3.device:
            raise ValueError(f"{name} must be shaped like q, in q's dtype and device")
    if grads is None:
        grads = (torch.empty_like(q3), torch.empty_like(k3), torch.empty_like(v3),
                 torch.empty_like(q_r), torch.empty_like(k_r))
    dq, dk, dv, dq_r, dk_r = grads
    for g_ in (dq, dk, dv):
        if _as_thd(g_).shape != q3.shape or not g_.is_contiguous() or g_.dtype != q3.dtype or g_.device != q3.device:
            raise ValueError("dq, dk, dv must be contiguous tensors shaped like q, in q's dtype and device")
    for g_ in (dq_r, dk_r):
        if g_.shape != q_r.shape or not g_.is_contiguous() or g_.dtype != q3.dtype or g_.device != q3.device:
            raise ValueError("dq_r, dk_r must be contiguous tensors shaped like q_r ([H, R, D]), in q's dtype")
    ws = _workspace(1, shape, span, buckets, q.device, workspace)
    q_r, k_r = q_r.contiguous(), k_r.contiguous()
    if dropout_p:
        _check(lib().df_attn_bwd_dropout(ctypes.byref(shape), _ptr(q3), _ptr(k3), _ptr(v3), _ptr(q_r),
                                         _ptr(k_r), int(span), int(buckets), _ptr(key_mask),
                                         _ptr(cu_seqlens), float(dropout_p), int(seed), int(offset),
                                         _ptr(out3), _ptr(lse), _ptr(dout3), _ptr(_as_thd(dq)),
                                         _ptr(_as_thd(dk)), _ptr(_as_thd(dv)), _ptr(dq_r), _ptr(dk_r),
                                         _ptr(ws), ws.numel(), _stream(q.device)))
    else:
        _check(lib().df_attn_bwd(ctypes.byref(shape), _ptr(q3), _ptr(k3), _ptr(v3), _ptr(q_r), _ptr(k_r),
                                 int(span), int(buckets), _ptr(key_mask), _ptr(cu_seqlens),
                                 _ptr(out3), _ptr(lse), _ptr(dout3), _ptr(_as_thd(dq)), _ptr(_as_thd(dk)),
                                 _ptr(_as_thd(dv)), _ptr(dq_r), _ptr(dk_r), _ptr(ws), ws.numel(),
                                 _stream(q.device)))
    if q.dim() == 4:
        dq, dk, dv = (x.view(q.shape) for x in (dq, dk, dv))
    return dq, dk, dv, dq_r, dk_r


def qkv_proj(x, w, bias, rel, num_heads: int, head_dim: int, out=None):
    """Fused Q/K/V and relative-position projections (``df_qkv_proj``).

    ``x`` [T, E], ``w`` [3*H*D, E] (rows W_q, W_k, W_v), ``bias`` [3*H*D] or
    None, ``rel`` [R, E] or None. Returns ``(q, k, v, q_r, k_r)``: q, k, v
    contiguous [T, H, D], q_r, k_r [H, R, D] (None without ``rel``)."""
    H, D = int(num_heads), int(head_dim)
    T, E = x.shape
    if w.shape != (3 * H * D, E) or w.dtype != x.dtype or (bias is not None and bias.shape != (3 * H * D,)):
        raise ValueError("w must be [3*H*D, E] and bias [3*H*D], in x's dtype")
    if x.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("df_qkv_proj takes bf16 or fp16")
    x, w = x.contiguous(), w.contiguous()
    bias = bias.contiguous() if bias is not None else None
    R = 0 if rel is None else rel.shape[0]
    if rel is not None:
        if rel.shape[1] != E or rel.dtype != x.dtype:
            raise ValueError("rel must be [R, E] in x's dtype")
        rel = rel.contiguous()
    if out is None:
        q, k, v = (torch.empty((T, H, D), dtype=x.dtype, device=x.device) for _ in range(3))
        q_r, k_r = ((torch.empty((H, R, D), dtype=x.dtype, device=x.device) for _ in range(2))
                    if rel is not None else (None, None))
    else:
        q, k, v, q_r, k_r = out
    _check(lib().df_qkv_proj(T, E, H, D, R, DTYPE_CODES[x.dtype], _ptr(x), _ptr(w), _ptr(bias), _ptr(rel),
                             _ptr(q), _ptr(k), _ptr(v), _ptr(q_r), _ptr(k_r), _stream(x.device)))
    return q, k, v, q_r, k_r


def pack_padded(padded, mask):
    """Right-padded ``[B, L, ...]`` rows and a ``[B, L]`` mask (nonzero =
    valid) to packed ``[T, ...]`` rows (``df_pack_padded``). Returns
    ``(packed, cu_seqlens, max_seqlen)``; reading T and max_seqlen back to the
    host synchronises the stream."""
    B, L = mask.shape
    if padded.shape[:2] != (B, L):
        raise ValueError("padded must be [B, L, ...] like mask")
    padded = padded.contiguous()
    m8 = mask.to(torch.uint8).contiguous()
    row_bytes = padded[0, 0].numel() * padded.element_size()
    packed = torch.empty((B * L,) + tuple(padded.shape[2:]), dtype=padded.dtype, device=padded.device)
    cu = torch.empty(B + 1, dtype=torch.int32, device=padded.device)
    mx = torch.empty(1, dtype=torch.int32, device=padded.device)
    _check(lib().df_pack_padded(B, L, row_bytes, _ptr(padded), _ptr(m8), _ptr(packed), _ptr(cu), _ptr(mx),
                                _stream(padded.device)))
    T = int(cu[-1].item())
    return packed[:T], cu, int(mx.item())


def unpack_packed(packed, cu_seqlens, mask):
    """Packed ``[T, ...]`` rows back to ``[B, L, ...]`` (zeros at invalid
    positions) for the mask they were packed with (``df_unpack_packed``)."""
    B, L = mask.shape
    packed = packed.contiguous()
    m8 = mask.to(torch.uint8).contiguous()
    row_bytes = packed[0].numel() * packed.element_size() if packed.shape[0] else \
        int(torch.tensor(packed.shape[1:]).prod().item()) * packed.element_size()
    out = torch.empty((B, L) + tuple(packed.shape[1:]), dtype=packed.dtype, device=packed.device)
    src = packed if packed.shape[0] else torch.empty((1,) + tuple(packed.shape[1:]), dtype=packed.dtype,
                                                     device=packed.device)
    _check(lib().df_unpack_packed(B, L, row_bytes, _ptr(src), _ptr(m8), _ptr(cu_seqlens.contiguous()), _ptr(out),
                                  _stream(packed.device)))
    return out


def qkv_proj_bwd(x, w, rel, dqkv, dq_r=None, dk_r=None, num_heads: int = 1, head_dim: int = 64,
                 workspace=None):
    """Backward of :func:`qkv_proj` (``df_qkv_proj_bwd``). ``dqkv`` is the
    output gradient as one ``[T, 3, H, D]`` (or ``[T, 3*H*D]``) tensor;
    ``dq_r``, ``dk_r`` ``[H, R, D]`` when ``rel`` is given. Returns
    ``(dx, dw, db, drel)`` (``drel`` None without ``rel``)."""
    H, D = int(num_heads), int(head_dim)
    T, E = x.shape
    if x.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("df_qkv_proj_bwd takes bf16 or fp16")
    dqkv = dqkv.reshape(T, 3 * H * D).contiguous()
    x, w = x.contiguous(), w.contiguous()
    R = 0 if rel is None else rel.shape[0]
    if rel is not None:
        rel, dq_r, dk_r = rel.contiguous(), dq_r.contiguous(), dk_r.contiguous()
    dt = DTYPE_CODES[x.dtype]
    need = lib().df_qkv_proj_bwd_workspace_size(T, E, H, D, R, dt)
    if need == 0:
        raise DfError(1, "invalid projection shape")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    dx = torch.empty_like(x)
    dw = torch.empty_like(w)
    db = torch.empty(3 * H * D, dtype=x.dtype, device=x.device)
    drel = torch.empty_like(rel) if rel is not None else None
    _check(lib().df_qkv_proj_bwd(T, E, H, D, R, dt, _ptr(x), _ptr(w), _ptr(rel), _ptr(dqkv), _ptr(dq_r),
                                 _ptr(dk_r), _ptr(dx), _ptr(dw), _ptr(db), _ptr(drel), _ptr(workspace),
                                 workspace.numel(), _stream(x.device)))
    return dx, dw, db, drel
