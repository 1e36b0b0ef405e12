"""CPU tests of the C ABI (no GPU needed, no kernel launched).

* the library loads and exports every function declared in include/df_attn.h;
* every invalid argument is rejected on the host with the documented code
  before anything touches a device (fake, never-dereferenced pointers);
* the two properties of the relative-index tables that the kernels rely on
  hold for the oracle's tables: the far-field bound (both tables at their end
  rows exactly when |d| >= span) and the no-skip criterion for log buckets.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "df_attn.h")


@pytest.fixture(scope="module")
def df():
    import deberta_disentangled_attention_rel_amd as m
    if not os.path.exists(m.LIB_PATH):
        from deberta_disentangled_attention_rel_amd import build
        build.build()
    m.lib()
    return m


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(df_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_function(df):
    names = header_functions()
    assert "df_attn_fwd" in names and "df_attn_bwd" in names
    lib = ctypes.CDLL(df.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(df.EXPORTED)
    assert lib.df_attn_version() >= 100


def _shape(df, **kw):
    d = dict(batch=2, max_seqlen=128, total_tokens=256, num_heads=4, head_dim=64, dtype=0,
             tok_stride=256, head_stride=64)
    d.update(kw)
    return df.Shape(**d)


@pytest.mark.parametrize("kw,span,buckets,code", [
    (dict(), 512, 256, 0),
    (dict(), 32, 0, 0),
    (dict(head_dim=48), 512, 256, 2),
    (dict(head_dim=256), 512, 256, 2),
    (dict(dtype=3), 512, 256, 2),
    (dict(batch=0), 512, 256, 1),
    (dict(max_seqlen=0), 512, 256, 1),
    (dict(num_heads=0), 512, 256, 1),
    (dict(total_tokens=-1), 512, 256, 1),
    (dict(tok_stride=252), 512, 256, 1),          # not a multiple of 8
    (dict(head_stride=32), 512, 256, 1),          # rows overlap
    (dict(tok_stride=128), 512, 256, 1),          # heads overlap the next token
    (dict(), 0, 0, 1),                             # span must be >= 1
    (dict(), 512, 1, 1),                           # buckets must be 0 or >= 2
    (dict(), 100, 256, 1),                         # span - 1 <= buckets / 2
    (dict(), 512, -2, 1),
    (dict(p2c_convention=1), 512, 256, 0),
    (dict(p2c_convention=2), 512, 256, 1),         # unknown P2C convention
    (dict(flags=1), 512, 256, 0),
    (dict(flags=2), 512, 256, 1),                  # unknown flag
])
def test_supported_codes(df, kw, span, buckets, code):
    assert df.supported(_shape(df, **kw), span, buckets) == code


def test_workspace_sizes(df):
    s = _shape(df)
    w0, w1 = df.workspace_size(0, s, 512, 256), df.workspace_size(1, s, 512, 256)
    assert 0 < w0 < w1
    # forward: two tables, the packed table with 256 entries of padding on each
    # side, two strips [H][T][R] and four end columns, 256-byte aligned pieces
    T, H, R, L = 256, 4, 512, 128
    expect = [2 * (2 * L - 1) * 4, (2 * L - 1 + 2 * 256) * 4, H * T * R * 2, H * T * R * 2, 4 * H * T * 2]
    assert w0 == sum((x + 255) // 256 * 256 for x in expect)
    assert df.workspace_size(2, s, 512, 256) == 0
    # the shared P2C convention adds the reversed q_r [H][R][D]
    sh = _shape(df, p2c_convention=1)
    assert df.workspace_size(0, sh, 512, 256) == w0 + (H * R * 64 * 2 + 255) // 256 * 256
    assert df.workspace_size(0, _shape(df, head_dim=48), 512, 256) == 0


FAKE = 1 << 20  # 256-byte aligned, never dereferenced


def _fwd(df, shape, ptrs, ws_bytes=1 << 40, span=512, buckets=256, cu=None):
    L = df.lib()
    vp = [ctypes.c_void_p(x) if x else None for x in ptrs]
    return L.df_attn_fwd(ctypes.byref(shape), vp[0], vp[1], vp[2], vp[3], vp[4], span, buckets,
                         None, cu, vp[5], vp[6], ctypes.c_void_p(FAKE), ws_bytes, None)


def test_fwd_rejects_on_host(df):
    L = df.lib()
    s = _shape(df)
    ok = [FAKE] * 7
    for k in range(7):
        bad = list(ok)
        bad[k] = 0
        assert _fwd(df, s, bad) == 1
        assert "NULL" in L.df_last_error().decode()
    mis = list(ok)
    mis[0] = FAKE + 2                         # q misaligned
    assert _fwd(df, s, mis) == 1
    assert _fwd(df, s, ok, ws_bytes=1024) == 3
    assert "workspace" in L.df_last_error().decode()
    assert _fwd(df, _shape(df, total_tokens=200), ok) == 1   # padded T mismatch
    assert _fwd(df, _shape(df, head_dim=32, dtype=2), ok, span=0) == 1
    assert L.df_strerror(3).decode() == "workspace too small"


def test_fwd_inference_rejects_on_host(df):
    """The inference forward shares the forward's checks and takes no lse."""
    L = df.lib()
    s = _shape(df)
    vp = [ctypes.c_void_p(FAKE)] * 6

    def call(ptrs, ws_bytes=1 << 40, shape=s, span=512):
        return L.df_attn_fwd_inference(ctypes.byref(shape), *ptrs[:5], span, 256, None, None, ptrs[5],
                                       ctypes.c_void_p(FAKE), ws_bytes, None)
    for k in range(6):
        bad = list(vp)
        bad[k] = None
        assert call(bad) == 1
        assert "NULL" in L.df_last_error().decode()
    assert call(vp, ws_bytes=1024) == 3
    assert call(vp, shape=_shape(df, total_tokens=200)) == 1
    assert call(vp, span=0) == 1
    # the training forward still requires lse
    assert _fwd(df, s, [FAKE] * 6 + [0]) == 1
    assert "df_attn_fwd_inference" in L.df_last_error().decode()


def test_dropout_entry_points_reject_on_host(df):
    L = df.lib()
    s = _shape(df)
    vp = [ctypes.c_void_p(FAKE)] * 7
    for p in (1.0, -0.1, float("nan")):
        rc = L.df_attn_fwd_dropout(ctypes.byref(s), *vp[:5], 512, 256, None, None, p, 1, 0, vp[5], vp[6],
                                   ctypes.c_void_p(FAKE), 1 << 40, None)
        assert rc == 1 and "dropout" in L.df_last_error().decode()
    p15 = [ctypes.c_void_p(FAKE)] * 15
    rc = L.df_attn_bwd_dropout(ctypes.byref(s), *p15[:5], 512, 256, None, None, 1.5, 1, 0, *p15[5:13],
                               ctypes.c_void_p(FAKE), 1 << 40, None)
    assert rc == 1 and "dropout" in L.df_last_error().decode()
    rc = L.df_attn_fwd_dropout(ctypes.byref(s), *vp[:5], 512, 256, None, None, 0.1, 1, 0, vp[5], None,
                               ctypes.c_void_p(FAKE), 1 << 40, None)
    assert rc == 1
    # fp16 keeps 1 / (1 - p) <= 1000: the backward carries dP / (1 - p) in fp16 operands
    s16 = _shape(df, dtype=1)
    for fn, args in ((L.df_attn_fwd_dropout, [*vp[:5], 512, 256, None, None, 0.9995, 1, 0, vp[5], vp[6]]),
                     (L.df_attn_bwd_dropout, [*p15[:5], 512, 256, None, None, 0.9995, 1, 0, *p15[5:13]])):
        rc = fn(ctypes.byref(s16), *args, ctypes.c_void_p(FAKE), 1 << 40, None)
        assert rc == 2 and "fp16" in L.df_last_error().decode()


def test_bwd_and_index_reject_on_host(df):
    L = df.lib()
    s = _shape(df)
    p = [ctypes.c_void_p(FAKE)] * 15
    rc = L.df_attn_bwd(ctypes.byref(s), *p[:5], 512, 256, None, None, *p[5:8],
                       *p[8:13], ctypes.c_void_p(FAKE), 16, None)
    assert rc == 3
    rc = L.df_attn_bwd(ctypes.byref(s), *p[:5], 512, 256, None, None, *p[5:7], None,
                       *p[8:13], ctypes.c_void_p(FAKE), 1 << 40, None)
    assert rc == 1 and "dout" in L.df_last_error().decode()
    assert L.df_build_rel_index(0, 512, 256, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None) == 1
    assert L.df_build_rel_index(64, 512, 256, None, ctypes.c_void_p(FAKE), None) == 1
    assert L.df_build_rel_index(64, 100, 256, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None) == 1


def test_qkv_proj_rejects_on_host(df):
    L = df.lib()
    f = ctypes.c_void_p(FAKE)

    def call(T=64, E=64, H=2, D=32, R=8, dt=0, x=f, w=f, b=f, rel=f, outs=(f,) * 5):
        return L.df_qkv_proj(T, E, H, D, R, dt, x, w, b, rel, *outs, None)
    assert call(dt=2) == 2 and "16-bit" in L.df_last_error().decode()
    assert call(dt=7) == 2
    assert call(D=48) == 2
    assert call(H=0) == 1
    assert call(E=60) == 1 and "multiple of 8" in L.df_last_error().decode()
    assert call(T=-1) == 1
    assert call(x=None) == 1 and "x" in L.df_last_error().decode()
    assert call(w=None) == 1
    assert call(x=ctypes.c_void_p(FAKE + 8)) == 1          # x must be 16-byte aligned
    assert call(outs=(f, None, f, f, f)) == 1               # k missing
    assert call(rel=None) == 1                               # rel_rows > 0 without rel
    assert call(outs=(f, f, f, None, f)) == 1               # q_r missing while rel given
    assert call(T=1 << 30, H=1) == 2                         # token rows counted in 32 bits
    assert call(E=1 << 23) == 2                              # 128-row blocks of x past 2 GiB


def test_qkv_proj_bwd_rejects_on_host(df):
    L = df.lib()
    f = ctypes.c_void_p(FAKE)
    assert L.df_qkv_proj_bwd_workspace_size(64, 64, 2, 32, 8, 0) > 0
    assert L.df_qkv_proj_bwd_workspace_size(64, 64, 2, 32, 8, 2) == 0    # fp32
    assert L.df_qkv_proj_bwd_workspace_size(64, 60, 2, 32, 8, 0) == 0    # hidden % 8

    def call(T=64, E=64, H=2, D=32, R=8, dt=0, ptrs=(f,) * 10, ws=1 << 40):
        return L.df_qkv_proj_bwd(T, E, H, D, R, dt, *ptrs, f, ws, None)
    assert call(dt=2) == 2
    assert call(D=48) == 2
    p = list((f,) * 10)
    p[3] = None                                   # dqkv
    assert call(ptrs=tuple(p)) == 1 and "dqkv" in L.df_last_error().decode()
    p = list((f,) * 10)
    p[2] = None                                   # rel missing while rel_rows > 0
    assert call(ptrs=tuple(p)) == 1
    assert call(ws=1024) == 3
    assert call(T=1 << 23) == 2                              # transposed rows of 2^23 tokens
    assert L.df_qkv_proj_bwd_workspace_size(1 << 23, 64, 2, 32, 8, 0) == 0


def test_pack_helpers_reject_on_host(df):
    L = df.lib()
    f = ctypes.c_void_p(FAKE)
    assert L.df_pack_padded(0, 8, 16, f, f, f, f, None, None) == 1
    assert L.df_pack_padded(2, 0, 16, f, f, f, f, None, None) == 1
    assert L.df_pack_padded(2, 8, 24, f, f, f, f, None, None) == 1 and "multiple of 16" in L.df_last_error().decode()
    assert L.df_pack_padded(2, 8, 16, None, f, f, f, None, None) == 1
    assert L.df_pack_padded(2, 8, 16, f, f, ctypes.c_void_p(FAKE + 8), f, None, None) == 1
    assert L.df_pack_padded(2, 8, 16, f, f, f, None, None, None) == 1
    assert L.df_unpack_packed(2, 8, 16, f, None, f, f, None) == 1
    assert L.df_unpack_packed(1 << 16, 1 << 15, 16, f, f, f, f, None) == 1   # batch * max_len >= 2^31


def test_profile_api_without_enable(df):
    L = df.lib()
    ms = (ctypes.c_float * 9)()
    n = (ctypes.c_int * 9)()
    assert L.df_attn_profile_read(ms, n, 9) == 1
    assert L.df_attn_stage_name(4).decode() == "bwd_dkv"
    assert L.df_attn_stage_name(99).decode() == ""


# ----------------------------------------------------------------------------
# table properties the kernels rely on

CONFIGS = [(512, 256), (512, 0), (32, 0), (12, 8), (81, 10), (300, 256), (6, 4), (40, 16),
           (1, 0), (4, 2), (5, 3), (200, 64), (64, 32)]


@pytest.mark.parametrize("span,buckets", CONFIGS)
def test_far_field_bound(span, buckets):
    # both tables at their end rows exactly when |d| >= span (no far field when mid = 1)
    L = 700
    c2p, p2c = oracle.rel_luts(L, span, buckets)
    att, R = oracle.att_and_rows(span, buckets)
    d = np.arange(-(L - 1), L)
    left = (c2p == R - 1) & (p2c == 0)
    right = (c2p == 0) & (p2c == R - 1)
    if buckets > 0 and buckets // 2 < 2:
        assert not left.any() and not right.any()
        return
    assert np.array_equal(left, d >= span)
    assert np.array_equal(right, d <= -span)


@pytest.mark.parametrize("span,buckets", CONFIGS + [(260, 256), (200, 256), (131, 256), (400, 200)])
def test_narrow_criterion(span, buckets):
    # (mid-1) <= mid ln((span-1)/mid) implies no table ever steps by more than one row
    c2p, p2c = oracle.rel_luts(1500, span, buckets)
    steps = max(np.abs(np.diff(c2p)).max(), np.abs(np.diff(p2c)).max())
    mid = buckets // 2
    narrow = buckets == 0 or mid <= 1 or (mid - 1) / (mid * math.log((span - 1) / mid)) <= 1 - 1e-9
    if narrow:
        assert steps <= 1
    if buckets == 256 and span in (260, 200, 131):
        assert not narrow and steps > 1   # these really skip rows


# ---------------------------------------------------------------------------
# Binding-side checks: the C ABI sees only raw pointers, so the binding
# rejects tensors whose shape, dtype or device differ from what the shape
# block tells the kernels, before any library call.

def _cpu_args(T=64, H=2, D=32, span=32, buckets=0, dtype=None):
    import torch
    dtype = dtype or torch.bfloat16
    R = 2 * (buckets if buckets > 0 else span)
    q = torch.zeros(T, H, D, dtype=dtype)
    qr = torch.zeros(H, R, D, dtype=dtype)
    return dict(q3=q, k3=q.clone(), v3=q.clone(), q_r=qr, k_r=qr.clone(), span=span, buckets=buckets,
                key_mask=None, cu_seqlens=None)


def test_binding_accepts_consistent_args(df):
    import torch
    a = _cpu_args()
    df._check_args(**a)
    a["key_mask"] = torch.ones(64, dtype=torch.uint8)
    a["cu_seqlens"] = torch.tensor([0, 30, 64], dtype=torch.int32)
    df._check_args(**a)
    a["key_mask"] = torch.ones(64, dtype=torch.bool)
    df._check_args(**a)


@pytest.mark.parametrize("case", [
    "qr_rows_span", "kr_rows", "qr_dtype", "k_shape", "v_dtype", "cu_int64", "cu_2d", "mask_len",
    "mask_dtype", "bucket_rows"])
def test_binding_rejects_inconsistent_args(df, case):
    import torch
    a = _cpu_args()
    if case == "qr_rows_span":      # span rows instead of 2*att
        a["q_r"] = torch.zeros(2, 32, 32, dtype=torch.bfloat16)
    elif case == "kr_rows":
        a["k_r"] = torch.zeros(2, 66, 32, dtype=torch.bfloat16)
    elif case == "qr_dtype":
        a["q_r"] = a["q_r"].to(torch.float16)
    elif case == "k_shape":
        a["k3"] = torch.zeros(64, 2, 64, dtype=torch.bfloat16)
    elif case == "v_dtype":
        a["v3"] = a["v3"].float()
    elif case == "cu_int64":        # torch's default integer type
        a["cu_seqlens"] = torch.tensor([0, 30, 64])
    elif case == "cu_2d":
        a["cu_seqlens"] = torch.tensor([[0, 30, 64]], dtype=torch.int32)
    elif case == "mask_len":
        a["key_mask"] = torch.ones(63, dtype=torch.uint8)
    elif case == "mask_dtype":
        a["key_mask"] = torch.ones(64, dtype=torch.int32)
    elif case == "bucket_rows":     # buckets 16 need R = 32 rows, q_r has 64
        a["buckets"] = 16
    with pytest.raises(ValueError):
        df._check_args(**a)


def test_binding_rejects_host_tensors_and_bad_lse(df):
    import torch
    a = _cpu_args()
    with pytest.raises(ValueError, match="GPU"):
        df.fwd(a["q3"], a["k3"], a["v3"], a["q_r"], a["k_r"], 32, 0, max_seqlen=64)
    with pytest.raises(ValueError, match="GPU"):
        df.bwd(a["q3"], a["k3"], a["v3"], a["q_r"], a["k_r"], 32, 0, a["q3"], torch.zeros(2, 64),
               a["q3"], max_seqlen=64)
    df._check_lse(torch.zeros(2, 64), a["q3"])
    for bad in (torch.zeros(64, 2), torch.zeros(2, 64, dtype=torch.float64), torch.zeros(2, 128)[:, ::2]):
        with pytest.raises(ValueError):
            df._check_lse(bad, a["q3"])


def test_noalloc_forward_rejects_on_host(df):
    """df_attn_fwd_noalloc: a shape whose forward workspace exceeds the static
    scratch (64 MiB) is refused with DF_ERR_WORKSPACE, and a bad shape with
    the forward's code, before any HIP call (fake pointers)."""
    L = df.lib()
    vp = [ctypes.c_void_p(FAKE)] * 7
    big = _shape(df, batch=1, max_seqlen=4096, total_tokens=4096, num_heads=12, tok_stride=768)
    assert df.workspace_size(0, big, 512, 256) > (64 << 20)
    rc = L.df_attn_fwd_noalloc(ctypes.byref(big), *vp[:5], 512, 256, None, None, vp[5], vp[6], None)
    assert rc == 3 and "static scratch" in L.df_last_error().decode()
    rc = L.df_attn_fwd_noalloc(ctypes.byref(_shape(df, head_dim=48)), *vp[:5], 512, 256, None, None, vp[5],
                               vp[6], None)
    assert rc == 2
    rc = L.df_attn_fwd_noalloc(ctypes.byref(_shape(df)), *vp[:5], 100, 256, None, None, vp[5], vp[6], None)
    assert rc == 1
