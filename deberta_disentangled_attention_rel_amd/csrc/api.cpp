// C ABI of the library: argument validation, workspace planning and launch
// sequencing. Validation is pure host code and runs before any HIP call.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "df_attn.h"
#include "params.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return DF_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t dtype_size(int dt) { return dt == DF_FP32 ? 4 : 2; }

int index_params(int32_t span, int32_t buckets, int* att, int* R) {
  if (span < 1) return fail(DF_ERR_INVALID, "span (max_relative_positions) must be >= 1, got %d", span);
  if (buckets < 0) return fail(DF_ERR_INVALID, "buckets must be >= 0, got %d", buckets);
  if (buckets > 0) {
    if (buckets < 2) return fail(DF_ERR_INVALID, "buckets must be 0 or >= 2, got %d", buckets);
    if (!(span - 1 > buckets / 2))
      return fail(DF_ERR_INVALID,
                  "log buckets need span - 1 > buckets / 2 (span %d, buckets %d)", span, buckets);
  }
  const long a = buckets > 0 ? buckets : span;
  if (2 * a > (1 << 20)) return fail(DF_ERR_INVALID, "relative rows 2*att = %ld too large", 2 * a);
  *att = int(a);
  *R = int(2 * a);
  return DF_OK;
}

int check_shape(const df_attn_shape* s) {
  if (!s) return fail(DF_ERR_INVALID, "shape is NULL");
  if (s->dtype != DF_BF16 && s->dtype != DF_FP16 && s->dtype != DF_FP32)
    return fail(DF_ERR_UNSUPPORTED, "unknown dtype %d", s->dtype);
  if (s->p2c_convention != DF_P2C_LITERAL && s->p2c_convention != DF_P2C_SHARED)
    return fail(DF_ERR_INVALID, "p2c_convention must be DF_P2C_LITERAL (0) or DF_P2C_SHARED (1), got %d",
                s->p2c_convention);
  if (s->flags & ~int32_t(DF_FLAG_BWD_REUSE_FWD))
    return fail(DF_ERR_INVALID, "unknown flags 0x%x", unsigned(s->flags));
  if (s->head_dim != 32 && s->head_dim != 64 && s->head_dim != 128)
    return fail(DF_ERR_UNSUPPORTED, "head_dim must be 32, 64 or 128, got %d", s->head_dim);
  if (s->batch < 1) return fail(DF_ERR_INVALID, "batch must be >= 1, got %d", s->batch);
  if (s->max_seqlen < 1 || s->max_seqlen > (1 << 24))
    return fail(DF_ERR_INVALID, "max_seqlen must be in [1, 2^24], got %d", s->max_seqlen);
  if (s->num_heads < 1 || s->num_heads > 65535)
    return fail(DF_ERR_INVALID, "num_heads must be in [1, 65535], got %d", s->num_heads);
  if (s->total_tokens < 0) return fail(DF_ERR_INVALID, "total_tokens must be >= 0");
  if (s->total_tokens > (int64_t(1) << 40)) return fail(DF_ERR_INVALID, "total_tokens too large");
  const int64_t D = s->head_dim, H = s->num_heads, T = s->total_tokens;
  const int64_t vec = s->dtype == DF_FP32 ? 4 : 8;
  if (s->tok_stride <= 0 || s->head_stride <= 0)
    return fail(DF_ERR_INVALID, "strides must be positive (tok %lld, head %lld)",
                (long long)s->tok_stride, (long long)s->head_stride);
  if (s->tok_stride % vec || s->head_stride % vec)
    return fail(DF_ERR_INVALID, "strides must be multiples of %lld elements", (long long)vec);
  // rows of distinct (token, head) pairs must not overlap: token-major
  // ([T,H,D]-like) or head-major ([H,T,D]-like) placement
  const bool tok_major = s->head_stride >= D && s->tok_stride >= (H - 1) * s->head_stride + D;
  const bool head_major = s->tok_stride >= D && s->head_stride >= (T > 0 ? T - 1 : 0) * s->tok_stride + D;
  if (!tok_major && !head_major)
    return fail(DF_ERR_INVALID, "strides (tok %lld, head %lld) make rows overlap",
                (long long)s->tok_stride, (long long)s->head_stride);
  return DF_OK;
}

int check_all(const df_attn_shape* s, int32_t span, int32_t buckets, bool packed, int* att, int* R) {
  int rc = check_shape(s);
  if (rc) return rc;
  rc = index_params(span, buckets, att, R);
  if (rc) return rc;
  if (!packed && int64_t(s->batch) * s->max_seqlen != s->total_tokens)
    return fail(DF_ERR_INVALID, "padded layout needs total_tokens == batch*max_seqlen (%lld != %d*%d)",
                (long long)s->total_tokens, s->batch, s->max_seqlen);
  {
    // the kernels address one sequence's rows of one head (and its strip
    // rows) with 32-bit byte offsets through buffer views
    const int64_t es = int64_t(dtype_size(s->dtype)), rp = (int64_t(*R) + 7) / 8 * 8;
    const int64_t row = s->tok_stride > rp ? s->tok_stride : rp;
    if (int64_t(s->max_seqlen) * row * es >= (int64_t(1) << 31))
      return fail(DF_ERR_UNSUPPORTED,
                  "one sequence's rows of a head must span less than 2 GiB (max_seqlen %d x row %lld elements)",
                  s->max_seqlen, (long long)row);
  }
  return DF_OK;
}

// Workspace plan. Offsets are relative to the workspace base.
struct Plan {
  size_t lut, lutp, qr_rev, c2ps, p2cs, ends, delta, krT, qrT, dc2p, dp2c, part, total;
  int RP, nchunk, chunk_tokens;
};

Plan make_plan(int pass, const df_attn_shape* s, int R) {
  Plan pl{};
  const size_t es = dtype_size(s->dtype);
  const size_t T = size_t(s->total_tokens), H = size_t(s->num_heads), D = size_t(s->head_dim);
  pl.RP = int((R + 7) / 8 * 8);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, kAlign);
    return at;
  };
  pl.lut = take(2 * (2 * size_t(s->max_seqlen) - 1) * sizeof(int32_t));
  pl.lutp = take((2 * size_t(s->max_seqlen) - 1 + 2 * dfa::kLutPad) * sizeof(uint32_t));
  pl.qr_rev = s->p2c_convention == DF_P2C_SHARED ? take(H * size_t(R) * D * es) : 0;
  pl.c2ps = take(H * T * pl.RP * es);
  pl.p2cs = take(H * T * pl.RP * es);
  pl.ends = take(4 * H * T * es);
  if (pass == 1) {
    // split-K over tokens for the [R, D] weight gradients: about 512
    // workgroups, chunk length a multiple of 32 tokens; a function of the
    // shape only, so the summation order is fixed
    const int64_t rtiles = (R + 127) / 128;
    int64_t nchunk = (512 + int64_t(H) * rtiles - 1) / (int64_t(H) * rtiles);
    const int64_t maxc = (int64_t(T) + 31) / 32;
    if (nchunk > maxc) nchunk = maxc;
    if (nchunk < 1) nchunk = 1;
    int64_t ct = (int64_t(T) + nchunk - 1) / nchunk;
    ct = (ct + 31) / 32 * 32;
    if (ct < 32) ct = 32;
    nchunk = T > 0 ? (int64_t(T) + ct - 1) / ct : 0;
    pl.nchunk = int(nchunk);
    pl.chunk_tokens = int(ct);
    pl.delta = take(H * T * sizeof(float));
    pl.krT = take(H * D * size_t(pl.RP) * es);
    pl.qrT = take(H * D * size_t(pl.RP) * es);
    pl.dc2p = take(H * T * pl.RP * es);
    pl.dp2c = take(H * T * pl.RP * es);
    pl.part = take(2 * H * size_t(nchunk) * size_t(R) * D * sizeof(float));
  }
  pl.total = o;
  return pl;
}

// Whether consecutive d never move either table by more than one row. The
// log part x(a) = (mid-1) ln(a/mid) / ln((span-1)/mid) has its largest slope,
// (mid-1) / (mid ln((span-1)/mid)), at a = mid; when that is at most one, the
// ceiling never skips a value (and the step from the identity part at mid is
// one). A small margin keeps borderline cases on the general path.
bool narrow_tables(int span, int buckets) {
  if (buckets <= 0) return true;
  const int mid = buckets / 2;
  if (mid <= 1) return true;
  const double slope = double(mid - 1) / (double(mid) * std::log(double(span - 1) / double(mid)));
  return slope <= 1.0 - 1e-9;
}

// Far field of the tables. For d >= 0, c2p[d] = R-1 and p2c[d] = 0 together
// hold iff bucket(d) >= att: unbucketed that is d >= span; with log buckets
// and mid >= 2, mid + ceil(x(d)) >= 2 mid iff x(d) > mid - 1 iff d > span - 1
// (x(span-1) = mid-1 exactly). By the oddness of bucket, c2p[d] = 0 and
// p2c[d] = R-1 hold iff d <= -span. With mid = 1 the log part is flat at 1
// and never reaches att, so there is no far field.
int far_bound(int span, int buckets, int Lmax) {
  if (buckets > 0 && buckets / 2 < 2) return Lmax;
  return span < Lmax ? span : Lmax;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

int check_ptr(const void* ptr, const char* name, size_t al) {
  if (!ptr) return fail(DF_ERR_INVALID, "%s is NULL", name);
  if (!aligned(ptr, al)) return fail(DF_ERR_INVALID, "%s must be %zu-byte aligned", name, al);
  return DF_OK;
}

dfa::Params base_params(const df_attn_shape* s, int32_t span, int32_t buckets, int att, int R,
                        const Plan& pl, char* ws, const uint8_t* key_mask, const int32_t* cu) {
  dfa::Params p{};
  p.nseq = s->batch;
  p.Lmax = s->max_seqlen;
  p.H = s->num_heads;
  p.D = s->head_dim;
  p.R = R;
  p.RP = pl.RP;
  p.att = att;
  p.span = span;
  p.buckets = buckets;
  p.dtype = s->dtype;
  p.T = s->total_tokens;
  p.ts = s->tok_stride;
  p.hs = s->head_stride;
  p.cu = cu;
  p.kmask = key_mask;
  p.scale = float(1.0 / std::sqrt(3.0 * s->head_dim));
  p.scale_log2 = float(1.4426950408889634 / std::sqrt(3.0 * s->head_dim));
  p.c2p = reinterpret_cast<int32_t*>(ws + pl.lut);
  p.p2c = p.c2p + (2 * size_t(s->max_seqlen) - 1);
  p.lutp = reinterpret_cast<const uint32_t*>(ws + pl.lutp);
  // narrow kernels keep both rows of a table entry as 16-bit byte offsets
  const size_t esize = s->dtype == DF_FP32 ? 4 : 2;
  p.narrow = (narrow_tables(span, buckets) && size_t(R - 1) * esize <= 0xffff) ? 1 : 0;
  p.p2c_shared = s->p2c_convention == DF_P2C_SHARED ? 1 : 0;
  p.d_hi = far_bound(span, buckets, s->max_seqlen);
  p.d_lo = -p.d_hi;
  p.c2ps = ws + pl.c2ps;
  p.p2cs = ws + pl.p2cs;
  p.ends = ws + pl.ends;
  p.nchunk = pl.nchunk;
  p.chunk_tokens = pl.chunk_tokens;
  return p;
}

int hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return DF_OK;
}

// Index tables, and for the shared P2C convention the reversed q_r the
// kernels then read (p.qr is redirected to it).
hipError_t launch_index(dfa::Params& p, int span, int buckets, char* ws, const Plan& pl, hipStream_t st) {
  hipError_t e = dfa::launch_lut(p.Lmax, span, buckets, p.p2c_shared, p.c2p, p.p2c, const_cast<uint32_t*>(p.lutp), st);
  if (e != hipSuccess || !p.p2c_shared) return e;
  e = dfa::launch_reverse_rows(p.qr, ws + pl.qr_rev, p.H, p.R, p.D, p.dtype == dfa::DF_FP32_T ? 4 : 2, st);
  p.qr = ws + pl.qr_rev;
  return e;
}

// Optional per-launch event timing (df_attn_profile_*).
struct Profiler {
  static constexpr int kCap = 4096;
  bool on = false;
  int n = 0;
  int stage[kCap];
  hipEvent_t ev[2 * kCap];
};
Profiler g_prof;

const char* const kStageNames[DF_NUM_STAGES] = {
    "rel_index", "strips", "fwd", "delta", "bwd_dkv", "bwd_dq", "relgrad_dx", "relgrad_dw", "relgrad_sum"};

// Run one launcher as stage `stage`, bracketed by events when profiling.
template <class F>
int run_stage(int stage, hipStream_t st, const char* what, F&& launch) {
  const bool rec = g_prof.on && g_prof.n < Profiler::kCap;
  const int k = rec ? g_prof.n++ : 0;
  if (rec) {
    g_prof.stage[k] = stage;
    hipEventRecord(g_prof.ev[2 * k], st);
  }
  const hipError_t e = launch();
  if (rec) hipEventRecord(g_prof.ev[2 * k + 1], st);
  return hip_check(e, what);
}

}  // namespace

extern "C" {

int df_attn_version(void) { return 100; }

const char* df_strerror(int code) {
  switch (code) {
    case DF_OK: return "ok";
    case DF_ERR_INVALID: return "invalid argument";
    case DF_ERR_UNSUPPORTED: return "unsupported configuration";
    case DF_ERR_WORKSPACE: return "workspace too small";
    case DF_ERR_HIP: return "HIP error";
    default: return "unknown error";
  }
}

const char* df_last_error(void) { return g_last_error.c_str(); }

int df_attn_profile_enable(int on) {
  if (on && !g_prof.on) {
    for (int k = 0; k < 2 * Profiler::kCap; ++k) {
      const hipError_t e = hipEventCreate(&g_prof.ev[k]);
      if (e != hipSuccess) {
        for (int j = 0; j < k; ++j) hipEventDestroy(g_prof.ev[j]);
        return hip_check(e, "hipEventCreate");
      }
    }
    g_prof.on = true;
    g_prof.n = 0;
  } else if (!on && g_prof.on) {
    for (int k = 0; k < 2 * Profiler::kCap; ++k) hipEventDestroy(g_prof.ev[k]);
    g_prof.on = false;
    g_prof.n = 0;
  }
  return ok();
}

int df_attn_profile_read(float* ms, int* launches, int n_stages) {
  if (!ms || !launches || n_stages < 0) return fail(DF_ERR_INVALID, "profile arrays must not be NULL");
  if (!g_prof.on) return fail(DF_ERR_INVALID, "profiling is not enabled");
  for (int k = 0; k < g_prof.n; ++k) {
    int rc = hip_check(hipEventSynchronize(g_prof.ev[2 * k + 1]), "hipEventSynchronize");
    if (rc) return rc;
    float t = 0.f;
    rc = hip_check(hipEventElapsedTime(&t, g_prof.ev[2 * k], g_prof.ev[2 * k + 1]), "hipEventElapsedTime");
    if (rc) return rc;
    const int sidx = g_prof.stage[k];
    if (sidx < n_stages) {
      ms[sidx] += t;
      launches[sidx] += 1;
    }
  }
  g_prof.n = 0;
  return ok();
}

const char* df_attn_stage_name(int stage) {
  return (stage >= 0 && stage < DF_NUM_STAGES) ? kStageNames[stage] : "";
}

int df_attn_supported(const df_attn_shape* shape, int32_t span, int32_t buckets) {
  int att, R;
  const int rc = check_all(shape, span, buckets, /*packed=*/true, &att, &R);
  return rc ? rc : ok();
}

size_t df_attn_workspace_size(int pass, const df_attn_shape* shape, int32_t span, int32_t buckets) {
  int att, R;
  if (pass != 0 && pass != 1) return 0;
  if (check_all(shape, span, buckets, true, &att, &R)) return 0;
  return make_plan(pass, shape, R).total;
}

int df_build_rel_index(int32_t max_seqlen, int32_t span, int32_t buckets, int32_t* c2p_lut,
                       int32_t* p2c_lut, void* stream) {
  int att, R;
  if (max_seqlen < 1 || max_seqlen > (1 << 24))
    return fail(DF_ERR_INVALID, "max_seqlen must be in [1, 2^24], got %d", max_seqlen);
  int rc = index_params(span, buckets, &att, &R);
  if (rc) return rc;
  if (!c2p_lut || !p2c_lut) return fail(DF_ERR_INVALID, "table pointers must not be NULL");
  rc = hip_check(dfa::launch_lut(max_seqlen, span, buckets, 0, c2p_lut, p2c_lut, nullptr, (hipStream_t)stream),
                 "relative index kernel");
  return rc ? rc : ok();
}

}  // extern "C"

namespace {

struct Dropout {
  float p;
  uint64_t seed;
  uint32_t offset;
};

// Dropout fields of the parameter block; DF_ERR_INVALID unless 0 <= p < 1.
int set_dropout(dfa::Params& prm, const Dropout* d) {
  if (!d || d->p == 0.f) return DF_OK;
  if (!(d->p > 0.f && d->p < 1.f)) return fail(DF_ERR_INVALID, "dropout probability must be in [0, 1), got %g", double(d->p));
  // the backward carries dS = P (dP / (1 - p) - Delta) as a 16-bit MFMA
  // operand; in fp16 (largest value 65504) keep 1 / (1 - p) <= 1000
  if (prm.dtype == dfa::DF_FP16_T && d->p > 0.999f)
    return fail(DF_ERR_UNSUPPORTED, "fp16 dropout needs dropout_p <= 0.999 (1/(1-p) must stay small in fp16), got %g",
                double(d->p));
  prm.drop = 1;
  // p < 1, so floor(p 2^16) <= 65535 fits the 16 bits a pair draws
  prm.drop_thr = uint32_t(std::floor(double(d->p) * 65536.0));
  prm.drop_scale = float(1.0 / (1.0 - double(d->p)));
  prm.seed_lo = uint32_t(d->seed);
  prm.seed_hi = uint32_t(d->seed >> 32);
  prm.drop_off = d->offset;
  return DF_OK;
}

// The forward on every entry point; lse == nullptr skips the LSE store.
int fwd_impl(const df_attn_shape* shape, const void* q, const void* k, const void* v, const void* q_r,
             const void* k_r, int32_t span, int32_t buckets, const uint8_t* key_mask,
             const int32_t* cu_seqlens, void* out, float* lse, void* workspace, size_t workspace_bytes,
             void* stream, const Dropout* drop = nullptr) {
  int att, R;
  int rc = check_all(shape, span, buckets, cu_seqlens != nullptr, &att, &R);
  if (rc) return rc;
  if ((rc = check_ptr(q, "q", 16)) || (rc = check_ptr(k, "k", 16)) || (rc = check_ptr(v, "v", 16)) ||
      (rc = check_ptr(q_r, "q_r", 16)) || (rc = check_ptr(k_r, "k_r", 16)) ||
      (rc = check_ptr(out, "out", 16)) || (lse && (rc = check_ptr(lse, "lse", 4))))
    return rc;
  const Plan pl = make_plan(0, shape, R);
  if (workspace_bytes < pl.total)
    return fail(DF_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", pl.total, workspace_bytes);
  if ((rc = check_ptr(workspace, "workspace", kAlign))) return rc;
  hipStream_t st = (hipStream_t)stream;
  dfa::Params p = base_params(shape, span, buckets, att, R, pl, (char*)workspace, key_mask, cu_seqlens);
  p.q = q;
  p.k = k;
  p.v = v;
  p.qr = q_r;
  p.kr = k_r;
  p.out = out;
  p.lse = lse;
  if ((rc = set_dropout(p, drop))) return rc;
  if (p.T == 0) return ok();
  if ((rc = run_stage(DF_STAGE_INDEX, st, "relative index kernel",
                     [&] { return launch_index(p, span, buckets, (char*)workspace, pl, st); })) ||
      (rc = run_stage(DF_STAGE_STRIPS, st, "strip kernel", [&] { return dfa::launch_strips(p, st); })) ||
      (rc = run_stage(DF_STAGE_FWD, st, "forward kernel", [&] { return dfa::launch_fwd(p, st); })))
    return rc;
  return ok();
}

}  // namespace

extern "C" {

int df_attn_fwd(const df_attn_shape* shape, const void* q, const void* k, const void* v,
                const void* q_r, const void* k_r, int32_t span, int32_t buckets,
                const uint8_t* key_mask, const int32_t* cu_seqlens, void* out, float* lse,
                void* workspace, size_t workspace_bytes, void* stream) {
  if (!lse) return fail(DF_ERR_INVALID, "lse is NULL (df_attn_fwd_inference is the forward without LSE)");
  return fwd_impl(shape, q, k, v, q_r, k_r, span, buckets, key_mask, cu_seqlens, out, lse, workspace,
                  workspace_bytes, stream);
}

int df_attn_fwd_inference(const df_attn_shape* shape, const void* q, const void* k, const void* v,
                          const void* q_r, const void* k_r, int32_t span, int32_t buckets,
                          const uint8_t* key_mask, const int32_t* cu_seqlens, void* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return fwd_impl(shape, q, k, v, q_r, k_r, span, buckets, key_mask, cu_seqlens, out, nullptr, workspace,
                  workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The forward without a caller workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). Its workspace is `scratch`, a static
// device array of a fixed size that each device holds until the process
// ends; calls on one device share it, so calls that overlap on one device
// race. The forward's kernels write every workspace byte they read (index
// tables, strips, end columns) before reading it, so nothing needs clearing
// between calls.

namespace {

constexpr size_t kScratchBytes = size_t(DF_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on each device, looked up once per device
// (with that device current). In host code `scratch` itself is a host-side
// stand-in, never a device address: only these pointers reach kernels.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_of_device(hipStream_t st, void** ptr) {
  int dev = -1;
  int rc = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (rc) return rc;
  if (st) {
    int sdev = -1;
    if ((rc = hip_check(hipStreamGetDevice(st, &sdev), "hipStreamGetDevice"))) return rc;
    if (sdev != dev)
      return fail(DF_ERR_INVALID, "the stream belongs to device %d but device %d is current", sdev, dev);
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(DF_ERR_UNSUPPORTED, "device %d beyond the first %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if ((rc = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"))) return rc;
    if (!p) return fail(DF_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return DF_OK;
}

// For packed batches of uneven sequences the backward runs the dK/dV and dQ
// kernels concurrently: they read the same inputs and write disjoint outputs
// and strips. Their grids are sized by the longest sequence, which leaves
// many work-groups short or empty, and the other kernel's work-groups fill
// the gaps (packed varlen D=128 bf16: fwd+bwd 3.94 -> 3.87 ms). On full
// grids the two only compete for the L2 (L=8192: the backward 2.41 -> 2.6
// ms), so they stay in sequence there. dQ goes on a second stream of the
// device (default priority, created on the first
// backward and kept until the process ends), forked from and joined back to
// the caller's stream by events. The fork and the join are enqueued under a
// lock, and a wait takes the event as recorded at that moment, so calls from
// several host threads stay ordered (their dQ launches share the side
// stream).
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

int side_stream_of_device(SideStream** out) {
  int dev = -1;
  int rc = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (rc) return rc;
  if (dev < 0 || dev >= kMaxDevices) return fail(DF_ERR_UNSUPPORTED, "device %d beyond the first %d", dev, kMaxDevices);
  SideStream& ss = g_side[dev];
  if (!ss.s) {
    hipStream_t s = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    if ((rc = hip_check(hipStreamCreateWithFlags(&s, hipStreamNonBlocking), "hipStreamCreateWithFlags"))) return rc;
    if ((rc = hip_check(hipEventCreateWithFlags(&f, hipEventDisableTiming), "hipEventCreateWithFlags")) ||
        (rc = hip_check(hipEventCreateWithFlags(&j, hipEventDisableTiming), "hipEventCreateWithFlags"))) {
      if (f) hipEventDestroy(f);
      hipStreamDestroy(s);
      return rc;
    }
    ss.s = s;
    ss.fork = f;
    ss.join = j;
  }
  *out = &ss;
  return DF_OK;
}

}  // namespace

extern "C" {

int df_attn_fwd_noalloc(const df_attn_shape* shape, const void* q, const void* k, const void* v,
                        const void* q_r, const void* k_r, int32_t span, int32_t buckets,
                        const uint8_t* key_mask, const int32_t* cu_seqlens, void* out, float* lse,
                        void* stream) {
  // every size check comes before the first HIP call
  int att, R;
  int rc = check_all(shape, span, buckets, cu_seqlens != nullptr, &att, &R);
  if (rc) return rc;
  const size_t need = make_plan(0, shape, R).total;
  if (need > kScratchBytes)
    return fail(DF_ERR_WORKSPACE,
                "this shape needs %zu bytes of workspace; the static scratch of df_attn_fwd_noalloc holds %zu "
                "(use df_attn_fwd with a caller workspace)",
                need, kScratchBytes);
  void* ws = nullptr;
  if ((rc = scratch_of_device((hipStream_t)stream, &ws))) return rc;
  return fwd_impl(shape, q, k, v, q_r, k_r, span, buckets, key_mask, cu_seqlens, out, lse, ws, kScratchBytes,
                  stream);
}

}  // extern "C"

namespace {

// A packed batch whose grid (row blocks of the longest sequence, per
// sequence) is at least 1.5 times its tokens: at least a third of the grid
// is past the ends of the sequences.
bool uneven_grid(const df_attn_shape* shape, const int32_t* cu_seqlens) {
  if (!cu_seqlens || shape->batch < 2) return false;
  const int64_t grid_rows = (int64_t(shape->max_seqlen) + 127) / 128 * 128 * shape->batch;
  return 2 * grid_rows >= 3 * shape->total_tokens;
}

// dK/dV on `st` and, with `side_by_side`, dQ beside it on the device's side
// stream, both after everything enqueued on `st` so far and before whatever
// follows. Without it, or with the stage profiler on, they run one after the
// other on `st` (then each stage's events time that kernel alone).
int dkv_and_dq(const dfa::Params& p, hipStream_t st, bool side_by_side) {
  if (g_prof.on || !side_by_side) {
    int rc;
    if ((rc = run_stage(DF_STAGE_DKV, st, "dk/dv kernel", [&] { return dfa::launch_bwd_dkv(p, st); })) ||
        (rc = run_stage(DF_STAGE_DQ, st, "dq kernel", [&] { return dfa::launch_bwd_dq(p, st); })))
      return rc;
    return DF_OK;
  }
  SideStream* ss = nullptr;
  std::lock_guard<std::mutex> lock(g_side_mu);
  int rc = side_stream_of_device(&ss);
  if (rc) return rc;
  if ((rc = hip_check(hipEventRecord(ss->fork, st), "hipEventRecord")) ||
      (rc = hip_check(hipStreamWaitEvent(ss->s, ss->fork, 0), "hipStreamWaitEvent")) ||
      (rc = hip_check(dfa::launch_bwd_dq(p, ss->s), "dq kernel")) ||
      (rc = hip_check(hipEventRecord(ss->join, ss->s), "hipEventRecord")) ||
      (rc = hip_check(dfa::launch_bwd_dkv(p, st), "dk/dv kernel")) ||
      (rc = hip_check(hipStreamWaitEvent(st, ss->join, 0), "hipStreamWaitEvent")))
    return rc;
  return DF_OK;
}

int bwd_impl(const df_attn_shape* shape, const void* q, const void* k, const void* v, const void* q_r,
             const void* k_r, int32_t span, int32_t buckets, const uint8_t* key_mask,
             const int32_t* cu_seqlens, const void* out, const float* lse, const void* dout, void* dq,
             void* dk, void* dv, void* dq_r, void* dk_r, void* workspace, size_t workspace_bytes,
             void* stream, const Dropout* drop) {
  int att, R;
  int rc = check_all(shape, span, buckets, cu_seqlens != nullptr, &att, &R);
  if (rc) return rc;
  if ((rc = check_ptr(q, "q", 16)) || (rc = check_ptr(k, "k", 16)) || (rc = check_ptr(v, "v", 16)) ||
      (rc = check_ptr(q_r, "q_r", 16)) || (rc = check_ptr(k_r, "k_r", 16)) ||
      (rc = check_ptr(out, "out", 16)) || (rc = check_ptr(lse, "lse", 4)) ||
      (rc = check_ptr(dout, "dout", 16)) || (rc = check_ptr(dq, "dq", 16)) ||
      (rc = check_ptr(dk, "dk", 16)) || (rc = check_ptr(dv, "dv", 16)) ||
      (rc = check_ptr(dq_r, "dq_r", 16)) || (rc = check_ptr(dk_r, "dk_r", 16)))
    return rc;
  const Plan pl = make_plan(1, shape, R);
  if (workspace_bytes < pl.total)
    return fail(DF_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", pl.total, workspace_bytes);
  if ((rc = check_ptr(workspace, "workspace", kAlign))) return rc;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  dfa::Params p = base_params(shape, span, buckets, att, R, pl, ws, key_mask, cu_seqlens);
  p.q = q;
  p.k = k;
  p.v = v;
  p.qr = q_r;
  p.kr = k_r;
  p.out = const_cast<void*>(out);
  p.lse = const_cast<float*>(lse);
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dqr = dq_r;
  p.dkr = dk_r;
  p.delta = reinterpret_cast<float*>(ws + pl.delta);
  p.krT = ws + pl.krT;
  p.qrT = ws + pl.qrT;
  p.dc2p = ws + pl.dc2p;
  p.dp2c = ws + pl.dp2c;
  p.part = reinterpret_cast<float*>(ws + pl.part);
  const bool reuse = (shape->flags & DF_FLAG_BWD_REUSE_FWD) != 0;
  if ((rc = set_dropout(p, drop))) return rc;
  if (p.T > 0) {
    // index tables (and the reversed q_r of the shared P2C convention), then
    // the relative rows transposed for the dQ and dK/dV epilogues
    if ((rc = run_stage(DF_STAGE_INDEX, st, "relative index kernel",
                       [&] {
                         // with DF_FLAG_BWD_REUSE_FWD the forward's tables and strips
                         // (and reversed q_r) are still in the workspace
                         hipError_t e = hipSuccess;
                         if (reuse)
                           p.qr = p.p2c_shared ? static_cast<const void*>(ws + pl.qr_rev) : q_r;
                         else
                           e = launch_index(p, span, buckets, ws, pl, st);
                         const int es = p.dtype == dfa::DF_FP32_T ? 4 : 2;
                         if (e == hipSuccess)
                           e = dfa::launch_transpose_rows(p.kr, ws + pl.krT, p.H, p.R, p.RP, p.D, es, st);
                         if (e == hipSuccess)
                           e = dfa::launch_transpose_rows(p.qr, ws + pl.qrT, p.H, p.R, p.RP, p.D, es, st);
                         return e;
                       })) ||
        (!reuse && (rc = run_stage(DF_STAGE_STRIPS, st, "strip kernel", [&] { return dfa::launch_strips(p, st); }))) ||
        (rc = run_stage(DF_STAGE_DELTA, st, "delta kernel", [&] { return dfa::launch_bwd_pre(p, st); })) ||
        (rc = dkv_and_dq(p, st, uneven_grid(shape, cu_seqlens))) ||
        (rc = run_stage(DF_STAGE_RELGRAD_DW, st, "relative gradient kernel",
                        [&] { return dfa::launch_relgrad_dw(p, st); })))
      return rc;
  }
  // with no tokens this only writes zero dq_r / dk_r
  if ((rc = run_stage(DF_STAGE_RELGRAD_SUM, st, "relative gradient sum kernel",
                     [&] { return dfa::launch_relgrad_sum(p, st); })))
    return rc;
  return ok();
}

}  // namespace

extern "C" {

int df_attn_bwd(const df_attn_shape* shape, const void* q, const void* k, const void* v,
                const void* q_r, const void* k_r, int32_t span, int32_t buckets,
                const uint8_t* key_mask, const int32_t* cu_seqlens, const void* out, const float* lse,
                const void* dout, void* dq, void* dk, void* dv, void* dq_r, void* dk_r,
                void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(shape, q, k, v, q_r, k_r, span, buckets, key_mask, cu_seqlens, out, lse, dout, dq, dk, dv,
                  dq_r, dk_r, workspace, workspace_bytes, stream, nullptr);
}

int df_attn_fwd_dropout(const df_attn_shape* shape, const void* q, const void* k, const void* v,
                        const void* q_r, const void* k_r, int32_t span, int32_t buckets,
                        const uint8_t* key_mask, const int32_t* cu_seqlens, float dropout_p, uint64_t seed,
                        uint32_t offset, void* out, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (!lse) return fail(DF_ERR_INVALID, "lse is NULL");
  const Dropout d{dropout_p, seed, offset};
  return fwd_impl(shape, q, k, v, q_r, k_r, span, buckets, key_mask, cu_seqlens, out, lse, workspace,
                  workspace_bytes, stream, &d);
}

int df_attn_bwd_dropout(const df_attn_shape* shape, const void* q, const void* k, const void* v,
                        const void* q_r, const void* k_r, int32_t span, int32_t buckets,
                        const uint8_t* key_mask, const int32_t* cu_seqlens, float dropout_p, uint64_t seed,
                        uint32_t offset, const void* out, const float* lse, const void* dout, void* dq,
                        void* dk, void* dv, void* dq_r, void* dk_r, void* workspace, size_t workspace_bytes,
                        void* stream) {
  const Dropout d{dropout_p, seed, offset};
  return bwd_impl(shape, q, k, v, q_r, k_r, span, buckets, key_mask, cu_seqlens, out, lse, dout, dq, dk, dv,
                  dq_r, dk_r, workspace, workspace_bytes, stream, &d);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Fused Q/K/V and relative-position projections.

extern "C" {

int df_qkv_proj(int64_t tokens, int32_t hidden, int32_t num_heads, int32_t head_dim, int32_t rel_rows,
                int32_t dtype, const void* x, const void* w, const void* bias, const void* rel, void* q, void* k,
                void* v, void* q_r, void* k_r, void* stream) {
  if (dtype == DF_FP32)
    return fail(DF_ERR_UNSUPPORTED, "df_qkv_proj takes 16-bit operands (bf16 or fp16), not fp32");
  if (dtype != DF_BF16 && dtype != DF_FP16) return fail(DF_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (head_dim != 32 && head_dim != 64 && head_dim != 128)
    return fail(DF_ERR_UNSUPPORTED, "head_dim must be 32, 64 or 128, got %d", head_dim);
  if (num_heads < 1 || num_heads > 65535)
    return fail(DF_ERR_INVALID, "num_heads must be in [1, 65535], got %d", num_heads);
  if (hidden < 8 || hidden % 8)
    return fail(DF_ERR_INVALID, "hidden must be a positive multiple of 8, got %d", hidden);
  if (tokens < 0) return fail(DF_ERR_INVALID, "tokens must be >= 0");
  if (rel_rows < 0) return fail(DF_ERR_INVALID, "rel_rows must be >= 0");
  const int64_t HD = int64_t(num_heads) * head_dim;
  // operand rows are addressed with 32-bit byte offsets per 128-row block;
  // token rows are counted in 32-bit integers
  if (int64_t(hidden) * 2 * 128 >= (int64_t(1) << 31) || 3 * HD >= (int64_t(1) << 31) ||
      tokens >= (int64_t(1) << 30) || tokens * HD >= (int64_t(1) << 40))
    return fail(DF_ERR_UNSUPPORTED, "projection too large (tokens %lld, hidden %d, heads x dim %lld)",
                (long long)tokens, hidden, (long long)HD);
  int rc;
  if ((rc = check_ptr(w, "w", 16)) || (tokens > 0 && (rc = check_ptr(x, "x", 16))) ||
      (tokens > 0 && ((rc = check_ptr(q, "q", 2)) || (rc = check_ptr(k, "k", 2)) || (rc = check_ptr(v, "v", 2)))))
    return rc;
  if (bias && !aligned(bias, 2)) return fail(DF_ERR_INVALID, "bias must be 2-byte aligned");
  const bool want_rel = rel != nullptr && rel_rows > 0;
  if (want_rel && ((rc = check_ptr(rel, "rel", 16)) || (rc = check_ptr(q_r, "q_r", 2)) ||
                   (rc = check_ptr(k_r, "k_r", 2))))
    return rc;
  if (!rel && rel_rows > 0) return fail(DF_ERR_INVALID, "rel is NULL but rel_rows = %d", rel_rows);
  const hipStream_t st = (hipStream_t)stream;
  dfa::ProjParams p{};
  p.w = w;
  p.bias = bias;
  p.K = hidden;
  p.lda = hidden;
  p.ldw = hidden;
  p.kchunk = 0;
  p.HD = int(HD);
  p.D = head_dim;
  p.R = rel_rows;
  p.dtype = dtype;
  if (tokens > 0) {
    p.a = x;
    p.M = int(tokens);
    p.N = int(3 * HD);
    p.mode = 0;
    p.out0 = q;
    p.out1 = k;
    p.out2 = v;
    if (tokens > (int64_t(1) << 31) - 1) return fail(DF_ERR_UNSUPPORTED, "tokens must be < 2^31");
    if ((rc = hip_check(dfa::launch_proj(p, st), "projection (tokens)"))) return rc;
  }
  if (want_rel) {
    p.a = rel;
    p.M = rel_rows;
    p.N = int(2 * HD);
    p.mode = 1;
    p.out0 = q_r;
    p.out1 = k_r;
    p.out2 = nullptr;
    if ((rc = hip_check(dfa::launch_proj(p, st), "projection (relative rows)"))) return rc;
  }
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Packing helpers for the packed layout.

namespace {

int check_pack_args(int32_t batch, int32_t max_len, int64_t row_bytes, const void* a, const char* an,
                    const uint8_t* mask, const void* b, const char* bn, const int32_t* cu) {
  if (batch < 1) return fail(DF_ERR_INVALID, "batch must be >= 1, got %d", batch);
  if (max_len < 1) return fail(DF_ERR_INVALID, "max_len must be >= 1, got %d", max_len);
  if (int64_t(batch) * max_len >= (int64_t(1) << 31))
    return fail(DF_ERR_INVALID, "batch * max_len must be < 2^31");
  if (row_bytes < 16 || row_bytes % 16)
    return fail(DF_ERR_INVALID, "row_bytes must be a positive multiple of 16, got %lld", (long long)row_bytes);
  int rc;
  if ((rc = check_ptr(a, an, 16)) || (rc = check_ptr(b, bn, 16)) || (rc = check_ptr(mask, "mask", 1)) ||
      (rc = check_ptr(cu, "cu_seqlens", 4)))
    return rc;
  return DF_OK;
}

}  // namespace

extern "C" {

int df_pack_padded(int32_t batch, int32_t max_len, int64_t row_bytes, const void* padded, const uint8_t* mask,
                   void* packed, int32_t* cu_seqlens, int32_t* max_seqlen, void* stream) {
  int rc = check_pack_args(batch, max_len, row_bytes, padded, "padded", mask, packed, "packed", cu_seqlens);
  if (rc) return rc;
  if ((rc = hip_check(dfa::launch_pack(batch, max_len, row_bytes, padded, mask, packed, cu_seqlens, max_seqlen,
                                       (hipStream_t)stream),
                      "pack")))
    return rc;
  return ok();
}

int df_unpack_packed(int32_t batch, int32_t max_len, int64_t row_bytes, const void* packed, const uint8_t* mask,
                     const int32_t* cu_seqlens, void* padded, void* stream) {
  int rc = check_pack_args(batch, max_len, row_bytes, packed, "packed", mask, padded, "padded", cu_seqlens);
  if (rc) return rc;
  if ((rc = hip_check(dfa::launch_unpack(batch, max_len, row_bytes, packed, mask, cu_seqlens, padded,
                                         (hipStream_t)stream),
                      "unpack")))
    return rc;
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Backward of the fused projections.

namespace {

struct ProjBwdPlan {
  size_t wt, dyt, xt, relt, dyr, dyrt, part, total;
  int64_t Tp, Rp;
  int nch, kchunk;
};

ProjBwdPlan proj_bwd_plan(int64_t T, int E, int64_t HD, int R) {
  ProjBwdPlan pl{};
  const int64_t N3 = 3 * HD, N2 = 2 * HD;
  pl.Tp = (T + 7) / 8 * 8;
  pl.Rp = (int64_t(R) + 7) / 8 * 8;
  // split the token contraction of dW into fixed chunks (a function of the
  // shape only): about 512 work-groups
  const int64_t tiles = ((N3 + 127) / 128) * ((int64_t(E) + 1 + 127) / 128);
  int64_t nch = (512 + tiles - 1) / tiles;
  int64_t kc = T > 0 ? ((T + nch - 1) / nch + 63) / 64 * 64 : 64;
  nch = T > 0 ? (T + kc - 1) / kc : 0;
  pl.nch = int(nch);
  pl.kchunk = int(kc);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, kAlign);
    return at;
  };
  pl.wt = take(size_t(E) * N3 * 2);
  pl.dyt = take(size_t(N3) * pl.Tp * 2);
  pl.xt = take(size_t(E + 1) * pl.Tp * 2);
  pl.relt = take(size_t(E + 1) * pl.Rp * 2);
  pl.dyr = take(size_t(R) * N2 * 2);
  pl.dyrt = take(size_t(N2) * pl.Rp * 2);
  pl.part = take(size_t(nch + 1) * N3 * (E + 1) * sizeof(float));
  pl.total = o;
  return pl;
}

int check_proj_dims(int64_t tokens, int32_t hidden, int32_t num_heads, int32_t head_dim, int32_t rel_rows,
                    int32_t dtype) {
  if (dtype == DF_FP32)
    return fail(DF_ERR_UNSUPPORTED, "the projections take 16-bit operands (bf16 or fp16), not fp32");
  if (dtype != DF_BF16 && dtype != DF_FP16) return fail(DF_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (head_dim != 32 && head_dim != 64 && head_dim != 128)
    return fail(DF_ERR_UNSUPPORTED, "head_dim must be 32, 64 or 128, got %d", head_dim);
  if (num_heads < 1 || num_heads > 65535)
    return fail(DF_ERR_INVALID, "num_heads must be in [1, 65535], got %d", num_heads);
  if (hidden < 8 || hidden % 8)
    return fail(DF_ERR_INVALID, "hidden must be a positive multiple of 8, got %d", hidden);
  if (tokens < 0 || rel_rows < 0) return fail(DF_ERR_INVALID, "tokens and rel_rows must be >= 0");
  const int64_t HD = int64_t(num_heads) * head_dim;
  // the transposed operands' rows (tokens long) are addressed with 32-bit
  // byte offsets per 128-row block
  if (tokens >= (int64_t(1) << 23) || int64_t(hidden) >= (int64_t(1) << 20) || 3 * HD >= (int64_t(1) << 20) ||
      rel_rows >= (1 << 20))
    return fail(DF_ERR_UNSUPPORTED, "projection too large (tokens %lld, hidden %d, heads x dim %lld)",
                (long long)tokens, hidden, (long long)HD);
  return DF_OK;
}

}  // namespace

extern "C" {

size_t df_qkv_proj_bwd_workspace_size(int64_t tokens, int32_t hidden, int32_t num_heads, int32_t head_dim,
                                      int32_t rel_rows, int32_t dtype) {
  if (check_proj_dims(tokens, hidden, num_heads, head_dim, rel_rows, dtype)) return 0;
  return proj_bwd_plan(tokens, hidden, int64_t(num_heads) * head_dim, rel_rows).total;
}

int df_qkv_proj_bwd(int64_t tokens, int32_t hidden, int32_t num_heads, int32_t head_dim, int32_t rel_rows,
                    int32_t dtype, const void* x, const void* w, const void* rel, const void* dqkv,
                    const void* dq_r, const void* dk_r, void* dx, void* dw, void* db, void* drel,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_proj_dims(tokens, hidden, num_heads, head_dim, rel_rows, dtype);
  if (rc) return rc;
  const bool want_rel = rel != nullptr && rel_rows > 0;
  if (!rel && rel_rows > 0) return fail(DF_ERR_INVALID, "rel is NULL but rel_rows = %d", rel_rows);
  if ((rc = check_ptr(w, "w", 16)) || (rc = check_ptr(dw, "dw", 2)) ||
      (tokens > 0 && ((rc = check_ptr(x, "x", 16)) || (rc = check_ptr(dqkv, "dqkv", 16)) ||
                      (rc = check_ptr(dx, "dx", 2)))) ||
      (want_rel && ((rc = check_ptr(rel, "rel", 16)) || (rc = check_ptr(dq_r, "dq_r", 16)) ||
                    (rc = check_ptr(dk_r, "dk_r", 16)) || (rc = check_ptr(drel, "drel", 2)))))
    return rc;
  if (db && !aligned(db, 2)) return fail(DF_ERR_INVALID, "db must be 2-byte aligned");
  const int64_t T = tokens, HD = int64_t(num_heads) * head_dim, N3 = 3 * HD, N2 = 2 * HD;
  const int E = hidden, R = want_rel ? rel_rows : 0;
  const ProjBwdPlan pl = proj_bwd_plan(T, E, HD, R);
  if (workspace_bytes < pl.total)
    return fail(DF_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", pl.total, workspace_bytes);
  if ((rc = check_ptr(workspace, "workspace", kAlign))) return rc;
  char* ws = (char*)workspace;
  const hipStream_t st = (hipStream_t)stream;
  const uint16_t one = dtype == DF_FP16 ? 0x3C00 : 0x3F80;
  float* part = reinterpret_cast<float*>(ws + pl.part);

  auto gemm = [&](const void* a, int lda, const void* b, int ldw, int M, int N, int K, int kchunk, int mode,
                  void* out) {
    dfa::ProjParams p{};
    p.a = a;
    p.w = b;
    p.M = M;
    p.N = N;
    p.K = K;
    p.lda = lda;
    p.ldw = ldw;
    p.kchunk = kchunk;
    p.HD = N;  // mode 0: a plain [M, N] output
    p.D = head_dim;
    p.mode = mode;
    p.dtype = dtype;
    p.out0 = out;
    return dfa::launch_proj(p, st);
  };
  hipError_t e = hipSuccess;
  auto run = [&](hipError_t r) {
    if (e == hipSuccess) e = r;
  };
  // transposed operands: W^T [E][3HD]; dY^T [3HD][Tp]; x^T [E + 1][Tp] with a
  // last row of ones (its column of the dW product is db)
  run(dfa::launch_transpose16(w, E, 0, ws + pl.wt, N3, 0, int(N3), E, 1, st));
  if (T > 0) {
    run(dfa::launch_transpose16(dqkv, N3, 0, ws + pl.dyt, pl.Tp, 0, int(T), int(N3), 1, st));
    run(dfa::launch_transpose16(x, E, 0, ws + pl.xt, pl.Tp, 0, int(T), E, 1, st));
    run(dfa::launch_fill16(ws + pl.xt + size_t(E) * pl.Tp * 2, T, one, st));
    // dx = dY W
    run(gemm(dqkv, int(N3), ws + pl.wt, int(N3), int(T), E, int(N3), 0, 0, dx));
    // dW partials over token chunks (and db in column E)
    run(gemm(ws + pl.dyt, int(pl.Tp), ws + pl.xt, int(pl.Tp), int(N3), E + 1, int(T), pl.kchunk, 2, part));
  }
  if (want_rel) {
    run(dfa::launch_transpose16(rel, E, 0, ws + pl.relt, pl.Rp, 0, R, E, 1, st));
    run(dfa::launch_fill16(ws + pl.relt + size_t(E) * pl.Rp * 2, R, one, st));
    run(dfa::launch_rel_rows(dq_r, dk_r, ws + pl.dyr, num_heads, R, head_dim, st));
    run(dfa::launch_transpose16(ws + pl.dyr, N2, 0, ws + pl.dyrt, pl.Rp, 0, R, int(N2), 1, st));
    // drel = dY_r W[:2HD]
    run(gemm(ws + pl.dyr, int(N2), ws + pl.wt, int(N3), R, E, int(N2), 0, 0, drel));
    // the relative rows' dW (and db) partial, after the token chunks
    run(gemm(ws + pl.dyrt, int(pl.Rp), ws + pl.relt, int(pl.Rp), int(N2), E + 1, R, 0, 2,
             part + size_t(pl.nch) * N3 * (E + 1)));
  }
  run(dfa::launch_proj_reduce(part, T > 0 ? pl.nch : 0, want_rel ? int(N2) : 0, int(N3), E, dtype, dw, db, st));
  if ((rc = hip_check(e, "projection backward"))) return rc;
  return ok();
}

}  // extern "C"
