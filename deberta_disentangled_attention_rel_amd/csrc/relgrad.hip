// Relative-position gradients from the dense dC2P / dP2C strips
// (DisentangledFlash 1.1.1 page, "Hugging Face usage": relative-position
// projections stay in the autograd graph; "Performance": the 12LRD term of
// the backward count).
//
//   dk_r = s * sum_t dC2P[t]^T Q[t]    dq_r = s * sum_t dP2C[t]^T K[t]    (per head)
//
// (The per-token terms s * dC2P K_r and s * dP2C Q_r are added by the dQ and
// dK/dV kernels themselves, at the end of each work-group.) The GEMM stages
// row-major tiles with coalesced 16-byte loads, prefetched into registers two
// token blocks ahead (two register sets in turn; double-buffered LDS, one
// barrier per step); operands that run down the rows are read with
// transposing LDS reads. The loads are range-checked buffer loads over the
// chunk's rows, issued unconditionally, so the wait before a block's LDS
// store leaves the next block's loads in flight. The token sums are split into fixed chunks; each
// chunk's [R, D] partial is written to the workspace and a second kernel adds
// the chunks in index order. No atomics; the chunking depends only on the
// shape.
#include "pipe.hpp"

namespace dfa {

namespace {

// A ROWS x COLS tile staged through registers: each thread's 16-byte chunks
// have fixed byte offsets in the view (init); a tile's first-row byte offset
// is added to them, so the whole per-lane offset is range-checked and rows
// past the view load zero without touching memory.
template <typename T, int ROWS, int COLS, int NT>
struct BufTile {
  static constexpr int CH = 16 / int(sizeof(T)), NC = COLS / CH, CHUNKS = ROWS * NC;
  static_assert(CHUNKS % NT == 0, "every thread owns whole chunks");
  static constexpr int PER = CHUNKS / NT;
  uint4 r[PER];
  int voff[PER];
  __device__ __forceinline__ void init(int ld, int col0) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int it = int(threadIdx.x) + u * NT;
      voff[u] = ((it / NC) * ld + col0 + (it % NC) * CH) * int(sizeof(T));
    }
  }
  __device__ __forceinline__ void load(BufView v, int boff) {
#pragma unroll
    for (int u = 0; u < PER; ++u) r[u] = buf_load16(v, voff[u] + boff);
  }
  template <int P>
  __device__ __forceinline__ void store(T* __restrict__ lds) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int it = int(threadIdx.x) + u * NT;
      {
        const int off = (it / NC) * P + (it % NC) * CH;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint4*>(lds + off) = r[u];
        } else {
          float* d = reinterpret_cast<float*>(lds) + off;
          d[0] = __uint_as_float(r[u].x);
          d[1] = __uint_as_float(r[u].y);
          d[2] = __uint_as_float(r[u].z);
          d[3] = __uint_as_float(r[u].w);
        }
      }
    }
  }
};

// Split-K partials of dk_r (which = 0: dC2P^T Q) and dq_r (which = 1: dP2C^T K).
// Workgroup: 128 strip rows r (4 waves x 32) x all D columns, over one chunk
// of tokens, TK tokens at a time.
template <int DT, int D>
__global__ __launch_bounds__(256) void dw_kernel(Params p) {
  using TR = Tr<DT>;
  using T = typename TR::T;
  constexpr int KS = TR::KS, ND = D / 32;
  constexpr int RM = 128, TK = 64;
  constexpr int GP = RowPitch<T, RM>::cols, XP = RowPitch<T, D>::cols;
  __shared__ __align__(16) T Gs[2][TK * GP];
  __shared__ __align__(16) T Xs[2][TK * XP];

  const int which = blockIdx.z / p.H, h = blockIdx.z % p.H;
  const int chunk = blockIdx.y;
  const int lane = threadIdx.x & 63, g = lane >> 5, li = lane & 31, wave = threadIdx.x >> 6;
  const int r0 = blockIdx.x * RM;
  const int R = p.R, RP = p.RP;
  const T* G = (const T*)(which ? p.dp2c : p.dc2p) + int64_t(h) * p.T * RP;
  const T* X = (const T*)(which ? p.k : p.q) + int64_t(h) * p.hs;
  const int64_t c0 = int64_t(chunk) * p.chunk_tokens;
  const int64_t c1 = c0 + p.chunk_tokens < p.T ? c0 + p.chunk_tokens : p.T;

  f32x16 acc[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) acc[nd] = zero16();
  // views of the chunk's token rows: rows at or past c1 read zero (strip
  // columns past RP only feed output rows that are never written)
  const int nt = int(c1 - c0);
  const BufView gv = buf_view(G + c0 * RP, uint32_t(nt > 0 ? nt : 0) * uint32_t(RP) * uint32_t(sizeof(T)));
  const BufView xv = buf_view(X + c0 * p.ts, uint32_t(nt > 0 ? nt : 0) * uint32_t(p.ts) * uint32_t(sizeof(T)));
  const int gstep = TK * RP * int(sizeof(T)), xstep = TK * int(p.ts) * int(sizeof(T));
  // token blocks two ahead in registers, the two register sets in turn
  BufTile<T, TK, RM, 256> ga, gb;
  BufTile<T, TK, D, 256> xa, xb;
  ga.init(RP, r0);
  gb.init(RP, r0);
  xa.init(int(p.ts), 0);
  xb.init(int(p.ts), 0);
  const int nk = nt > 0 ? (nt + TK - 1) / TK : 0;
  if (nk > 0) {
    ga.load(gv, 0);
    xa.load(xv, 0);
    ga.template store<GP>(Gs[0]);
    xa.template store<XP>(Xs[0]);
    ga.load(gv, gstep);  // block 1 (zeros past the chunk)
    xa.load(xv, xstep);
  }
  __syncthreads();
  // step k: LDS buffer k % 2 holds block k, `cur` holds block k + 1 in
  // flight; block k + 2 goes into `nxt`, and `cur` is stored after the
  // MFMAs. Blocks past the chunk are zeros and add nothing, so the steps run
  // in pairs without conditions (the loop body has no branch that would
  // split the two register sets)
  auto step = [&](int k, int buf, auto& cur_g, auto& cur_x, auto& nxt_g, auto& nxt_x) {
    nxt_g.load(gv, (k + 2) * gstep);
    nxt_x.load(xv, (k + 2) * xstep);
    __builtin_amdgcn_sched_barrier(0);  // the loads go out before the MFMAs and the stores
#pragma unroll
    for (int q = 0; q < TK / KS; ++q) {
      const auto a = ld_col<TR>(Gs[buf], GP, 0, 32 * wave, q);
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) acc[nd] = TR::mma(a, ld_col<TR>(Xs[buf], XP, 0, 32 * nd, q), acc[nd]);
    }
    cur_g.template store<GP>(Gs[buf ^ 1]);
    cur_x.template store<XP>(Xs[buf ^ 1]);
    __syncthreads();
  };
  for (int k = 0; k < nk; k += 2) {
    step(k, 0, ga, xa, gb, xb);
    step(k + 1, 1, gb, xb, ga, xa);
  }
  float* part = p.part + ((int64_t(which) * p.H + h) * p.nchunk + chunk) * int64_t(R) * D;
#pragma unroll
  for (int nd = 0; nd < ND; ++nd)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = r0 + 32 * wave + acc_row(v, g);
      if (r < R) part[int64_t(r) * D + 32 * nd + li] = acc[nd][v];
    }
}

// Fixed-order sum of the chunk partials: out[h][r][d] = s * sum_c part[c].
// A thread sums 4 consecutive elements (one 16-byte load per chunk; D is a
// multiple of 4, so the 4 share a row) with the chunk loop unrolled, so its
// loads overlap; every element still adds its chunks in index order.
template <int DT>
__global__ __launch_bounds__(256) void reduce_kernel(Params p) {
  using TR = Tr<DT>;
  using T = typename TR::T;
  const int64_t per = int64_t(p.R) * p.D;
  const int64_t n = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  const int64_t total = 2 * int64_t(p.H) * per;
  if (n >= total) return;
  const int64_t which = n / (int64_t(p.H) * per);
  const int64_t rest = n % (int64_t(p.H) * per);
  const int64_t h = rest / per, e = rest % per;
  const float4* part = reinterpret_cast<const float4*>(p.part + (which * p.H + h) * p.nchunk * per + e);
  const int64_t per4 = per / 4;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll 8
  for (int c = 0; c < p.nchunk; ++c) {
    const float4 v = part[c * per4];
    s0 += v.x;
    s1 += v.y;
    s2 += v.z;
    s3 += v.w;
  }
  T* out = (T*)(which ? p.dqr : p.dkr);
  // dq_r of the shared P2C convention was accumulated in reversed row order
  const int64_t e_out = (which && p.p2c_shared) ? (int64_t(p.R - 1) - e / p.D) * p.D + e % p.D : e;
  T* o = out + h * per + e_out;
  o[0] = TR::from_f(s0 * p.scale);
  o[1] = TR::from_f(s1 * p.scale);
  o[2] = TR::from_f(s2 * p.scale);
  o[3] = TR::from_f(s3 * p.scale);
}

template <int DT, int D>
void launch_dw_d(const Params& p, hipStream_t st) {
  dim3 g2(unsigned((p.R + 127) / 128), unsigned(p.nchunk), unsigned(2 * p.H));
  dw_kernel<DT, D><<<g2, 256, 0, st>>>(p);
}

template <int DT>
void launch_sum_dt(const Params& p, hipStream_t st) {
  const int64_t total = 2 * int64_t(p.H) * p.R * p.D;  // a multiple of 4 (D is)
  reduce_kernel<DT><<<unsigned((total / 4 + 255) / 256), 256, 0, st>>>(p);
}

#define DF_DISPATCH(FN, p, st)                     \
  switch (p.dtype) {                               \
    case DF_BF16_T:                                \
      if (p.D == 32) FN<DF_BF16_T, 32>(p, st);     \
      else if (p.D == 64) FN<DF_BF16_T, 64>(p, st); \
      else FN<DF_BF16_T, 128>(p, st);              \
      break;                                       \
    case DF_FP16_T:                                \
      if (p.D == 32) FN<DF_FP16_T, 32>(p, st);     \
      else if (p.D == 64) FN<DF_FP16_T, 64>(p, st); \
      else FN<DF_FP16_T, 128>(p, st);              \
      break;                                       \
    default:                                       \
      if (p.D == 32) FN<DF_FP32_T, 32>(p, st);     \
      else if (p.D == 64) FN<DF_FP32_T, 64>(p, st); \
      else FN<DF_FP32_T, 128>(p, st);              \
      break;                                       \
  }

}  // namespace

hipError_t launch_relgrad_dw(const Params& p, hipStream_t st) {
  if (p.T == 0) return hipSuccess;
  DF_DISPATCH(launch_dw_d, p, st)
  return hipGetLastError();
}

hipError_t launch_relgrad_sum(const Params& p, hipStream_t st) {
  switch (p.dtype) {
    case DF_BF16_T: launch_sum_dt<DF_BF16_T>(p, st); break;
    case DF_FP16_T: launch_sum_dt<DF_FP16_T>(p, st); break;
    default: launch_sum_dt<DF_FP32_T>(p, st); break;
  }
  return hipGetLastError();
}

}  // namespace dfa
