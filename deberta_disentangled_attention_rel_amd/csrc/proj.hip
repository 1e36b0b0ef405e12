// Fused Q/K/V and relative-position projections (DisentangledFlash 1.1.1
// page, "Status": the fused QKV projection is always enabled; "Hugging Face
// usage": the Q/K/V and relative-position projections stay in the model's
// graph). One GEMM Y = A W^T + b with the weights of the three maps stacked
// as one [3 H D, E] matrix (rows W_q, W_k, W_v):
//   tokens   (A = x [T, E], all 3 H D columns)  -> q, k, v [T, H, D]
//   relative (A = rel [R, E], the first 2 H D)  -> q_r, k_r [H, R, D]
// (the relative-position rows go through the query and key maps, DeBERTa's
// shared attention key).
//
// Work-group: a 128 x 128 tile of Y, 4 waves as 2 x 2 blocks of 64 x 64
// (2 x 2 MFMA 32x32x16 accumulators each), the contraction in 64-wide steps.
// Both operands are K-contiguous rows, so A and W tiles are staged row-major
// in LDS (two buffers) and both fragments are plain 16-byte row reads. The
// tiles go through registers two steps ahead (two register sets in turn):
// each thread's 16-byte chunks have fixed offsets, the step's column is added
// to them, rows past the matrix read zero (range check) and columns past the
// contraction are sent past the view by a select, so every load is
// unconditional and a step's LDS stores wait only for the loads of the step
// before (one step of copies in flight, as LDS-DMA into two buffers allows,
// left the steps waiting on memory latency). Work-groups are renumbered so that each XCD runs a
// contiguous range of tiles, column tile fastest: the tiles of one row block
// share its A rows in that XCD's L2.
#include "pipe.hpp"

namespace dfa {

namespace {

constexpr int PBM = 128, PBN = 128, PBK = 64, PP = PBK + 8;  // tile and LDS row pitch (elements)

// One operand tile (128 rows x 64 columns) of a step in registers: chunk
// u of thread t is row (t + 256u) / 8, columns 8 ((t + 256u) % 8) .. + 7.
struct ProjRegs {
  static constexpr int PER = PBM * (PBK / 8) / 256;
  uint4 r[PER];
  __device__ __forceinline__ static int row_of(int u) { return (int(threadIdx.x) + 256 * u) / (PBK / 8); }
  __device__ __forceinline__ static int col_of(int u) { return ((int(threadIdx.x) + 256 * u) % (PBK / 8)) * 8; }
  // columns k0 .. k0 + 63 of the view's rows (row stride ld elements);
  // columns at or past K read zero
  __device__ __forceinline__ void load(BufView b, int ld, int k0, int K) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = k0 + col_of(u);
      r[u] = buf_load16(b, c < K ? (row_of(u) * ld + c) * 2 : kBufSkip);
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) *reinterpret_cast<uint4*>(lds + row_of(u) * PP + col_of(u)) = r[u];
  }
};

template <int DT>
__global__ __launch_bounds__(256, 2) void proj_kernel(ProjParams p) {
  using TR = Tr<DT>;
  using T = typename TR::T;
  constexpr int E = TR::E, KS = TR::KS;
  static_assert(sizeof(T) == 2, "16-bit operands");
  __shared__ __align__(16) uint16_t As[2][PBM * PP];
  __shared__ __align__(16) uint16_t Bs[2][PBN * PP];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, li = lane & 31, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nn = (p.N + PBN - 1) / PBN;
  // XCD-contiguous renumbering of the 1-D grid (the dispatcher deals
  // consecutive ids to the 8 XCDs in turn)
  const int nb = gridDim.x, id = blockIdx.x;
  const int qx = nb / 8, rx = nb % 8, xcd = id % 8, slot = id / 8;
  const int logical = xcd * qx + (xcd < rx ? xcd : rx) + slot;
  const int m0 = (logical / nn) * PBM, n0 = (logical % nn) * PBN;

  // this chunk's contraction range
  const int kb = p.kchunk > 0 ? int(blockIdx.y) * p.kchunk : 0;
  const int K = p.kchunk > 0 ? min(p.K, kb + p.kchunk) : p.K;
  const T* A = (const T*)p.a + int64_t(m0) * p.lda;
  const T* W = (const T*)p.w + int64_t(n0) * p.ldw;
  const BufView av = buf_view(A, uint32_t(min(PBM, p.M - m0)) * uint32_t(p.lda) * 2u);
  const BufView wv = buf_view(W, uint32_t(min(PBN, p.N - n0)) * uint32_t(p.ldw) * 2u);
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = zero16();

  const int nk = K > kb ? (K - kb + PBK - 1) / PBK : 0;
  ProjRegs ra0, rb0, ra1, rb1;
  if (nk > 0) {
    ra0.load(av, p.lda, kb, K);
    rb0.load(wv, p.ldw, kb, K);
    ra0.store(As[0]);
    rb0.store(Bs[0]);
    ra0.load(av, p.lda, kb + PBK, K);  // step 1 (zeros past K)
    rb0.load(wv, p.ldw, kb + PBK, K);
  }
  __syncthreads();
  // step kt: LDS buffer kt % 2 holds step kt, `cur` step kt + 1 in flight;
  // step kt + 2 goes into `nxt`. Steps past nk read zeros and add nothing,
  // so the steps run in pairs without conditions.
  auto step = [&](int kt, int buf, ProjRegs& cur_a, ProjRegs& cur_b, ProjRegs& nxt_a, ProjRegs& nxt_b) {
    nxt_a.load(av, p.lda, kb + (kt + 2) * PBK, K);
    nxt_b.load(wv, p.ldw, kb + (kt + 2) * PBK, K);
    __builtin_amdgcn_sched_barrier(0);  // the loads go out before the MFMAs and the stores
    const T* a_s = reinterpret_cast<const T*>(As[buf]);
    const T* b_s = reinterpret_cast<const T*>(Bs[buf]);
#pragma unroll
    for (int kk = 0; kk < PBK / KS; ++kk) {
      typename TR::frag af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = ld_row<TR>(a_s, PP, wm * 64 + i * 32 + li, kk * KS + g * E);
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = ld_row<TR>(b_s, PP, wn * 64 + j * 32 + li, kk * KS + g * E);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = TR::mma(af[i], bf[j], acc[i][j]);
    }
    cur_a.store(As[buf ^ 1]);
    cur_b.store(Bs[buf ^ 1]);
    __syncthreads();
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, 0, ra0, rb0, ra1, rb1);
    step(kt + 1, 1, ra1, rb1, ra0, rb0);
  }

  // lane: column n = n0 + wn*64 + 32j + li; register v: row m0 + wm*64 + 32i + acc_row(v, g)
  if (p.mode == 2) {
    float* part = (float*)p.out0 + int64_t(blockIdx.y) * p.M * p.N;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + 32 * j + li;
      if (n >= p.N) continue;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + wm * 64 + 32 * i + acc_row(v, g);
          if (m < p.M) part[int64_t(m) * p.N + n] = acc[i][j][v];
        }
    }
    return;
  }
  const int HD = p.HD, D = p.D;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + 32 * j + li;
    if (n >= p.N) continue;
    const float bn = p.bias ? TR::to_f(((const T*)p.bias)[n]) : 0.f;
    const int which = n / HD, hd = n - which * HD;
    T* out = (T*)(which == 0 ? p.out0 : (which == 1 ? p.out1 : p.out2));
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * 64 + 32 * i + acc_row(v, g);
        if (m >= p.M) continue;
        const int64_t at = p.mode == 0 ? int64_t(m) * HD + hd
                                       : (int64_t(hd / D) * p.R + m) * D + (hd % D);
        out[at] = TR::from_f(acc[i][j][v] + bn);
      }
  }
}

}  // namespace

hipError_t launch_proj(const ProjParams& p, hipStream_t st) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  const unsigned nb = unsigned((p.M + PBM - 1) / PBM) * unsigned((p.N + PBN - 1) / PBN);
  const unsigned nch = p.kchunk > 0 ? unsigned((p.K + p.kchunk - 1) / p.kchunk) : 1u;
  const dim3 grid(nb, nch);
  if (p.dtype == DF_FP16_T)
    proj_kernel<DF_FP16_T><<<grid, 256, 0, st>>>(p);
  else
    proj_kernel<DF_BF16_T><<<grid, 256, 0, st>>>(p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Pieces of the projections' backward.

namespace {

// 64 x 64 tiles through LDS: coalesced reads along the source rows and
// coalesced writes along the destination rows
__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t* __restrict__ src, int64_t src_ld,
                                                          int64_t src_bs, uint16_t* __restrict__ dst,
                                                          int64_t dst_ld, int64_t dst_bs, int rows, int cols) {
  __shared__ uint16_t tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const uint16_t* s = src + int64_t(blockIdx.z) * src_bs;
  uint16_t* d = dst + int64_t(blockIdx.z) * dst_bs;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int k = ty; k < 64; k += 4) {
    const int r = r0 + k, c = c0 + tx;
    tile[k][tx] = (r < rows && c < cols) ? s[int64_t(r) * src_ld + c] : uint16_t(0);
  }
  __syncthreads();
  for (int k = ty; k < 64; k += 4) {
    const int c = c0 + k, r = r0 + tx;  // destination row c, column r
    if (c < cols && r < dst_ld) d[int64_t(c) * dst_ld + r] = tile[tx][k];
  }
}

__global__ void fill16_kernel(uint16_t* __restrict__ dst, int64_t n, uint16_t bits) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = bits;
}

// one thread per 8 elements (16 bytes) of a destination row
__global__ void rel_rows_kernel(const uint4* __restrict__ dq_r, const uint4* __restrict__ dk_r,
                                uint4* __restrict__ dst, int H, int R, int D) {
  const int cpr = D / 8;  // chunks per (head, relative row)
  const int64_t n = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_row = 2 * int64_t(H) * cpr;
  if (n >= per_row * R) return;
  const int64_t r = n / per_row, rest = n % per_row;
  const int which = int(rest / (int64_t(H) * cpr)), hc = int(rest % (int64_t(H) * cpr));
  const int h = hc / cpr, c = hc % cpr;
  const uint4* src = which ? dk_r : dq_r;
  dst[n] = src[(int64_t(h) * R + r) * cpr + c];
}

template <int DT>
__global__ void proj_reduce_kernel(const float* __restrict__ part, int nch, int nrel, int M, int E,
                                   typename Tr<DT>::T* __restrict__ out, typename Tr<DT>::T* __restrict__ db) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t N = int64_t(E) + 1;
  if (i >= int64_t(M) * N) return;
  const int n = int(i / N), e = int(i % N);
  float s = 0.f;
  for (int c = 0; c < nch; ++c) s += part[int64_t(c) * M * N + i];
  if (n < nrel) s += part[int64_t(nch) * M * N + i];
  if (e < E)
    out[int64_t(n) * E + e] = Tr<DT>::from_f(s);
  else if (db)
    db[n] = Tr<DT>::from_f(s);
}

}  // namespace

hipError_t launch_transpose16(const void* src, int64_t src_ld, int64_t src_bs, void* dst, int64_t dst_ld,
                              int64_t dst_bs, int rows, int cols, int batch, hipStream_t st) {
  if (cols <= 0 || batch <= 0 || dst_ld <= 0) return hipSuccess;
  const dim3 grid(unsigned((cols + 63) / 64), unsigned((dst_ld + 63) / 64), unsigned(batch));
  transpose16_kernel<<<grid, 256, 0, st>>>((const uint16_t*)src, src_ld, src_bs, (uint16_t*)dst, dst_ld, dst_bs,
                                           rows, cols);
  return hipGetLastError();
}

hipError_t launch_fill16(void* dst, int64_t n, uint16_t bits, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  fill16_kernel<<<unsigned((n + 255) / 256), 256, 0, st>>>((uint16_t*)dst, n, bits);
  return hipGetLastError();
}

hipError_t launch_rel_rows(const void* dq_r, const void* dk_r, void* dst, int H, int R, int D, hipStream_t st) {
  const int64_t n = 2 * int64_t(H) * R * (D / 8);
  if (n <= 0) return hipSuccess;
  rel_rows_kernel<<<unsigned((n + 255) / 256), 256, 0, st>>>((const uint4*)dq_r, (const uint4*)dk_r, (uint4*)dst,
                                                              H, R, D);
  return hipGetLastError();
}

hipError_t launch_proj_reduce(const float* part, int nch, int nrel, int M, int E, int dtype, void* out, void* db,
                              hipStream_t st) {
  const int64_t n = int64_t(M) * (E + 1);
  if (n <= 0) return hipSuccess;
  const unsigned nb = unsigned((n + 255) / 256);
  if (dtype == DF_FP16_T)
    proj_reduce_kernel<DF_FP16_T><<<nb, 256, 0, st>>>(part, nch, nrel, M, E, (uint16_t*)out, (uint16_t*)db);
  else
    proj_reduce_kernel<DF_BF16_T><<<nb, 256, 0, st>>>(part, nch, nrel, M, E, (uint16_t*)out, (uint16_t*)db);
  return hipGetLastError();
}

}  // namespace dfa
