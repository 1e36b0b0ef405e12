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
// Both operands are K-contiguous rows, so A and W tiles are copied row-major
// into LDS by buffer LDS-DMA (fixed per-thread offsets, the step's column as
// the scalar offset; rows past the matrix and columns past E load zero) one
// step ahead into the other of two buffers, and both fragments are plain
// 16-byte row reads. Work-groups are renumbered so that each XCD runs a
// contiguous range of tiles, column tile fastest: the tiles of one row block
// share its A rows in that XCD's L2.
#include "pipe.hpp"

namespace dfa {

namespace {

constexpr int PBM = 128, PBN = 128, PBK = 64, PP = PBK + 8;  // tile and LDS row pitch (elements)

// One operand tile (128 rows x 64 columns) per step: slot s = row * 9 + chunk,
// chunk 8 is row padding and never loaded.
struct ProjDma {
  static constexpr int PC = PP / 8, SLOTS = PBM * PC, NI = (SLOTS + 255) / 256;
  int voff[NI];  // byte offset of this thread's chunk in the view, or kBufSkip
  int col[NI];   // element column of the chunk within a step (>= PBK: padding)

  __device__ __forceinline__ void init(int ld_bytes) {
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int s = k * 256 + int(threadIdx.x);
      const int row = s / PC, c = s % PC;
      col[k] = c < PBK / 8 ? c * 8 : PBK;
      voff[k] = (s < SLOTS && c < PBK / 8) ? row * ld_bytes + c * 16 : kBufSkip;
    }
  }
  // columns k0 .. k0 + 63 of the view's rows (K = row length in elements)
  __device__ __forceinline__ void issue(uint16_t* lds, BufView b, int k0, int K) const {
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int s0 = k * 256 + wave * 64;
      if (s0 >= SLOTS) break;  // wave-uniform
      if (k * 256 + int(threadIdx.x) < SLOTS) {
        const int vo = k0 + col[k] < K ? voff[k] : kBufSkip;
#if defined(__HIP_DEVICE_COMPILE__)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(b.r, (__attribute__((address_space(3))) void*)(lds + s0 * 8), 16,
                                                 vo, k0 * 2, 0, 0);
#endif
      }
    }
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

  const int K = p.K;
  const T* A = (const T*)p.a + int64_t(m0) * K;
  const T* W = (const T*)p.w + int64_t(n0) * K;
  const BufView av = buf_view(A, uint32_t(min(PBM, p.M - m0)) * uint32_t(K) * 2u);
  const BufView wv = buf_view(W, uint32_t(min(PBN, p.N - n0)) * uint32_t(K) * 2u);
  ProjDma dma;
  dma.init(K * 2);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = zero16();

  const int nk = (K + PBK - 1) / PBK;
  dma.issue(As[0], av, 0, K);
  dma.issue(Bs[0], wv, 0, K);
  wait_vmem();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      dma.issue(As[buf ^ 1], av, (kt + 1) * PBK, K);
      dma.issue(Bs[buf ^ 1], wv, (kt + 1) * PBK, K);
    }
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
    wait_vmem();
    __syncthreads();
  }

  // lane: column n = n0 + wn*64 + 32j + li; register v: row m0 + wm*64 + 32i + acc_row(v, g)
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
  if (p.dtype == DF_FP16_T)
    proj_kernel<DF_FP16_T><<<nb, 256, 0, st>>>(p);
  else
    proj_kernel<DF_BF16_T><<<nb, 256, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace dfa
