// Relative-position strips: the L x R score products that the C2P and P2C
// terms gather from (DisentangledFlash 1.1.1 page, "Performance": the C2P and
// P2C relative-position score products, 4LRD FLOPs of the forward count).
//
//   c2ps[h][t][r] = s*log2(e) * Q[t,h,:] . K_r[h,r,:]
//   p2cs[h][t][r] = s*log2(e) * K[t,h,:] . Q_r[h,r,:]
//
// stored in the working dtype, pre-scaled into the log2 domain the attention
// kernels use, rows padded to RP. Columns 0 and R-1 (the rows every
// far-field pair saturates to) are also written contiguously per head into
// `ends` [4][H][T].
//
// One workgroup computes a 128-token x 64-row tile of one strip (blockIdx.z
// selects strip and head): 4 waves, each 32 tokens x 2 MFMA column tiles,
// K = D in one pass, operands straight from global memory. The tile is
// converted in registers, staged in LDS and written back as whole 16-byte
// chunks of each row (the kernel is bound by its HBM writes).
#include "common.hpp"

namespace dfa {

namespace {

template <int DT, int D>
__global__ __launch_bounds__(256) void strip_kernel(Params p) {
  using TR = Tr<DT>;
  using T = typename TR::T;
  using frag = typename TR::frag;
  constexpr int E = TR::E, KS = TR::KS, NQ = D / KS;
  constexpr int TM = 128, TN = 64;
  constexpr int CH = 16 / int(sizeof(T));
  constexpr int OP = TN + CH;  // LDS pitch of the output tile
  __shared__ __align__(16) T tile[TM * OP];

  const int lane = threadIdx.x & 63, g = lane >> 5, li = lane & 31;
  const int wave = threadIdx.x >> 6;
  const int which = blockIdx.z / p.H, h = blockIdx.z % p.H;
  const int64_t t0 = int64_t(blockIdx.x) * TM;
  const int r0 = blockIdx.y * TN;
  const T* A = (const T*)(which ? p.k : p.q);
  const T* B = (const T*)(which ? p.qr : p.kr);
  T* out = (T*)(which ? p.p2cs : p.c2ps);

  const int64_t ta = t0 + wave * 32 + li;
  const bool a_ok = ta < p.T;
  const T* arow = A + (a_ok ? ta : 0) * p.ts + int64_t(h) * p.hs;
  const T* brow[2];
  bool b_ok[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r = r0 + 32 * nt + li;
    b_ok[nt] = r < p.R;
    brow[nt] = B + (int64_t(h) * p.R + (b_ok[nt] ? r : 0)) * D;
  }
  f32x16 acc[2] = {zero16(), zero16()};
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    frag a = a_ok ? TR::ld(arow + q * KS + g * E) : TR::zero();
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      frag b = b_ok[nt] ? TR::ld(brow[nt] + q * KS + g * E) : TR::zero();
      acc[nt] = TR::mma(a, b, acc[nt]);
    }
  }
  // C[m = token][n = row]: lane holds row 32nt + li, tokens acc_row(v, g)
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      tile[(wave * 32 + acc_row(v, g)) * OP + 32 * nt + li] = TR::from_f(acc[nt][v] * p.scale_log2);
  __syncthreads();

  const int64_t HT = int64_t(p.H) * p.T;
  T* ends = (T*)p.ends + (which ? 2 : 0) * HT + int64_t(h) * p.T;
  T* obase = out + int64_t(h) * p.T * p.RP;
  for (int it = threadIdx.x; it < TM * (TN / CH); it += 256) {
    const int m = it / (TN / CH), c = (it % (TN / CH)) * CH;
    const int64_t t = t0 + m;
    if (t >= p.T || r0 + c >= p.RP) continue;
    *reinterpret_cast<uint4*>(obase + t * p.RP + r0 + c) = *reinterpret_cast<const uint4*>(&tile[m * OP + c]);
  }
  if (threadIdx.x < TM) {
    const int m = threadIdx.x;
    const int64_t t = t0 + m;
    if (t < p.T) {
      if (r0 == 0) ends[t] = tile[m * OP];
      const int last = p.R - 1 - r0;
      if (last >= 0 && last < TN) ends[HT + t] = tile[m * OP + last];
    }
  }
}

template <int DT>
void launch_strips_dt(const Params& p, hipStream_t st) {
  dim3 grid(unsigned((p.T + 127) / 128), unsigned((p.R + 63) / 64), unsigned(2 * p.H));
  switch (p.D) {
    case 32: strip_kernel<DT, 32><<<grid, 256, 0, st>>>(p); break;
    case 64: strip_kernel<DT, 64><<<grid, 256, 0, st>>>(p); break;
    default: strip_kernel<DT, 128><<<grid, 256, 0, st>>>(p); break;
  }
}

}  // namespace

hipError_t launch_strips(const Params& p, hipStream_t st) {
  if (p.T == 0) return hipSuccess;
  switch (p.dtype) {
    case DF_BF16_T: launch_strips_dt<DF_BF16_T>(p, st); break;
    case DF_FP16_T: launch_strips_dt<DF_FP16_T>(p, st); break;
    default: launch_strips_dt<DF_FP32_T>(p, st); break;
  }
  return hipGetLastError();
}

}  // namespace dfa
