// Backward preprocess: Delta[h][t] = sum_d dO[t,h,d] * O[t,h,d], the row term
// of the softmax gradient dS = P (dP - Delta) (DisentangledFlash 1.1.1 page,
// "Hugging Face usage" / "Performance": the fused backward that recomputes the
// score products instead of storing the attention matrix).
//
// A work-group covers 64 tokens x 4 heads. Each (token, head) row is read as
// D/CH 16-byte chunks by D/CH neighbouring threads (the 4 heads of a token are
// contiguous, so a pass reads whole cache lines) and reduced with a fixed
// butterfly, so the result does not depend on timing. The sums go through LDS
// so that Delta, stored head-major, is written in whole 64-token runs.
#include "common.hpp"

namespace dfa {

namespace {

constexpr int kTB = 64, kHB = 4;  // tokens x heads per work-group

template <int DT, int D>
__global__ __launch_bounds__(256) void delta_kernel(Params p) {
  using TR = Tr<DT>;
  using T = typename TR::T;
  constexpr int CH = 16 / sizeof(T), G = D / CH;  // threads per row
  constexpr int RPP = 256 / G;                     // rows per pass
  constexpr int NP = kTB * kHB / RPP;              // passes
  __shared__ float sum_s[kHB][kTB];
  const int tid = threadIdx.x;
  const int64_t t0 = int64_t(blockIdx.x) * kTB;
  const int h0 = blockIdx.y * kHB;
  const int c = (tid % G) * CH;
  constexpr int NB = NP < 8 ? NP : 8;  // passes whose loads are issued together
  static_assert(NP % NB == 0, "whole batches");
#pragma unroll
  for (int k0 = 0; k0 < NP; k0 += NB) {
    uint4 a[NB], b[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int r = (k0 + u) * RPP + tid / G, tl = r / kHB, hl = r % kHB;
      const int64_t t = t0 + tl;
      const int h = h0 + hl;
      a[u] = b[u] = make_uint4(0, 0, 0, 0);
      if (t < p.T && h < p.H) {
        const int64_t o = t * p.ts + int64_t(h) * p.hs + c;
        a[u] = *reinterpret_cast<const uint4*>((const T*)p.out + o);
        b[u] = *reinterpret_cast<const uint4*>((const T*)p.dout + o);
      }
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const T* ae = reinterpret_cast<const T*>(&a[u]);
      const T* be = reinterpret_cast<const T*>(&b[u]);
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < CH; ++e) s += TR::to_f(ae[e]) * TR::to_f(be[e]);
#pragma unroll
      for (int o = G / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, G);
      const int r = (k0 + u) * RPP + tid / G;
      if (c == 0) sum_s[r % kHB][r / kHB] = s;
    }
  }
  __syncthreads();
  const int hl = tid / kTB, tl = tid % kTB;
  const int64_t t = t0 + tl;
  if (t < p.T && h0 + hl < p.H) p.delta[int64_t(h0 + hl) * p.T + t] = sum_s[hl][tl];
}

template <int DT>
void launch_dt(const Params& p, hipStream_t st) {
  const dim3 grid(unsigned((p.T + kTB - 1) / kTB), unsigned((p.H + kHB - 1) / kHB));
  switch (p.D) {
    case 32: delta_kernel<DT, 32><<<grid, 256, 0, st>>>(p); break;
    case 64: delta_kernel<DT, 64><<<grid, 256, 0, st>>>(p); break;
    default: delta_kernel<DT, 128><<<grid, 256, 0, st>>>(p); break;
  }
}

}  // namespace

hipError_t launch_bwd_pre(const Params& p, hipStream_t st) {
  if (p.T == 0) return hipSuccess;
  switch (p.dtype) {
    case DF_BF16_T: launch_dt<DF_BF16_T>(p, st); break;
    case DF_FP16_T: launch_dt<DF_FP16_T>(p, st); break;
    default: launch_dt<DF_FP32_T>(p, st); break;
  }
  return hipGetLastError();
}

}  // namespace dfa
