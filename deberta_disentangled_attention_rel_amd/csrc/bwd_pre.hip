// Backward preprocess: Delta[h][t] = sum_d dO[t,h,d] * O[t,h,d], the row term
// of the softmax gradient dS = P (dP - Delta) (DisentangledFlash 1.1.1 page,
// "Hugging Face usage" / "Performance": the fused backward that recomputes the
// score products instead of storing the attention matrix).
//
// Each thread reads one 16-byte chunk of O and dO; the D/CH threads of a row
// reduce with a fixed butterfly, so the result does not depend on timing.
#include "common.hpp"

namespace dfa {

namespace {

template <int DT, int D>
__global__ __launch_bounds__(256) void delta_kernel(Params p) {
  using TR = Tr<DT>;
  using T = typename TR::T;
  constexpr int CH = 16 / sizeof(T), G = D / CH;
  const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = gid / G;  // row = t * H + h
  const int c = int(gid % G) * CH;
  const bool ok = row < p.T * p.H;
  float s = 0.f;
  int64_t t = 0;
  int h = 0;
  if (ok) {
    t = row / p.H;
    h = int(row % p.H);
    const int64_t o = t * p.ts + int64_t(h) * p.hs + c;
    const uint4 a = *reinterpret_cast<const uint4*>((const T*)p.out + o);
    const uint4 b = *reinterpret_cast<const uint4*>((const T*)p.dout + o);
    const T* ae = reinterpret_cast<const T*>(&a);
    const T* be = reinterpret_cast<const T*>(&b);
#pragma unroll
    for (int e = 0; e < CH; ++e) s += TR::to_f(ae[e]) * TR::to_f(be[e]);
  }
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, G);
  if (ok && c == 0) p.delta[int64_t(h) * p.T + t] = s;
}

template <int DT>
void launch_dt(const Params& p, hipStream_t st) {
  const int64_t rows = p.T * p.H;
  const int CH = DT == DF_FP32_T ? 4 : 8;
  const int64_t threads = rows * (p.D / CH);
  const unsigned blocks = unsigned((threads + 255) / 256);
  switch (p.D) {
    case 32: delta_kernel<DT, 32><<<blocks, 256, 0, st>>>(p); break;
    case 64: delta_kernel<DT, 64><<<blocks, 256, 0, st>>>(p); break;
    default: delta_kernel<DT, 128><<<blocks, 256, 0, st>>>(p); break;
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
