// Global -> LDS staging of token tiles of a [T,H,D] tensor (one head).
// Rows past `nvalid` are written as zeros, so the MFMA loops need no guards.
#pragma once

#include "common.hpp"

namespace dfa {

// Row-major copy: dst[r * PR + c] = src[(row0 + r) tokens][c], 16-byte chunks,
// consecutive threads on consecutive chunks of a row (coalesced).
template <typename T, int D, int ROWS, int PR, int NT>
__device__ __forceinline__ void stage_rows(T* __restrict__ dst, const T* __restrict__ src,
                                           int64_t ts, int row0, int nvalid) {
  constexpr int CH = 16 / sizeof(T);
  constexpr int NC = D / CH;
  for (int it = threadIdx.x; it < ROWS * NC; it += NT) {
    const int r = it / NC, c = (it % NC) * CH;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (row0 + r < nvalid) val = *reinterpret_cast<const uint4*>(src + int64_t(row0 + r) * ts + c);
    *reinterpret_cast<uint4*>(dst + r * PR + c) = val;
  }
}

// Row-major and/or transposed copy. Transposed: dstT[c * PT + r]. For 16-bit
// types each work item takes two consecutive rows so that the transposed
// stores are whole dwords (row pair packed), consecutive lanes on consecutive
// row pairs.
template <typename T, int D, int ROWS, int PR, int PT, int NT>
__device__ __forceinline__ void stage_rows_tr(T* __restrict__ dst, T* __restrict__ dstT,
                                              const T* __restrict__ src, int64_t ts, int row0,
                                              int nvalid) {
  constexpr int CH = 16 / sizeof(T);
  constexpr int NC = D / CH;
  if constexpr (sizeof(T) == 2) {
    static_assert(ROWS % 2 == 0 && PT % 2 == 0, "row pairs");
    constexpr int RP = ROWS / 2;
    for (int it = threadIdx.x; it < RP * NC; it += NT) {
      const int r = 2 * (it % RP), c = (it / RP) * CH;
      uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
      if (row0 + r < nvalid) a = *reinterpret_cast<const uint4*>(src + int64_t(row0 + r) * ts + c);
      if (row0 + r + 1 < nvalid) b = *reinterpret_cast<const uint4*>(src + int64_t(row0 + r + 1) * ts + c);
      if (dst) {
        *reinterpret_cast<uint4*>(dst + r * PR + c) = a;
        *reinterpret_cast<uint4*>(dst + (r + 1) * PR + c) = b;
      }
      const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (aw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        const uint32_t hi = (bw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        *reinterpret_cast<uint32_t*>(dstT + (c + e) * PT + r) = lo | (hi << 16);
      }
    }
  } else {
    for (int it = threadIdx.x; it < ROWS * NC; it += NT) {
      const int r = it % ROWS, c = (it / ROWS) * CH;
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
      if (row0 + r < nvalid) a = *reinterpret_cast<const float4*>(src + int64_t(row0 + r) * ts + c);
      if (dst) *reinterpret_cast<float4*>(dst + r * PR + c) = a;
      dstT[(c + 0) * PT + r] = a.x;
      dstT[(c + 1) * PT + r] = a.y;
      dstT[(c + 2) * PT + r] = a.z;
      dstT[(c + 3) * PT + r] = a.w;
    }
  }
}

// LDS row pitches (elements). 16-bit: +8 keeps rows 16-byte aligned and moves
// consecutive rows by 4 banks; transposed tiles read 8 bytes at a time and use
// +4. fp32: +4 / +1.
template <typename T, int W> struct Pitch {
  static constexpr int rm = W + (sizeof(T) == 2 ? 8 : 4);
  static constexpr int tr = W + (sizeof(T) == 2 ? 4 : 1);
};

}  // namespace dfa
