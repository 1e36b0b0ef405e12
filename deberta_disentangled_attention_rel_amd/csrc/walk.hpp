// Ordered segmented sum of dS into one dense row of a relative gradient strip.
//
// dC2P[i, r] = sum over keys j with delta(i,j) = r of dS[i,j], and
// dP2C[j, r] = sum over queries i with delta(j,i) = r of dS[i,j].
// Walking a row's partners in increasing order, the index r never increases
// (the bucket is monotone in i - j), so every r is a contiguous run. The walk
// keeps the open run in registers, writes it when r changes, writes zeros for
// any r the row skips, and after the last partner writes zeros for the rest
// (and the row padding up to RP). Every element of the row is written exactly
// once, in a fixed order, by the lane that owns the row: no atomics, no
// initialisation of the strip, bitwise-reproducible.
#pragma once

#include "common.hpp"

namespace dfa {

template <typename TR>
struct StripWalk {
  using T = typename TR::T;
  T* row;
  int R, RP;
  int r_open;  // R while no run is open
  float s_open;

  __device__ __forceinline__ void init(T* row_, int R_, int RP_) {
    row = row_;
    R = R_;
    RP = RP_;
    r_open = R_;
    s_open = 0.f;
  }
  // close the open run and zero-fill down to (excluding) r
  __device__ __forceinline__ void close_to(int r) {
    if (r_open < R) row[r_open] = TR::from_f(s_open);
    for (int rr = r_open - 1; rr > r; --rr) row[rr] = TR::from_f(0.f);
  }
  __device__ __forceinline__ void step(int r, float val) {
    if (r != r_open) {
      close_to(r);
      r_open = r;
      s_open = 0.f;
    }
    s_open += val;
  }
  __device__ __forceinline__ void finish() {
    close_to(-1);
    for (int rr = R; rr < RP; ++rr) row[rr] = TR::from_f(0.f);
  }
};

// Position of the k-th (0..31) row of a 32-row accumulator tile in the
// register file: lane group k>>2 & 1, register 4*(k>>3) + (k&3).
__device__ __forceinline__ constexpr int walk_grp(int k) { return (k >> 2) & 1; }
__device__ __forceinline__ constexpr int walk_reg(int k) { return 4 * (k >> 3) + (k & 3); }

}  // namespace dfa
