// Ordered segmented sum of dS into one dense row of a relative gradient strip.
//
// dC2P[i, r] = sum over keys j with delta(i,j) = r of dS[i,j], and
// dP2C[j, r] = sum over queries i with delta(j,i) = r of dS[i,j].
// Walking a row's partners in increasing order, the index r never increases
// (the bucket is monotone in i - j), so every r is a contiguous run. The
// lane pair that owns a row (lanes l and l ^ 32) walks a tile's partners in
// two halves at once (the tiles are stored half-major, so each lane group's
// registers hold one contiguous half): half 0 takes the first half and
// carries the row's open run across tiles; half 1 takes the second half and
// holds back its first run (the "head"). A merge then joins half 0's open
// run with half 1's head. A run is written when the walk leaves it, rows the
// walk skips are written as zeros, and after the last partner the open run,
// the rows below it and the padding up to RP are written. Every element of
// the row is written exactly once, in a fixed order, by one of the two lanes
// that own the row: no atomics, no initialisation, bitwise-reproducible.
//
// NARROW (no table ever steps by more than one row): the walk never skips a
// row, so a step is a compare, a predicated store and two selects. The rows
// above the first partner's row are zeroed up front (walk_open), and the
// open run always holds a real row.
#pragma once

#include "common.hpp"

namespace dfa {

// Write run (r_from, s) and zeros for the rows strictly between r_to and
// r_from. r_from = R means "no run yet" (everything above r_to is still
// unwritten); r_from < 0 means "nothing open" (write nothing).
template <typename TR>
__device__ __forceinline__ void walk_close(typename TR::T* row, int R, int r_from, float s, int r_to) {
  if (r_from < 0) return;
  if (r_from < R) row[r_from] = TR::from_f(s);
  for (int rr = (r_from < R ? r_from : R) - 1; rr > r_to; --rr) row[rr] = TR::from_f(0.f);
}

// State of one half's walk through a tile.
struct WalkHalf {
  int r;      // open run row (-1: half 1 has met no partner yet)
  float s;    // open run sum
  bool headp; // half 1: the first run has not been closed yet
  int rh;     // half 1: head row
  float sh;   // half 1: head sum
};

// Start of a tile: half 0 continues the row's open run (rc, sc); half 1
// starts at its first partner's row r1 (-1 when it has no partner).
__device__ __forceinline__ WalkHalf walk_begin(int g, int rc, float sc, int r1) {
  return g == 0 ? WalkHalf{rc, sc, false, -1, 0.f} : WalkHalf{r1, 0.f, true, -1, 0.f};
}

// One partner (row r, value v); a step with active == false changes nothing.
template <typename TR, bool NARROW>
__device__ __forceinline__ void walk_step(typename TR::T* row, int R, WalkHalf& w, int r, float v,
                                          bool active = true) {
  if constexpr (NARROW) {
    // predicated: one masked store, no branches
    const bool ch = active && r != w.r;
    if (ch && !w.headp) row[w.r] = TR::from_f(w.s);
    const bool hd = ch && w.headp;
    w.rh = hd ? w.r : w.rh;
    w.sh = hd ? w.s : w.sh;
    w.headp = w.headp && !ch;
    w.s = ch ? v : (active ? w.s + v : w.s);
    w.r = active ? r : w.r;
  } else {
    if (!active) return;
    if (r != w.r) {
      if (w.headp) {
        if (w.r >= 0) {  // close the head: hold its sum, zero the gap below it
          w.rh = w.r;
          w.sh = w.s;
          w.headp = false;
          for (int rr = w.r - 1; rr > r; --rr) row[rr] = TR::from_f(0.f);
        }
      } else {
        walk_close<TR>(row, R, w.r, w.s, r);
      }
      w.r = r;
      w.s = 0.f;
    }
    w.s += v;
  }
}

// The same NARROW step writing through a range-checked view of the rows of
// a work-group (`rbase`: byte offset of this lane's row in the view): the
// store is always issued, with an offset past the view when nothing is
// written, so a step has no branch and no 64-bit address arithmetic.
template <typename TR>
__device__ __forceinline__ void walk_step_narrow(BufView rv, int rbase, WalkHalf& w, int r, float v, bool active) {
  using T = typename TR::T;
  const bool ch = active && r != w.r;
  buf_store<T>(rv, ch && !w.headp ? rbase + w.r * int(sizeof(T)) : kBufSkip, TR::from_f(w.s));
  const bool hd = ch && w.headp;
  w.rh = hd ? w.r : w.rh;
  w.sh = hd ? w.s : w.sh;
  w.headp = w.headp && !ch;
  w.s = ch ? v : (active ? w.s + v : w.s);
  w.r = active ? r : w.r;
}

// Join half 0's open run with what half 1 found; afterwards rc/sc hold the
// row's open run (in half 0 lanes). Called by both halves (cross-lane
// exchange inside), outside any lane-divergent branch.
template <typename TR>
__device__ __forceinline__ void walk_merge(typename TR::T* row, int R, int g, const WalkHalf& w, int& rc,
                                           float& sc, bool owner) {
  // half 1 publishes its head (or its only run) and its open tail run
  const bool single = w.headp;
  const int hr = single ? w.r : w.rh;
  const float hs = single ? w.s : w.sh;
  const int o_hr = __float_as_int(xor32(__int_as_float(hr)));
  const float o_hs = xor32(hs);
  const int o_tr = __float_as_int(xor32(__int_as_float(w.r)));
  const float o_ts = xor32(w.s);
  const int o_single = __float_as_int(xor32(__int_as_float(single ? 1 : 0)));
  if (g != 0 || !owner) return;
  if (o_hr < 0) {  // half 1 had no partners in this tile
    rc = w.r;
    sc = w.s;
    return;
  }
  float merged = o_hs;
  if (w.r == o_hr)
    merged += w.s;
  else
    walk_close<TR>(row, R, w.r, w.s, o_hr);
  if (o_single) {
    rc = o_hr;
    sc = merged;
  } else {
    row[o_hr] = TR::from_f(merged);
    rc = o_tr;
    sc = o_ts;
  }
}

// Before the first tile (NARROW): zero the rows above the first partner's
// row r_first, which becomes the open run.
template <typename TR>
__device__ __forceinline__ void walk_open(typename TR::T* row, int R, int r_first) {
  for (int rr = R - 1; rr > r_first; --rr) row[rr] = TR::from_f(0.f);
}

// After the last tile: the open run, the rows below it and the padding.
template <typename TR>
__device__ __forceinline__ void walk_finish(typename TR::T* row, int R, int RP, int rc, float sc) {
  walk_close<TR>(row, R, rc, sc, -1);
  for (int rr = R; rr < RP; ++rr) row[rr] = TR::from_f(0.f);
}

// Single-walker form: the lane that owns the row (lane group 0) walks all of
// a tile's partners; the other lane group hands over its accumulator rows.
// The open run is kept in registers, written when r changes, with zeros for
// any r the row skips; after the last partner the rest of the row (and its
// padding up to RP) is written.
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
// register file: lane group (k >> 2) & 1, register 4*(k >> 3) + (k & 3).
__device__ __forceinline__ constexpr int walk_grp(int k) { return (k >> 2) & 1; }
__device__ __forceinline__ constexpr int walk_reg(int k) { return 4 * (k >> 3) + (k & 3); }

// Relative-gradient epilogue of the dQ and dK/dV kernels:
//   acc[nd] += relT[32 nd + m][:] . strip[partner][:]
// for the accumulator tiles of a lane's partner (column = this lane's query
// or key, rows m = acc_row(v, g) of d-block nd): dQ^T += K_r^T dC2P^T and
// dK^T += Q_r^T dP2C^T. `rows` views the work-group's strip rows (`row_off`:
// byte offset of this lane's partner row; partners past the sequence read
// zero), `relT` the head's relative rows transposed in 16-byte chunks,
// [RP / CE][D][CE] with CE = 16 bytes of elements (a load instruction's 32
// rows d are then one contiguous run). Chunks at or past RP are skipped (they
// would run into the next row). The strip rows
// must be complete and visible: every lane that wrote them has waited for
// its stores. The contraction runs in batches of U steps, double-buffered:
// a batch's loads go out before the previous batch's MFMAs (a scheduling
// barrier keeps them there), so each batch waits only for loads issued a
// batch earlier. Batches past RP load zeros without touching memory (range
// check) and add nothing, so every batch's loads are issued unconditionally.
template <typename TR, int ND>
__device__ __forceinline__ void rel_epilogue(f32x16 (&acc)[ND], BufView rows, int row_off, BufView relT, int RP) {
  using frag = typename TR::frag;
  constexpr int E = TR::E, KS = TR::KS, ES = int(sizeof(typename TR::T));
  constexpr int U = ND <= 2 ? 4 : 2;  // steps per batch (two batches of U (1 + ND) fragments live)
  constexpr int CE = 16 / ES;  // elements per 16-byte chunk of relT
  const int lane = threadIdx.x & 63, g = lane >> 5, li = lane & 31;
  auto ld = [&](BufView v, int off) -> frag {
    if constexpr (E == 8)
      return __builtin_bit_cast(frag, buf_load16(v, off));
    else
      return buf_load<typename TR::T>(v, off, 0);
  };
  auto load = [&](frag (&b)[U], frag (&a)[U][ND], int r0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * KS + g * E;
      const bool in = r < RP;
      b[u] = ld(rows, in ? row_off + r * ES : kBufSkip);
#pragma unroll
      for (int nd = 0; nd < ND; ++nd)
        a[u][nd] = ld(relT, in ? (((r / CE) * (ND * 32) + 32 * nd + li) * CE + r % CE) * ES : kBufSkip);
    }
  };
  auto mma = [&](const frag (&b)[U], const frag (&a)[U][ND]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) acc[nd] = TR::mma(a[u][nd], b[u], acc[nd]);
  };
  frag b0[U], a0[U][ND], b1[U], a1[U][ND];
  load(b0, a0, 0);
  for (int r0 = 0; r0 < RP; r0 += 2 * U * KS) {
    load(b1, a1, r0 + U * KS);
    __builtin_amdgcn_sched_barrier(0);
    mma(b0, a0);
    __builtin_amdgcn_sched_barrier(0);
    load(b0, a0, r0 + 2 * U * KS);
    __builtin_amdgcn_sched_barrier(0);
    mma(b1, a1);
    __builtin_amdgcn_sched_barrier(0);
  }
}

}  // namespace dfa
