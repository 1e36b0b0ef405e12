// Tile classes and LDS staging of the relative-position terms.
//
// A tile covers queries [i0, i0+BM) and keys [j0, j0+BN); its pairs have
// d = i - j in [dlo, dhi] = [i0 - j0 - BN + 1, i0 + BM - 1 - j0].
//  * far-left  (dlo >= d_hi): every pair uses C2P row R-1 and P2C row 0, so
//    the C2P term is one value per query and the P2C term one value per key;
//  * far-right (dhi <= d_lo): C2P row 0 and P2C row R-1, likewise;
//  * band: anything else. The pair's rows come from the index tables (a
//    slice of BM+BN-1 entries, packed c2p | p2c << 16, staged in LDS; the
//    narrow kernels store them as byte offsets) and the values from LDS
//    windows of the strips (a kernel may instead read the term whose row is
//    shared by the lanes of a half straight from the strip):
//      C2P window, one row per query il: strip columns [cs_il, cs_il + BN + 8)
//        with cs_il = c2p[i0+il - (j0+BN-1)] rounded down to 8 (the smallest
//        row the query meets in this tile);
//      P2C window, one row per key jl: columns [ps_jl, ps_jl + BM + 8) with
//        ps_jl = p2c[i0+BM-1 - (j0+jl)] rounded down to 8.
//    When no table ever steps by more than one row ("narrow" tables), BN
//    consecutive d meet at most BN rows, so the windows hold every value the
//    tile needs.
#pragma once

#include "tiles.hpp"

namespace dfa {

enum { TILE_BAND = 0, TILE_FAR_LEFT = 1, TILE_FAR_RIGHT = 2 };

__device__ __forceinline__ int tile_class(int dlo, int dhi, int d_hi, int d_lo) {
  if (dlo >= d_hi) return TILE_FAR_LEFT;
  if (dhi <= d_lo) return TILE_FAR_RIGHT;
  return TILE_BAND;
}

// ends[4][H][T]: C2P column 0, C2P column R-1, P2C column 0, P2C column R-1.
// Index of the end array holding a tile's per-query C2P / per-key P2C value.
__device__ __forceinline__ int c2p_end_of(int cls) { return cls == TILE_FAR_LEFT ? 1 : 0; }
__device__ __forceinline__ int p2c_end_of(int cls) { return cls == TILE_FAR_LEFT ? 2 : 3; }

// Packed table entry for d (clamped to the table).
__device__ __forceinline__ uint32_t lut_entry(const Params& p, int d) {
  const int off = p.Lmax - 1;
  const int n = d < -off ? 0 : (d > off ? 2 * off : d + off);
  return uint32_t(p.c2p[n]) | (uint32_t(p.p2c[n]) << 16);
}

__device__ __forceinline__ int lut_c(uint32_t e) { return int(e & 0xffffu); }
__device__ __forceinline__ int lut_p(uint32_t e) { return int(e >> 16); }

// The same entry with both rows scaled to byte offsets into rows of ES-byte
// elements (narrow kernels: the window gathers then need one add each).
template <int ES>
__device__ __forceinline__ uint32_t lut_entry_bytes(const Params& p, int d) {
  const uint32_t e = lut_entry(p, d);
  return (e & 0xffffu) * ES | ((e >> 16) * ES) << 16;
}
// Byte offset of the 8-element-aligned window start below a scaled row.
template <int ES>
__device__ __forceinline__ int win_start_bytes(int row_bytes) {
  return row_bytes & ~(8 * ES - 1);
}

// Row pitches (elements) of the strip windows: an odd number of dwords for
// 16-bit types (odd number of floats for fp32), so that lanes reading
// different rows at nearby columns fall in different banks.
template <typename T, int W> struct WinPitch {
  static constexpr int v = sizeof(T) == 2 ? W + 2 : W + 1;
};

// Stage `rows` skewed strip rows into LDS. Row r reads strip row
// base_row + min(row0 + r, nvalid - 1) (clamped so every load is in bounds),
// columns [start(r), start(r) + WCOLS) where start(r) is a multiple of 8;
// columns at or past RP are zero.
template <typename T, int WCOLS, int PITCH, int NT, class StartFn>
__device__ __forceinline__ void stage_window(T* __restrict__ dst, const T* __restrict__ strip, int RP,
                                             int rows, int row0, int nvalid, StartFn start) {
  constexpr int CH = 16 / sizeof(T);
  constexpr int NC = WCOLS / CH;
  for (int it = threadIdx.x; it < rows * NC; it += NT) {
    const int r = it / NC, c = (it % NC) * CH;
    const int col = start(r) + c;
    const int rr = min(row0 + r, nvalid - 1);
    uint4 val = make_uint4(0, 0, 0, 0);
    if (col < RP) val = *reinterpret_cast<const uint4*>(strip + int64_t(rr) * RP + col);
    uint32_t* d = reinterpret_cast<uint32_t*>(dst + r * PITCH + c);
    d[0] = val.x;
    d[1] = val.y;
    d[2] = val.z;
    d[3] = val.w;
  }
}

// A strip window in LDS filled by LDS-DMA (16-bit types): ROWS rows of CPR
// 16-byte chunks; with PAD16 one padding chunk follows every 16 rows, so lanes
// reading different rows at nearby columns spread over the banks. Row r sits
// at element row_offset(r). Slot s of the copy (16 bytes each, consecutive
// lanes filling consecutive slots) holds chunk `chunk` of row `row` (row -1:
// padding, loads a harmless duplicate).
template <typename T, int ROWS, int CPR, bool PAD16, int NT>
struct WinDma {
  static_assert(sizeof(T) == 2 && ROWS % 16 == 0, "16-bit rows, whole groups of 16");
  static constexpr int GROUP = 16 * CPR + (PAD16 ? 1 : 0);
  static constexpr int SLOTS = (ROWS / 16) * GROUP;
  static constexpr int NI = (SLOTS + NT - 1) / NT;
  static constexpr int ELEMS = SLOTS * 8;

  static __device__ __forceinline__ constexpr int row_offset(int r) {
    return (r * CPR + (PAD16 ? r / 16 : 0)) * 8;
  }
  static __device__ __forceinline__ void slot(int s, int& row, int& chunk) {
    const int grp = s / GROUP, rem = s % GROUP;
    const bool pad = PAD16 && rem == 16 * CPR;
    row = pad ? -1 : grp * 16 + rem / CPR;
    chunk = pad ? 0 : rem % CPR;
  }
  // Copy strip rows row0 + r (clamped to nvalid - 1), columns from
  // start_of(k, r) (a multiple of 8, k = this thread's instruction index).
  // The strip is read through a buffer view of the sequence's strip rows
  // (RP elements each): buffer LDS-DMA copies, unlike global ones, let the
  // compiler see that later LDS reads of other buffers do not depend on
  // them.
  // Copy strip rows row0 + r (clamped to nvalid - 1), columns from
  // start_of(k, r), with global LDS-DMA loads from `strip` (the strip rows
  // of the sequence and head).
  template <class StartFn>
  static __device__ __forceinline__ void issue_global(T* lds, const T* strip, int RP, int row0, int nvalid,
                                                      StartFn start_of) {
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int s0 = k * NT + wave * 64;
      if (s0 >= SLOTS) break;  // wave-uniform
      const int s = k * NT + int(threadIdx.x);
      if (s < SLOTS) {
        int row, chunk;
        slot(s, row, chunk);
        const int rr = row < 0 ? 0 : row;
        const int r = min(row0 + rr, nvalid - 1);
        // chunks past the strip row are never read; keep the copy in bounds
        const int col = min(start_of(k, rr) + chunk * 8, RP - 8);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(strip + int64_t(r) * RP + col),
                                         (__attribute__((address_space(3))) void*)(lds + s0 * 8), 16, 0, 0);
      }
    }
  }
  template <class StartFn>
  static __device__ __forceinline__ void issue(T* lds, BufView strip, int RP, int row0, int nvalid,
                                               StartFn start_of) {
    const int wave = threadIdx.x >> 6;
    // the thread index is taken through an empty asm statement so the slot
    // arithmetic below is redone per call instead of being hoisted out of
    // the caller's tile loop (where its results would stay live)
    int tx = int(threadIdx.x);
    asm volatile("" : "+v"(tx));
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int s0 = k * NT + wave * 64;
      if (s0 >= SLOTS) break;  // wave-uniform
      const int s = k * NT + tx;
      if (s < SLOTS) {
        int row, chunk;
        slot(s, row, chunk);
        const int rr = row < 0 ? 0 : row;
        const int r = min(row0 + rr, nvalid - 1);
        // chunks past the strip row are never read; keep the copy in bounds
        const int col = min(start_of(k, rr) + chunk * 8, RP - 8);
        // device pass only: in the host pass this builtin inside the kernels'
        // lambdas silently drops the kernels' launch stubs
#if defined(__HIP_DEVICE_COMPILE__)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(strip.r, (__attribute__((address_space(3))) void*)(lds + s0 * 8), 16,
                                                 (r * RP + col) * int(sizeof(T)), 0, 0, 0);
#endif
      }
    }
  }
};

// The forward's C2P window of a band tile (one row of BN + 8 = 72 columns per
// query), copied one tile ahead into one of two buffers. The start column of
// each row (its smallest C2P row in the tile, rounded down to 8) comes from
// the index table in global memory, loaded one tile before the copy is issued
// (load_starts), so issuing never waits on it.
template <typename T, int ROWS, int NT>
struct C2PWindowDma {
  using W = WinDma<T, ROWS, 9, true, NT>;
  static constexpr int NI = W::NI;
  static constexpr int ELEMS = W::ELEMS;
  int start[NI];  // smallest C2P row of this thread's rows in the next window

  static __device__ __forceinline__ constexpr int row_offset(int il) { return W::row_offset(il); }
  // rows of the tile whose smallest relative distance is dmin + row
  __device__ __forceinline__ void load_starts(const Params& p, int dmin) {
    const int off = p.Lmax - 1;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int s = k * NT + int(threadIdx.x);
      int row, chunk;
      W::slot(s, row, chunk);
      const int d = dmin + (row < 0 ? 0 : row);
      const int n = d < -off ? 0 : (d > off ? 2 * off : d + off);
      start[k] = p.c2p[n];  // raw: rounded when the copy is issued, so nothing waits for it here
    }
  }
  __device__ __forceinline__ void issue(T* lds, const T* strip, int RP, int row0, int nvalid) const {
    W::issue_global(lds, strip, RP, row0, nvalid, [&](int k, int) { return start[k] & ~7; });
  }
};

}  // namespace dfa
