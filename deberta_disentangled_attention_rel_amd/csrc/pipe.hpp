// Row tiles of a [T,H,D] tensor (one head): register prefetch from global
// memory, 16-byte stores into a row-major LDS tile, and MFMA fragment reads.
//
// Fragments read from a row-major LDS tile X (pitch P elements):
//  * ld_row: 8 (16-bit) or 1 (fp32) consecutive elements of one row, for an
//    operand whose lane index is the tile row and whose contraction index
//    runs along the row;
//  * ld_col: for an operand whose lane index is the tile COLUMN and whose
//    contraction index runs down the rows, lane (li, g) needs
//      X[r0 + 4g + s][c0 + li], X[r0 + 8 + 4g + s][c0 + li], s = 0..3
//    (16-bit; the register order of a 32x32 accumulator fed back as an
//    operand) or X[r0 + acc_row(q, g)][c0 + li] (fp32). For 16-bit types this
//    is two gfx950 transposing LDS reads: within each 16-lane group, lane i
//    receives element i % 4 of the 8-byte words addressed by lanes
//    4k + i / 4 (k = 0..3), so pointing source lane s of the group at row
//    r0 + 4g + s/4, column c0 + 16*(group parity) + 4*(s % 4) hands lane i
//    rows r0 + 4g + k of column c0 + li.
#pragma once

#include "common.hpp"

namespace dfa {

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <typename TR>
__device__ __forceinline__ typename TR::frag ld_row(const typename TR::T* X, int P, int row, int col) {
  return TR::ld(X + row * P + col);
}

// Row interleave inside each group of 8 LDS rows: row 4h + m (h < 2, m < 4)
// sits at slot 2m + h. A transposing read takes rows 4h .. 4h+3 of a group in
// one half-wave (64 bytes of each); interleaved, they sit at slots 2m + h,
// whose pieces fall on disjoint banks of the 64 for the V / Q / dO pitch
// (D + 16 elements), where consecutive rows wrap onto each other.
__device__ __forceinline__ constexpr int swz8_slot(int row) { return (row & ~7) | ((row & 3) << 1) | ((row >> 2) & 1); }
__device__ __forceinline__ constexpr int swz8_row(int slot) { return (slot & ~7) | ((slot & 1) << 2) | ((slot >> 1) & 3); }

// Column fragment for contraction step q: rows r0 + 16q + {4g..4g+3, 8+4g..8+4g+3}
// (16-bit, two transposing reads) or row r0 + acc_row(q, g) (fp32), column
// c0 + (lane % 32). SWZ: the 16-bit tile's rows are interleaved (swz8_slot;
// r0 a multiple of 8).
template <typename TR, bool SWZ = false>
__device__ __forceinline__ typename TR::frag ld_col(const typename TR::T* X, int P, int r0, int c0, int q) {
  using T = typename TR::T;
  const int lane = threadIdx.x & 63;
  if constexpr (TR::E == 8) {
    const int b = lane >> 4, s = lane & 15;
    const int rr = SWZ ? swz8_slot(4 * (b >> 1) + (s >> 2)) : 4 * (b >> 1) + (s >> 2);
    const T* a = X + (r0 + 16 * q + rr) * P + c0 + 16 * (b & 1) + 4 * (s & 3);
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 8 * P));
    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(typename TR::frag, make_uint4(l2.x, l2.y, h2.x, h2.y));
  } else {
    return X[(r0 + acc_row(q, lane >> 5)) * P + c0 + (lane & 31)];
  }
}

// Pitches (elements) of row-major tiles. 16-bit: +8 keeps rows 16-byte
// aligned and puts consecutive rows 4 banks apart (conflict-free 16-byte row
// reads); tiles read only through ld_col use +16 (the four rows of a
// transposing read land 8 banks apart). fp32: odd pitch.
template <typename T, int W> struct RowPitch {
  static constexpr int rows = sizeof(T) == 2 ? W + 8 : W + 1;
  static constexpr int cols = sizeof(T) == 2 ? W + 16 : W + 1;
};

// Half-major partner order. A block of 32*NS partners (keys or queries) is
// processed as NS MFMA subtiles of 32; storing partner p at LDS row
// half_major_slot(p) makes register v of lane group g in subtile t hold
// partner half_major_partner(t, g, v) = 16*NS*g + 16t + v: lane group 0 holds
// partners [0, 16NS) and group 1 [16NS, 32NS), each in increasing order of
// (t, v). The fragment reads of the tile are unchanged; only the partner an
// LDS row stands for changes.
template <int NS>
__device__ __forceinline__ constexpr int half_major_partner(int t, int g, int v) {
  return 16 * NS * g + 16 * t + v;
}
// LDS row of partner p, and its inverse: the partner stored at LDS row
// `slot` (slot = 32t + acc_row(v, g)).
template <int NS>
__device__ __forceinline__ constexpr int half_major_slot(int p) {
  const int g = p / (16 * NS), t = (p % (16 * NS)) / 16, v = p % 16;
  return 32 * t + acc_row(v, g);
}
template <int NS>
__device__ __forceinline__ constexpr int half_major_at(int slot) {
  const int t = slot >> 5, m = slot & 31;
  const int g = (m >> 2) & 1, v = 4 * (m >> 3) + (m & 3);
  return half_major_partner<NS>(t, g, v);
}

// A ROWS x D tile of one head of a [T,H,D] tensor, prefetched into registers
// by all NT threads (16-byte chunks) and committed to a row-major LDS tile
// (tile row p at LDS row p, or half_major_slot(p) with HALF_MAJOR).
template <typename T, int ROWS, int D, int NT, bool HALF_MAJOR = false>
struct RowTile {
  static constexpr int CH = 16 / int(sizeof(T));
  static constexpr int NC = D / CH;
  static constexpr int CHUNKS = ROWS * NC;
  static constexpr int PER = (CHUNKS + NT - 1) / NT;
  uint4 r[PER];

  // chunk u of this thread: tile row and column (recomputed at each use
  // instead of being held in registers across the loop)
  static __device__ __forceinline__ int row_of(int u) {
    const int it = threadIdx.x + u * NT;
    return it < CHUNKS ? it / NC : ROWS;  // ROWS marks an idle slot
  }
  static __device__ __forceinline__ int col_of(int u) { return ((threadIdx.x + u * NT) % NC) * CH; }

  __device__ __forceinline__ void init() {}
  // rows row0 .. row0+ROWS-1 of `base` (token stride ts); rows >= nvalid -> 0
  __device__ __forceinline__ void load(const T* __restrict__ base, int64_t ts, int row0, int nvalid) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int row = row_of(u);
      r[u] = make_uint4(0, 0, 0, 0);
      if (row < ROWS && row0 + row < nvalid)
        r[u] = *reinterpret_cast<const uint4*>(base + int64_t(row0 + row) * ts + col_of(u));
    }
  }
  // the same rows through a buffer view of the sequence's rows (token stride
  // ts elements): row0 * ts * sizeof(T) = soff; rows past the view load zero
  // with no branch
  __device__ __forceinline__ void load_buf(BufView b, int64_t ts, int soff) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int row = row_of(u);
      const int voff = row < ROWS ? int(row * ts * int64_t(sizeof(T))) + col_of(u) * int(sizeof(T)) : kBufSkip;
      r[u] = buf_load16(b, voff, soff);
    }
  }
  template <int P>
  __device__ __forceinline__ void store(T* __restrict__ lds) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int row = row_of(u);
      if (row < ROWS) {
        const int off = (HALF_MAJOR ? half_major_slot<ROWS / 32>(row) : row) * P + col_of(u);
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint4*>(lds + off) = r[u];
        } else {
          // odd fp32 pitch: rows are only 4-byte aligned
          float* d = reinterpret_cast<float*>(lds) + off;
          const float* s = reinterpret_cast<const float*>(&r[u]);
          d[0] = s[0];
          d[1] = s[1];
          d[2] = s[2];
          d[3] = s[3];
        }
      }
    }
  }
};

// Asynchronous copy of a ROWS x D tile of one head of a [T,H,D] tensor of a
// 16-bit type into a row-major LDS tile of pitch P elements (P a multiple of
// 8) with LDS-DMA loads, which bypass registers: every lane's 16 bytes land
// at the instruction's (wave-uniform) LDS address + 16 * lane, so the NT
// threads fill consecutive 16-byte slots. Slot s is LDS row s / (P/8), chunk
// s % (P/8); chunks past D/8 are row padding and load a duplicate of chunk 0.
// LDS row n holds tile row n, or half_major_at(n) with HALF_MAJOR. Rows >=
// nvalid re-read row nvalid - 1 (finite data; the kernels mask those rows
// through their bias). Completion: s_waitcnt vmcnt(0) by every thread, then
// a barrier.
template <typename T, int ROWS, int D, int P, int NT, bool HALF_MAJOR = false>
struct DmaTile {
  static_assert(sizeof(T) == 2 && P % 8 == 0 && D % 8 == 0, "16-bit rows of whole 16-byte chunks");
  static constexpr int PC = P / 8, NC = D / 8;
  static constexpr int SLOTS = ROWS * PC;
  static constexpr int NI = (SLOTS + NT - 1) / NT;

  static __device__ __forceinline__ void issue(T* lds, const T* base, int64_t ts, int row0, int nvalid) {
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int s0 = k * NT + wave * 64;  // first slot of this wave's instruction
      if (s0 >= SLOTS) break;             // wave-uniform
      const int s = k * NT + int(threadIdx.x);
      if (s < SLOTS) {
        const int slot = s / PC, c = s % PC;
        const int row = HALF_MAJOR ? half_major_at<ROWS / 32>(slot) : slot;  // tile row stored at this LDS row
        const int r = min(row0 + row, nvalid - 1);
        const T* src = base + int64_t(r) * ts + (c < NC ? c : 0) * 8;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                         (__attribute__((address_space(3))) void*)(lds + s0 * 8), 16,
                                         0, 0);
      }
    }
  }
};

// The same copy through a buffer view of one sequence's rows of one head
// (`bytes` = rows x token stride x element size): each thread's byte offsets
// within a tile are fixed (init), the tile's first row enters as a scalar
// offset, so issuing a tile takes no address arithmetic. Rows at or past the
// end of the view, and the row-padding chunks, load zeros without touching
// memory (the hardware range check).
// SWZ interleaves the rows (LDS slot n holds logical row swz8_row(n)).
template <typename T, int ROWS, int D, int P, int NT, bool HALF_MAJOR = false, bool SWZ = false>
struct DmaRows {
  static constexpr int PC = P / 8, NC = D / 8;
  static constexpr int SLOTS = ROWS * PC;
  static constexpr int NI = (SLOTS + NT - 1) / NT;
  int voff[NI];

  __device__ __forceinline__ void init(int64_t ts) {
    static_assert(sizeof(T) == 2 && P % 8 == 0 && D % 8 == 0, "16-bit rows of whole 16-byte chunks");
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int s = k * NT + int(threadIdx.x);
      const int slot = s / PC, c = s % PC;
      const int lrow = SWZ ? swz8_row(slot) : slot;
      const int row = HALF_MAJOR ? half_major_at<ROWS / 32>(lrow) : lrow;
      voff[k] = (s < SLOTS && c < NC) ? int(row * ts * int64_t(sizeof(T))) + c * 16 : kBufSkip;
    }
  }
  // rows row0 .. row0 + ROWS - 1 of the view, row0 * ts * sizeof(T) = soff
  __device__ __forceinline__ void issue(T* lds, BufView b, int soff) const {
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int s0 = k * NT + wave * 64;
      if (s0 >= SLOTS) break;  // wave-uniform
      if (k * NT + int(threadIdx.x) < SLOTS) {
        // device pass only: in the host pass this builtin inside the kernels'
        // lambdas silently drops the kernels' launch stubs
#if defined(__HIP_DEVICE_COMPILE__)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(b.r, (__attribute__((address_space(3))) void*)(lds + s0 * 8), 16,
                                                 voff[k], soff, 0, 0);
#endif
      }
    }
  }
};

// Wait for this thread's outstanding vector-memory loads, LDS-DMA included
// (vmcnt(0); export and LDS counters left alone).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this thread's vector-memory operations are still
// outstanding: they complete in issue order, so every one issued before the
// last N is done (vmcnt(N); bits 3:0 and 15:14 of the count).
template <int N>
__device__ __forceinline__ void wait_vmem_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

}  // namespace dfa
