// Device-side building blocks shared by the kernels: dtype traits, MFMA
// wrappers and the lane layout of a 32x32 MFMA accumulator on gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "params.hpp"

namespace dfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// dtype traits. A 32x32 MFMA consumes, per lane, E consecutive elements of a
// K-step of KS (16-bit types: 32x32x16, E = 8; fp32: 32x32x2, E = 1).
//
// Operand convention used everywhere: lane l feeds row (A) or column (B)
// l % 32, from K-group g = l / 32; slot s of group g stands for contraction
// index g*E + s of the step. The hardware pairs equal (group, slot) of A and
// B, so any relabelling of the contraction index that both operands share
// gives the same product.

template <int DT> struct Tr;

template <> struct Tr<DF_BF16_T> {
  using T = uint16_t;
  using frag = bf16x8;
  static constexpr int E = 8, KS = 16;
  static __device__ __forceinline__ float to_f(T x) { return __uint_as_float(uint32_t(x) << 16); }
  static __device__ __forceinline__ T from_f(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag pack(const float* x) {
    frag r;
#pragma unroll
    for (int s = 0; s < 8; ++s) r[s] = (__bf16)x[s];
    return r;
  }
  static __device__ __forceinline__ frag ld(const T* p) {  // 8 consecutive, 16-byte aligned
    return __builtin_bit_cast(frag, *reinterpret_cast<const uint4*>(p));
  }
  static __device__ __forceinline__ frag ld2x4(const T* p0, const T* p1) {  // 4 + 4 consecutive
    uint2 a = *reinterpret_cast<const uint2*>(p0), b = *reinterpret_cast<const uint2*>(p1);
    return __builtin_bit_cast(frag, make_uint4(a.x, a.y, b.x, b.y));
  }
  static __device__ __forceinline__ frag zero() { return __builtin_bit_cast(frag, make_uint4(0, 0, 0, 0)); }
  // a + b + c for two stored values (one packed dot product with (1, 1))
  static __device__ __forceinline__ float add2(T a, T b, float c) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    const uint32_t pk = uint32_t(a) | (uint32_t(b) << 16);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), ones, c, false);
  }
  // c + the sum of a fragment's 8 elements (four packed dot products with (1, 1))
  static __device__ __forceinline__ float sum(frag f, float c) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    const uint4 u = __builtin_bit_cast(uint4, f);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.x), ones, c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.y), ones, c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.z), ones, c, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.w), ones, c, false);
  }
};

template <> struct Tr<DF_FP16_T> {
  using T = uint16_t;
  using frag = f16x8;
  static constexpr int E = 8, KS = 16;
  static __device__ __forceinline__ float to_f(T x) { return (float)__builtin_bit_cast(_Float16, x); }
  static __device__ __forceinline__ T from_f(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag pack(const float* x) {
    frag r;
#pragma unroll
    for (int s = 0; s < 8; ++s) r[s] = (_Float16)x[s];
    return r;
  }
  static __device__ __forceinline__ frag ld(const T* p) {
    return __builtin_bit_cast(frag, *reinterpret_cast<const uint4*>(p));
  }
  static __device__ __forceinline__ frag ld2x4(const T* p0, const T* p1) {
    uint2 a = *reinterpret_cast<const uint2*>(p0), b = *reinterpret_cast<const uint2*>(p1);
    return __builtin_bit_cast(frag, make_uint4(a.x, a.y, b.x, b.y));
  }
  static __device__ __forceinline__ frag zero() { return __builtin_bit_cast(frag, make_uint4(0, 0, 0, 0)); }
  static __device__ __forceinline__ float add2(T a, T b, float c) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    const uint32_t pk = uint32_t(a) | (uint32_t(b) << 16);
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk), ones, c, false);
  }
  static __device__ __forceinline__ float sum(frag f, float c) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    const uint4 u = __builtin_bit_cast(uint4, f);
    c = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, u.x), ones, c, false);
    c = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, u.y), ones, c, false);
    c = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, u.z), ones, c, false);
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, u.w), ones, c, false);
  }
};

template <> struct Tr<DF_FP32_T> {
  using T = float;
  using frag = float;
  static constexpr int E = 1, KS = 2;
  static __device__ __forceinline__ float to_f(T x) { return x; }
  static __device__ __forceinline__ T from_f(float f) { return f; }
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag pack(const float* x) { return x[0]; }
  static __device__ __forceinline__ frag ld(const T* p) { return *p; }
  static __device__ __forceinline__ frag ld2x4(const T* p0, const T*) { return *p0; }
  static __device__ __forceinline__ frag zero() { return 0.f; }
  static __device__ __forceinline__ float add2(T a, T b, float c) { return (a + b) + c; }
  static __device__ __forceinline__ float sum(frag f, float c) { return c + f; }
};

// ---------------------------------------------------------------------------
// Accumulator layout of a 32x32 MFMA (C/D operand): lane l holds column
// n = l % 32 and, in register v (0..15), row acc_row(v, l / 32).
__device__ __forceinline__ constexpr int acc_row(int v, int g) { return 8 * (v >> 2) + 4 * g + (v & 3); }

// When a 32x32 accumulator tile is fed back as the B operand of a product
// that contracts over its rows, step q of that product takes registers
// v = q*E .. q*E + E - 1 from each lane. The other operand must then supply,
// for lane group g and slot s, contraction index acc_row(q*E + s, g). For
// 16-bit types these are two runs of four: [16q + 4g, +4) and [16q + 8 + 4g, +4).
template <int E>
__device__ __forceinline__ constexpr int fed_row(int q, int s, int g) { return acc_row(q * E + s, g); }

// An accumulator tile whose register v holds src[acc_row(v, g)]: a value per
// row of the tile (four 16-byte LDS reads), to start an MFMA chain from.
__device__ __forceinline__ f32x16 bias16(const float* src, int g) {
  f32x16 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 b = *reinterpret_cast<const float4*>(src + 8 * k + 4 * g);
    r[4 * k] = b.x;
    r[4 * k + 1] = b.y;
    r[4 * k + 2] = b.z;
    r[4 * k + 3] = b.w;
  }
  return r;
}

// An accumulator tile whose register v holds src[v] (four 16-byte LDS
// reads), for partners laid out half-major (register v of a lane group is
// partner base + v).
__device__ __forceinline__ f32x16 seq16(const float* src) {
  f32x16 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 b = *reinterpret_cast<const float4*>(src + 4 * k);
    r[4 * k] = b.x;
    r[4 * k + 1] = b.y;
    r[4 * k + 2] = b.z;
    r[4 * k + 3] = b.w;
  }
  return r;
}

// An accumulator tile with every register equal to x.
__device__ __forceinline__ f32x16 splat16(float x) {
  f32x16 r;
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = x;
  return r;
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Exchange with the lane 32 apart (lanes l and l ^ 32 hold the two halves of
// an accumulator column).
__device__ __forceinline__ float xor32(float x) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(int(((threadIdx.x & 63) ^ 32) << 2), __float_as_int(x)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer view of `bytes` bytes at `base`: loads at offsets past the end
// return zero (the hardware range check, which on gfx950 covers the per-lane
// offset, the scalar offset and their sum; checked with an in-bounds probe),
// so a gather may run past the end of a sequence without touching memory
// there.
struct BufView {
  __amdgpu_buffer_rsrc_t r;
};
__device__ __forceinline__ BufView buf_view(const void* base, uint32_t bytes) {
  // word 3 = 0x00020000: 32-bit raw data, no swizzle (gfx9 family)
  return {__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000)};
}
template <typename T>
__device__ __forceinline__ T buf_load(BufView b, int voff, int soff) {
  if constexpr (sizeof(T) == 2)
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b16(b.r, voff, soff, 0));
  else
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(b.r, voff, soff, 0));
}

__device__ __forceinline__ uint32_t buf_load_u8(BufView b, int voff) {
  return __builtin_amdgcn_raw_buffer_load_b8(b.r, voff, 0, 0);
}

// Range-checked stores: a store whose bytes lie past the view is dropped by
// the hardware. kBufSkip as the offset drops a store on purpose, so that a
// guarded store needs no branch (and the wait counts around it stay exact).
constexpr int kBufSkip = 0x7ff00000;
template <typename T>
__device__ __forceinline__ void buf_store(BufView b, int voff, T v) {
  if constexpr (sizeof(T) == 2)
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), b.r, voff, 0, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), b.r, voff, 0, 0);
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void buf_store16(BufView b, int voff, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, b.r, voff, 0, 0);
}
__device__ __forceinline__ uint4 buf_load16(BufView b, int voff, int soff = 0) {
  const u32x4 r = __builtin_amdgcn_raw_buffer_load_b128(b.r, voff, soff, 0);
  return make_uint4(r.x, r.y, r.z, r.w);
}

// ---------------------------------------------------------------------------
// Attention-probability dropout (DisentangledFlash 1.1.1 page, "Status":
// dropout is applied inside the fused kernels and the backward recomputes the
// mask from the Philox counter). Philox4x32 with 10 rounds, written from its definition
// (Salmon, Moraes, Dror and Shaw, SC 2011): a round maps counter
// (c0, c1, c2, c3) and key (k0, k1) to (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2),
// hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key grows by (W0, W1) before every
// round after the first. One call with counter (j / 8, i, n H + h, offset)
// and key (seed low, seed high) covers the keys 8m .. 8m+7 of query i of
// sequence n, head h: key j takes the low (j even) or high (j odd) 16 bits of
// word (j % 8) / 2, and the pair is kept iff those bits, as an unsigned
// number, are >= the threshold floor(p 2^16).
struct Philox4 {
  uint32_t w[4];
};
__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    // each 32 x 32 -> 64-bit product is one v_mad_u64_u32 (a separate
    // high and low multiply costs ~30% more per call), each three-way xor
    // one v_bitop3_b32 (truth table 0x96)
    const uint64_t x0 = uint64_t(M0) * c0, x1 = uint64_t(M1) * c2;
    const uint32_t hi0 = uint32_t(x0 >> 32), lo0 = uint32_t(x0);
    const uint32_t hi1 = uint32_t(x1 >> 32), lo1 = uint32_t(x1);
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32(hi1, c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32(hi0, c3, k1, 0x96);
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return {{c0, c1, c2, c3}};
}

// Keep tests of the two keys of one word: the low half compared as a 16-bit
// number (one SDWA compare), the high half by comparing the whole word with
// the threshold moved up 16 bits (the low half cannot change that order).
__device__ __forceinline__ bool keep_lo(uint32_t w, uint32_t thr) { return uint16_t(w) >= uint16_t(thr); }
__device__ __forceinline__ bool keep_hi(uint32_t w, uint32_t thr) { return w >= (thr << 16); }

// Exchange between lanes l and l ^ 4 inside each group of 8 lanes: lanes with
// bit 2 clear take `a` of lane l + 4 into `b`, lanes with bit 2 set take `b` of
// lane l - 4 into `a`. Two DPP row shifts, each writing only the banks (4-lane
// groups of a 16-lane row) it serves.
__device__ __forceinline__ void xor4_swap(uint32_t& a, uint32_t& b) {
  // row_shl:4 (lane l reads l + 4) into banks 0 and 2, row_shr:4 (l reads
  // l - 4) into banks 1 and 3
  const uint32_t nb = uint32_t(__builtin_amdgcn_update_dpp(int(b), int(a), 0x104, 0xF, 0x5, false));
  const uint32_t na = uint32_t(__builtin_amdgcn_update_dpp(int(a), int(b), 0x114, 0xF, 0xA, false));
  a = na;
  b = nb;
}

// 4 x 4 transpose inside each quad of lanes (lanes 4m .. 4m+3): on entry
// lane e of the quad holds row e of a matrix in (w0, w1, w2, w3), on exit it
// holds column e. Two exchange steps with the lane 2 apart, then the lane 1
// apart (quad-permute DPP moves); e = lane % 4.
__device__ __forceinline__ uint32_t quad_xor(uint32_t x, int ctrl_xor) {
  // quad_perm [2,3,0,1] (xor 2) = 0x4E, [1,0,3,2] (xor 1) = 0xB1
  return ctrl_xor == 2 ? uint32_t(__builtin_amdgcn_mov_dpp(int(x), 0x4E, 0xF, 0xF, false))
                       : uint32_t(__builtin_amdgcn_mov_dpp(int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ void quad_transpose(uint32_t& w0, uint32_t& w1, uint32_t& w2, uint32_t& w3, int e) {
  // step 1: exchange the off-diagonal 2 x 2 blocks between lanes e and e ^ 2
  {
    const bool hi = (e & 2) != 0;
    const uint32_t x = quad_xor(hi ? w0 : w2, 2), y = quad_xor(hi ? w1 : w3, 2);
    if (hi) {
      w0 = x;
      w1 = y;
    } else {
      w2 = x;
      w3 = y;
    }
  }
  // step 2: exchange the off-diagonal elements of each 2 x 2 block between
  // lanes e and e ^ 1
  {
    const bool odd = (e & 1) != 0;
    const uint32_t x = quad_xor(odd ? w0 : w1, 1), y = quad_xor(odd ? w2 : w3, 1);
    if (odd) {
      w0 = x;
      w2 = y;
    } else {
      w1 = x;
      w3 = y;
    }
  }
}

// Two gathered raw values (C2P term, P2C term) of a pair held until they are
// added: for 16-bit types one 32-bit register (the halves are loaded
// separately, so each load completes on its own), for fp32 two.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
template <typename T> struct RawPair {
  using type = u16x2;
  static __device__ __forceinline__ void set(type& r, T c, T p) {
    r.x = c;
    r.y = p;
  }
  template <typename TR>
  static __device__ __forceinline__ float add2(type r, float c) {
    return TR::add2(r.x, r.y, c);
  }
};
template <> struct RawPair<float> {
  struct type {
    float c, p;
  };
  static __device__ __forceinline__ void set(type& r, float c, float p) {
    r.c = c;
    r.p = p;
  }
  template <typename TR>
  static __device__ __forceinline__ float add2(type r, float c) {
    return (r.c + r.p) + c;
  }
};

// An empty asm statement that reads x: the value is then computed before
// this point (it cannot sink past it into a later block).
template <typename F>
__device__ __forceinline__ void keep_here(const F& x) {
  if constexpr (sizeof(F) == 16) {
    const uint4 u = __builtin_bit_cast(uint4, x);
    asm volatile("" ::"v"(u.x), "v"(u.y), "v"(u.z), "v"(u.w));
  } else {
    static_assert(sizeof(F) == 4, "one or four registers");
    asm volatile("" ::"v"(x));
  }
}

// Compile-time flag passed to a generic lambda, so that a loop body can be
// instantiated once per tile class (band / far) as straight-line code.
template <bool B> struct BoolC {
  static constexpr bool value = B;
};
// Compile-time integer for the same purpose (e.g. the parity of a
// double-buffered tile, so that each buffer is a distinct LDS object).
template <int V> struct IntC {
  static constexpr int value = V;
};

// Work-group placement over the 8 XCDs of the chip, each with its own L2.
// The dispatcher hands consecutive work-group ids to the XCDs in turn;
// attn_block() renumbers a 1-D grid of nx * H * nseq groups so that every XCD
// runs one contiguous range of logical blocks, row block fastest, then
// sequence, then head. The row blocks of one (sequence, head) run together on
// one XCD and share that head's streamed operands in its L2, and every head's
// work is the same sum over the sequences, so the XCDs get equal shares even
// when the sequences of a packed batch differ in length (ordered head before
// sequence, the busiest XCD of an 18-sequence packed batch had 2.3 times the
// mean work).
constexpr int kXcds = 8;
struct AttnBlock {
  int x, h, z;
};
__device__ __forceinline__ AttnBlock attn_block(int nx, int H) {
  const int nb = gridDim.x, id = blockIdx.x;
  const int q = nb / kXcds, r = nb % kXcds, xcd = id % kXcds, slot = id / kXcds;
  const int logical = xcd * q + (xcd < r ? xcd : r) + slot;
  const int nz = nb / (nx * H);  // sequences
  return {logical % nx, logical / (nx * nz), (logical / nx) % nz};
}

// Sequence bounds of blockIdx.z: padded (cu == nullptr) or packed.
struct SeqRange {
  int64_t start;
  int len;
};
__device__ __forceinline__ SeqRange seq_range(const int32_t* cu, int z, int Lmax) {
  if (cu) {
    int a = cu[z], b = cu[z + 1];
    return {int64_t(a), b - a};
  }
  return {int64_t(z) * Lmax, Lmax};
}

}  // namespace dfa
