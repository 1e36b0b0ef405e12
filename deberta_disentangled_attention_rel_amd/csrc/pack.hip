// Packing helpers for the packed layout (DisentangledFlash 1.1.1 page,
// "Packed unpadded inference and training": right-padded [B, L, ...] input
// converted to FlashAttention-style [total_tokens, ...] rows with cu_seqlens,
// and the packed output converted back).
//
// Sequence b's length is the number of valid tokens of mask row b; its valid
// tokens, in order, become packed rows cu_seqlens[b] .. cu_seqlens[b+1]-1.
// Three launches pack: per-row counts, one scan of the counts (cu_seqlens and
// the largest length), then one work-group per sequence that numbers its
// valid tokens 256 positions at a time (ballot + popcount inside each wave,
// wave totals through LDS) and copies the rows with all its threads in
// 16-byte chunks, consecutive threads on consecutive chunks of a row.
// Unpacking runs the same numbering and writes zeros at invalid positions.
#include "common.hpp"

namespace dfa {

namespace {

constexpr int PK_NT = 256;

__global__ __launch_bounds__(PK_NT) void count_kernel(const uint8_t* __restrict__ mask, int L,
                                                      int32_t* __restrict__ cu) {
  const int b = blockIdx.x;
  const uint8_t* m = mask + int64_t(b) * L;
  int c = 0;
  for (int l = threadIdx.x; l < L; l += PK_NT) c += m[l] != 0;
  __shared__ int part[PK_NT / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
#pragma unroll
    for (int w = 0; w < PK_NT / 64; ++w) t += part[w];
    cu[b + 1] = t;  // the count, turned into an offset by scan_kernel
  }
}

// cu[1..B] holds the counts: in place, cu[b+1] = cu[b] + count_b, cu[0] = 0.
__global__ void scan_kernel(int32_t* __restrict__ cu, int B, int32_t* __restrict__ max_len) {
  if (threadIdx.x != 0) return;
  int run = 0, mx = 0;
  cu[0] = 0;
  for (int b = 0; b < B; ++b) {
    const int c = cu[b + 1];
    mx = c > mx ? c : mx;
    run += c;
    cu[b + 1] = run;
  }
  if (max_len) *max_len = mx;
}

// Number the valid tokens of positions [l0, l0 + 256) of row b: returns, for
// this thread's position, its rank among the row's valid tokens (or -1), and
// adds the chunk's count to `base`.
__device__ __forceinline__ int rank_in_row(const uint8_t* __restrict__ m, int l0, int L, int& base, int* wsum) {
  const int l = l0 + int(threadIdx.x);
  const bool valid = l < L && m[l] != 0;
  const uint64_t bal = __ballot(valid);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pre = __popcll(bal & ((uint64_t(1) << lane) - 1));
  if (lane == 0) wsum[wave] = __popcll(bal);
  __syncthreads();
  int off = base;
  int total = 0;
#pragma unroll
  for (int w = 0; w < PK_NT / 64; ++w) {
    off += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
  __syncthreads();  // wsum is reused by the next chunk
  base += total;
  return valid ? off + pre : -1;
}

// mode 0: pack (padded row -> packed row); mode 1: unpack (packed row ->
// padded row, zeros at invalid positions).
template <int MODE>
__global__ __launch_bounds__(PK_NT) void move_kernel(const uint8_t* __restrict__ mask, int L, int64_t row_bytes,
                                                     const int32_t* __restrict__ cu, const char* __restrict__ src,
                                                     char* __restrict__ dst) {
  const int b = blockIdx.x;
  const uint8_t* m = mask + int64_t(b) * L;
  const int64_t start = cu[b];
  __shared__ int rank_s[PK_NT];
  __shared__ int wsum[PK_NT / 64];
  const int64_t nc = row_bytes / 16;  // 16-byte chunks per row
  int base = 0;
  for (int l0 = 0; l0 < L; l0 += PK_NT) {
    rank_s[threadIdx.x] = rank_in_row(m, l0, L, base, wsum);
    __syncthreads();
    const int nrow = min(PK_NT, L - l0);
    for (int64_t it = threadIdx.x; it < int64_t(nrow) * nc; it += PK_NT) {
      const int r = int(it / nc);
      const int64_t c = it - int64_t(r) * nc;
      const int rk = rank_s[r];
      const int64_t pad_row = int64_t(b) * L + l0 + r;
      if (MODE == 0) {
        if (rk >= 0)
          reinterpret_cast<uint4*>(dst + (start + rk) * row_bytes)[c] =
              reinterpret_cast<const uint4*>(src + pad_row * row_bytes)[c];
      } else {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (rk >= 0) v = reinterpret_cast<const uint4*>(src + (start + rk) * row_bytes)[c];
        reinterpret_cast<uint4*>(dst + pad_row * row_bytes)[c] = v;
      }
    }
    __syncthreads();  // rank_s is rewritten by the next chunk
  }
}

}  // namespace

hipError_t launch_pack(int B, int L, int64_t row_bytes, const void* padded, const uint8_t* mask, void* packed,
                       int32_t* cu, int32_t* max_len, hipStream_t st) {
  count_kernel<<<B, PK_NT, 0, st>>>(mask, L, cu);
  scan_kernel<<<1, 64, 0, st>>>(cu, B, max_len);
  move_kernel<0><<<B, PK_NT, 0, st>>>(mask, L, row_bytes, cu, (const char*)padded, (char*)packed);
  return hipGetLastError();
}

hipError_t launch_unpack(int B, int L, int64_t row_bytes, const void* packed, const uint8_t* mask,
                         const int32_t* cu, void* padded, hipStream_t st) {
  move_kernel<1><<<B, PK_NT, 0, st>>>(mask, L, row_bytes, cu, (const char*)packed, (char*)padded);
  return hipGetLastError();
}

}  // namespace dfa
