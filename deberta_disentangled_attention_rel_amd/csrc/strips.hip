// Relative-position strips: the L x R score products that the C2P and P2C
// terms gather from (DisentangledFlash 1.1.1 page, "Performance": the C2P and
// P2C relative-position score products, 4LRD FLOPs of the forward count).
//
//   c2ps[h][t][r] = s*log2(e) * Q[t,h,:] . K_r[h,r,:]
//   p2cs[h][t][r] = s*log2(e) * K[t,h,:] . Q_r[h,r,:]
//
// stored in the working dtype, pre-scaled into the log2 domain the attention
// kernels use, rows padded to RP (columns R..RP-1 are zero). Columns 0 and
// R-1 (the rows every far-field pair saturates to) are also written
// contiguously per head into `ends` [4][H][T].
//
// The kernel is bound by its HBM writes (2*H*T*RP elements). Each wave owns
// 32*MT tokens and sweeps all R rows in 64-row chunks, computing the
// transposed product C^T = K_r Q^T with 32x32 MFMAs (lane l holds token
// l % 32 of each token tile and, per register group, 4 consecutive rows).
// The token operand stays in registers for the whole sweep and every K_r /
// Q_r fragment (read from L2) feeds MT MFMAs. Each 32-token x 64-row block is
// staged in a wave-private LDS buffer and written back as whole 128-byte row
// segments (8 rows per store instruction), so no cache line of the strip is
// written in pieces.
#include "common.hpp"

namespace dfa {

namespace {

template <int DT, int D>
__global__ __launch_bounds__(256) void strip_kernel(Params p) {
  using TR = Tr<DT>;
  using T = typename TR::T;
  using frag = typename TR::frag;
  constexpr int E = TR::E, KS = TR::KS, NQ = D / KS, ES = int(sizeof(T));
  constexpr int MT = 4;        // 32-token tiles per wave (4: measured best)
  constexpr int WT = 32 * MT;  // tokens per wave
  constexpr int RC = 64;       // rows per chunk
  constexpr int NRT = RC / 32;  // 32-row tiles per chunk
  constexpr int CH = 16 / int(sizeof(T));
  constexpr int SP = RC + CH;  // staging pitch (elements): rows stay 16-byte aligned
  __shared__ __align__(16) T stage_s[4][32 * SP];

  const int lane = threadIdx.x & 63, g = lane >> 5, li = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: buffer views need it
  const int which = blockIdx.y / p.H, h = blockIdx.y % p.H;
  const int64_t tw = (int64_t(blockIdx.x) * 4 + wave) * WT;  // first token of this wave
  if (tw >= p.T) return;
  const T* A = (const T*)(which ? p.k : p.q);    // token operand [T,H,D]
  const T* B = (const T*)(which ? p.qr : p.kr);  // relative rows [H,R,D]
  T* out = (T*)(which ? p.p2cs : p.c2ps) + int64_t(h) * p.T * p.RP;
  T* ends = (T*)p.ends + (which ? 2 : 0) * int64_t(p.H) * p.T + int64_t(h) * p.T;
  T* st = stage_s[wave];

  // token fragments, resident for the whole sweep (rows past T read row T-1)
  frag a[MT][NQ];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int64_t t = min(tw + 32 * m + li, p.T - 1);
    const T* row = A + t * p.ts + int64_t(h) * p.hs;
#pragma unroll
    for (int q = 0; q < NQ; ++q) a[m][q] = TR::ld(row + q * KS + g * E);
  }
  const int rlast = p.R - 1;
  // Every access of the sweep goes through a range-checked view: relative
  // rows past R read zero, stores to tokens past T (or columns past RP) are
  // dropped. The next chunk's fragments are loaded before this chunk's
  // stores (vector memory operations complete in issue order). The waits
  // before a chunk's MFMAs still cover about half of the previous chunk's
  // stores (the compiler takes the tighter count of the loop's entry and
  // back edge). Exact counts that left all stores in flight measured slower
  // (0.100 -> 0.110 ms at L=8192 H=12 D=64 bf16): this write-bound sweep
  // does better with each wave's store stream paced by its own chunks.
  const int nt = int(min<int64_t>(WT, p.T - tw));  // tokens of this wave
  const BufView bv = buf_view(B + int64_t(h) * p.R * D, uint32_t(p.R) * D * ES);
  const BufView ov = buf_view(out + tw * p.RP, uint32_t(nt) * uint32_t(p.RP) * ES);
  const BufView e0 = buf_view(ends + tw, uint32_t(nt) * ES);
  const BufView e1 = buf_view(ends + int64_t(p.H) * p.T + tw, uint32_t(nt) * ES);

  frag bf[NRT][NQ];
  auto load_b = [&](int r0) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int r = r0 + 32 * rt + li;  // relative row fed by this lane
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if constexpr (sizeof(T) == 2)
          bf[rt][q] = __builtin_bit_cast(frag, buf_load16(bv, (r * D + q * KS + g * E) * ES));
        else
          bf[rt][q] = buf_load<T>(bv, (r * D + q * KS + g * E) * ES, 0);
      }
    }
  };
  load_b(0);
  for (int r0 = 0; r0 < p.RP; r0 += RC) {
    f32x16 acc[MT][NRT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) acc[m][rt] = zero16();
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m][rt] = TR::mma(bf[rt][q], a[m][q], acc[m][rt]);
    if (r0 + RC < p.RP) load_b(r0 + RC);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      // C^T[r][t]: lane holds token 32m + li, rows r0 + 32rt + 8grp + 4g + 0..3
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          T* d = st + li * SP + 32 * rt + 8 * grp + 4 * g;
          const float x0 = acc[m][rt][4 * grp] * p.scale_log2, x1 = acc[m][rt][4 * grp + 1] * p.scale_log2;
          const float x2 = acc[m][rt][4 * grp + 2] * p.scale_log2, x3 = acc[m][rt][4 * grp + 3] * p.scale_log2;
          if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<uint2*>(d) =
                make_uint2(uint32_t(TR::from_f(x0)) | (uint32_t(TR::from_f(x1)) << 16),
                           uint32_t(TR::from_f(x2)) | (uint32_t(TR::from_f(x3)) << 16));
          } else {
            *reinterpret_cast<float4*>(d) = make_float4(x0, x1, x2, x3);
          }
        }
      // the end columns, as stored in the strip
      const int tl = 32 * m + li;
      buf_store<T>(e0, r0 == 0 && g == 0 ? tl * ES : kBufSkip, TR::from_f(acc[m][0][0] * p.scale_log2));
      float x = 0.f;
      bool hit = false;
      if (rlast >= r0 && rlast < r0 + RC) {
        const int k = rlast - r0, rt = k >> 5, kk = k & 31;
        hit = g == ((kk >> 2) & 1);
        const int vr = 4 * (kk >> 3) + (kk & 3);
#pragma unroll
        for (int t = 0; t < NRT; ++t)
#pragma unroll
          for (int v = 0; v < 16; ++v) x = (t == rt && v == vr) ? acc[m][t][v] : x;
      }
      buf_store<T>(e1, hit ? tl * ES : kBufSkip, TR::from_f(x * p.scale_log2));
      // wave-private buffer: a wave's LDS operations complete in order
      // 32 rows x RC columns, RC/CH lanes per row, 64/(RC/CH) rows per instruction
      constexpr int LPR = RC / CH, RPI = 64 / LPR;
#pragma unroll
      for (int k = 0; k < 32 / RPI; ++k) {
        const int row = k * RPI + lane / LPR, c = (lane % LPR) * CH;
        const uint4 val = *reinterpret_cast<const uint4*>(st + row * SP + c);
        buf_store16(ov, r0 + c < p.RP ? ((32 * m + row) * p.RP + r0 + c) * ES : kBufSkip, val);
      }
    }
  }
}

template <int DT>
void launch_strips_dt(const Params& p, hipStream_t st) {
  const int wt = 128;  // tokens per wave (32 * MT)
  dim3 grid(unsigned((p.T + 4 * wt - 1) / (4 * wt)), unsigned(2 * p.H));
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
