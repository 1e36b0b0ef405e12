// Internal parameter block and launcher declarations (host and device).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace dfa {

constexpr int DF_BF16_T = 0, DF_FP16_T = 1, DF_FP32_T = 2;

// Entries on each side of the padded packed index table (at least the
// largest tile edge, so a tile's table slice never needs a clamp).
constexpr int kLutPad = 256;

// Everything a kernel of the path may need. Pointers are device pointers.
struct Params {
  // shape
  int nseq, Lmax, H, D, R, att, span, buckets, dtype;
  int RP;                   // row pitch of every [H][T][.] strip: R rounded up to 8
  int64_t T;
  int64_t ts, hs;           // token / head element strides of [T,H,D] tensors
  const int32_t* cu;        // [nseq+1] or nullptr (padded)
  const uint8_t* kmask;     // [T] or nullptr
  float scale;              // s = 1/sqrt(3D)
  float scale_log2;         // s * log2(e)
  // relative index tables, entry d + Lmax - 1
  int32_t* c2p;
  int32_t* p2c;
  // the same tables packed (c2p | p2c << 16), entry d + Lmax - 1 + kLutPad, with
  // kLutPad copies of the end entries on each side: [2 Lmax - 1 + 2 kLutPad]
  const uint32_t* lutp;
  int d_hi, d_lo;           // far field: both tables at their end rows iff d >= d_hi or d <= d_lo
  int narrow;               // 1 if neither table ever steps by more than one row
  // 1: the shared P2C convention (P2C uses the row C2P uses). The kernels
  // then see q_r with its rows reversed (qr points at that copy) and a P2C
  // table in reversed coordinates, clamp(att - 1 - bucket(d)), which is
  // non-increasing in d like the literal one; dq_r is written back reversed.
  int p2c_shared;
  // user tensors
  const void *q, *k, *v, *qr, *kr;
  void* out;
  float* lse;
  const void* dout;
  void *dq, *dk, *dv, *dqr, *dkr;
  // workspace
  void* c2ps;               // [H][T][RP] dtype: s*log2(e) * Q . K_r^T
  void* p2cs;               // [H][T][RP] dtype: s*log2(e) * K . Q_r^T
  void* ends;               // [4][H][T] dtype: c2ps[..][0], c2ps[..][R-1],
                            //   p2cs[..][0], p2cs[..][R-1]
  float* delta;             // [H][T]: rowsum(dO * O)
  const void* krT;          // [H][RP/CE][D][CE] dtype: k_r transposed in 16-byte chunks (CE elements; columns >= R zero)
  const void* qrT;          // [H][RP/CE][D][CE] dtype: the q_r the kernels read, transposed the same way
  void* dc2p;               // [H][T][RP] dtype: segmented sums of dS over delta(i,j)
  void* dp2c;               // [H][T][RP] dtype: segmented sums of dS over delta(j,i)
  float* part;              // [2][H][nchunk][R][D] split-K partials
  // attention-probability dropout (drop = 0: none)
  int drop;
  uint32_t drop_thr;        // floor(p 2^16): a pair is kept iff its 16 Philox bits >= drop_thr
  float drop_scale;         // 1 / (1 - p)
  uint32_t seed_lo, seed_hi, drop_off;
  int nchunk;
  int chunk_tokens;
};

// One projection GEMM Y = A W^T + bias (16-bit operands, fp32 accumulation):
// A [M, K] (row stride lda), W rows [N, K] (row stride ldw), both
// K-contiguous, bias [N] or null. mode 0: column n = which * HD + hd goes to
// out<which>[m * HD + hd] ([T, H, D]; HD = N gives a plain [M, N]); mode 1:
// to out<which>[(hd / D) * R + m) * D + hd % D] ([H, R, D]); mode 2: split-K
// partials, fp32 out0[(chunk * M + m) * N + n] for the contraction range
// [chunk * kchunk, (chunk + 1) * kchunk) of chunk = blockIdx.y (kchunk = 0:
// all of K in one chunk).
struct ProjParams {
  const void* a;
  const void* w;
  const void* bias;
  int M, N, K;
  int lda, ldw;
  int kchunk;
  int HD, D, R;
  int mode;
  int dtype;
  void *out0, *out1, *out2;
};

// launchers (each returns hipGetLastError() after its launches)
hipError_t launch_lut(int Lmax, int span, int buckets, int p2c_shared, int32_t* c2p, int32_t* p2c, uint32_t* packed,
                      hipStream_t st);  // packed may be null
hipError_t launch_reverse_rows(const void* src, void* dst, int H, int R, int D, int elem_bytes, hipStream_t st);
hipError_t launch_transpose_rows(const void* src, void* dst, int H, int R, int RP, int D, int elem_bytes,
                                 hipStream_t st);  // [H][R][D] -> [H][D][RP], zero columns >= R
hipError_t launch_strips(const Params& p, hipStream_t st);  // both strips
hipError_t launch_fwd(const Params& p, hipStream_t st);
hipError_t launch_bwd_pre(const Params& p, hipStream_t st);
hipError_t launch_bwd_dkv(const Params& p, hipStream_t st);
hipError_t launch_bwd_dq(const Params& p, hipStream_t st);
hipError_t launch_relgrad_dw(const Params& p, hipStream_t st);
hipError_t launch_relgrad_sum(const Params& p, hipStream_t st);
hipError_t launch_proj(const ProjParams& p, hipStream_t st);  // gridDim.y = number of K chunks
// dst[b][c][r] = src[b][r][c] for a batch of [rows, cols] 16-bit matrices
// (row strides src_ld / dst_ld, batch strides src_bs / dst_bs); columns r in
// [rows, dst_ld) of dst are written as zero
hipError_t launch_transpose16(const void* src, int64_t src_ld, int64_t src_bs, void* dst, int64_t dst_ld,
                              int64_t dst_bs, int rows, int cols, int batch, hipStream_t st);
// fill n 16-bit elements with `bits`
hipError_t launch_fill16(void* dst, int64_t n, uint16_t bits, hipStream_t st);
// rows [R, 2 H D] of the relative-row gradients: row r, column
// which * H D + h D + d = (which ? dk_r : dq_r)[h][r][d]
hipError_t launch_rel_rows(const void* dq_r, const void* dk_r, void* dst, int H, int R, int D, hipStream_t st);
// out[n][e] (dtype) = sum_{c < nch} part[c][n][e] + (n < nrel ? part[nch][n][e] : 0)
// for e < E, and db[n] (dtype) likewise from column E (when db != null)
hipError_t launch_proj_reduce(const float* part, int nch, int nrel, int M, int E, int dtype, void* out, void* db,
                              hipStream_t st);
hipError_t launch_pack(int B, int L, int64_t row_bytes, const void* padded, const uint8_t* mask, void* packed,
                       int32_t* cu, int32_t* max_len, hipStream_t st);
hipError_t launch_unpack(int B, int L, int64_t row_bytes, const void* packed, const uint8_t* mask,
                         const int32_t* cu, void* padded, hipStream_t st);

}  // namespace dfa
