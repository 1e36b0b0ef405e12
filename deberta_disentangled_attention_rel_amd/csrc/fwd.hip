// Fused forward: output and log-sum-exp of disentangled attention without
// the L x L matrix (DisentangledFlash 1.1.1 page, "Status" and "Hugging Face
// usage": the LSE-producing training forward).
//
// Work item: one sequence, one head, 128 query rows (4 waves x 32). The key
// loop walks BN = 32*NKT keys at a time. The next key tile (K rows, V rows,
// per-key P2C far-field values with the key mask folded in, and the
// index-table slice) is loaded into registers while the current one is
// computed, then written to the other half of a double-buffered LDS area:
// one barrier per tile. Both tiles stay row-major; the V^T operand is read
// with transposing LDS reads.
//
// Each wave computes S^T = K Q^T with 32x32 MFMAs, so lane l owns query row
// l % 32 and holds 16 of every 32 keys (the other 16 sit in lane l ^ 32).
// Row max and row sum are lane-local plus one exchange; the output is
// accumulated transposed, O^T = V^T P^T, so the rescale is lane-local and P
// feeds the MFMA straight from the score registers.
//
// Scores are in the log2 domain: y = s*log2(e)*QK + (relative terms). In a
// far-field tile the per-key P2C value is added in the same FMA and the
// per-query C2P value a is folded into the row max (exp2(y - (m - a))). A
// band tile stages the strip windows it needs in LDS and gathers both terms
// per pair from there (or from global memory when the tables can skip rows).
#include "band.hpp"
#include "pipe.hpp"

namespace dfa {

namespace {

template <int DT, int D, int NKT, bool NARROW>
__global__ __launch_bounds__(256, (D <= 64 && DT != DF_FP32_T) ? 2 : 1) void fwd_kernel(Params p) {
  using TR = Tr<DT>;
  using T = typename TR::T;
  using frag = typename TR::frag;
  constexpr int E = TR::E, KS = TR::KS, NQ = D / KS, ND = D / 32;
  constexpr int BM = 128, BN = 32 * NKT, NL = BM + BN - 1;
  constexpr int KP = RowPitch<T, D>::rows, VP = RowPitch<T, D>::cols;
  constexpr int WC = BN + 8, WCP = WinPitch<T, WC>::v;
  constexpr int WPW = BM + 8, WPP = WinPitch<T, WPW>::v;
  static_assert(NL <= 256, "one table entry per thread");
  using KTile = RowTile<T, BN, D, 256>;

  __shared__ __align__(16) T Ks[2][BN * KP];
  __shared__ __align__(16) T Vs[2][BN * VP];
  __shared__ __align__(16) float bj_s[2][BN];
  __shared__ uint32_t lut_s[2][NL];
  __shared__ __align__(16) T Wc[NARROW ? BM * WCP : 1];
  __shared__ __align__(16) T Wp[NARROW ? BN * WPP : 1];
  __shared__ int ps_s[NARROW ? BN : 1];

  const int lane = threadIdx.x & 63, g = lane >> 5, li = lane & 31, wave = threadIdx.x >> 6;
  const int tid = threadIdx.x;
  const SeqRange sq = seq_range(p.cu, blockIdx.z, p.Lmax);
  const int h = blockIdx.y;
  const int i0 = blockIdx.x * BM;
  if (i0 >= sq.len) return;
  const int64_t T_ = p.T, HT = int64_t(p.H) * p.T;
  const int RP = p.RP;
  const int d_hi = p.d_hi, d_lo = p.d_lo;

  const int il = wave * 32 + li;
  const int iw = i0 + il;  // this lane's query (local index)
  const bool qin = iw < sq.len;
  const int64_t tok_i = sq.start + (qin ? iw : sq.len - 1);
  const bool qvalid = qin && (!p.kmask || p.kmask[tok_i]);

  frag Qf[NQ];
  {
    const T* qp = (const T*)p.q + tok_i * p.ts + int64_t(h) * p.hs;
#pragma unroll
    for (int q = 0; q < NQ; ++q) Qf[q] = TR::ld(qp + q * KS + g * E);
  }
  const T* ends = (const T*)p.ends + int64_t(h) * T_;
  const float a_end0 = TR::to_f(ends[tok_i]);
  const float a_end1 = TR::to_f(ends[HT + tok_i]);
  const T* c2pstrip = (const T*)p.c2ps + (int64_t(h) * T_ + sq.start) * RP;
  const T* p2cstrip = (const T*)p.p2cs + (int64_t(h) * T_ + sq.start) * RP;
  const T* kbase = (const T*)p.k + sq.start * p.ts + int64_t(h) * p.hs;
  const T* vbase = (const T*)p.v + sq.start * p.ts + int64_t(h) * p.hs;
  const uint8_t* kmask = p.kmask ? p.kmask + sq.start : nullptr;

  auto cls_of = [&](int kb) {
    const int j0 = kb * BN;
    return tile_class(i0 - j0 - BN + 1, i0 + BM - 1 - j0, d_hi, d_lo);
  };

  // ---- next-tile registers
  KTile kt, vt;
  kt.init();
  vt.init();
  float breg = 0.f;
  uint32_t lreg = 0;

  auto prefetch = [&](int kb) {
    const int j0 = kb * BN;
    const int cls = cls_of(kb);
    kt.load(kbase, p.ts, j0, sq.len);
    vt.load(vbase, p.ts, j0, sq.len);
    if (tid < BN) {
      const int j = j0 + tid;
      const bool in = j < sq.len;
      const int jc = in ? j : sq.len - 1;
      const bool ok = in && (!kmask || kmask[jc]);
      float b = 0.f;
      if (cls != TILE_BAND) b = TR::to_f(ends[p2c_end_of(cls) * HT + sq.start + jc]);
      breg = ok ? b : -INFINITY;
    }
    if (cls == TILE_BAND && tid < NL) lreg = lut_entry(p, i0 - j0 - BN + 1 + tid);
  };

  auto commit = [&](int buf) {
    kt.template store<KP>(Ks[buf]);
    vt.template store<VP>(Vs[buf]);
    if (tid < BN) bj_s[buf][tid] = breg;
    if (tid < NL) lut_s[buf][tid] = lreg;
  };

  f32x16 O[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) O[nd] = zero16();
  float m = -INFINITY, l = 0.f;

  const int nkb = (sq.len + BN - 1) / BN;
  prefetch(0);
  commit(0);
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    const int j0 = kb * BN;
    const int cls = cls_of(kb);
    if (kb + 1 < nkb) prefetch(kb + 1);

    if constexpr (NARROW) {
      if (cls == TILE_BAND) {
        stage_window<T, WC, WCP, 256>(Wc, c2pstrip, RP, BM, i0, sq.len,
                                      [&](int r) { return lut_c(lut_s[buf][r]) & ~7; });
        stage_window<T, WPW, WPP, 256>(Wp, p2cstrip, RP, BN, j0, sq.len,
                                       [&](int r) { return lut_p(lut_s[buf][NL - 1 - r]) & ~7; });
        if (tid < BN) ps_s[tid] = lut_p(lut_s[buf][NL - 1 - tid]) & ~7;
        __syncthreads();
      }
    }

    float a = 0.f;
    if (cls == TILE_FAR_LEFT) a = a_end1;
    if (cls == TILE_FAR_RIGHT) a = a_end0;
    const int cs = NARROW ? (lut_c(lut_s[buf][il]) & ~7) : 0;

    float y[NKT][16];
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      f32x16 acc = zero16();
#pragma unroll
      for (int q = 0; q < NQ; ++q) acc = TR::mma(ld_row<TR>(Ks[buf], KP, 32 * t + li, q * KS + g * E), Qf[q], acc);
      if (cls != TILE_BAND) {
#pragma unroll
        for (int v = 0; v < 16; ++v) y[t][v] = fmaf(acc[v], p.scale_log2, bj_s[buf][32 * t + acc_row(v, g)]);
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int jl = 32 * t + acc_row(v, g);
          const uint32_t e = lut_s[buf][il - jl + BN - 1];
          float rel;
          if constexpr (NARROW) {
            rel = TR::to_f(Wc[il * WCP + lut_c(e) - cs]) + TR::to_f(Wp[jl * WPP + lut_p(e) - ps_s[jl]]);
          } else {
            const int jj = min(j0 + jl, sq.len - 1);
            rel = TR::to_f(c2pstrip[int64_t(qin ? iw : sq.len - 1) * RP + lut_c(e)]) +
                  TR::to_f(p2cstrip[int64_t(jj) * RP + lut_p(e)]);
          }
          y[t][v] = fmaf(acc[v], p.scale_log2, rel + bj_s[buf][jl]);
        }
      }
    }
    // online softmax (log2 domain); a is this tile's per-row C2P value
    float mt = -INFINITY;
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) mt = fmaxf(mt, y[t][v]);
    mt = fmaxf(mt, xor32(mt)) + a;
    const float mnew = fmaxf(m, mt);
    const float msafe = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = fast_exp2(m - msafe);
    const float shift = msafe - a;
    float ls = 0.f;
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        y[t][v] = fast_exp2(y[t][v] - shift);
        ls += y[t][v];
      }
    l = l * alpha + ls;
    m = mnew;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int nd = 0; nd < ND; ++nd)
#pragma unroll
        for (int v = 0; v < 16; ++v) O[nd][v] *= alpha;
    }
    // O^T += V^T P^T
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int q = 0; q < 32 / KS; ++q) {
        const frag pb = TR::pack(&y[t][q * E]);
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) O[nd] = TR::mma(ld_col<TR>(Vs[buf], VP, 32 * t, 32 * nd, q), pb, O[nd]);
      }
    if (kb + 1 < nkb) commit(buf ^ 1);
    __syncthreads();
  }

  const float lt = l + xor32(l);
  if (!qin) return;
  const bool ok = qvalid && lt > 0.f;
  const float inv = ok ? 1.f / lt : 0.f;
  T* op = (T*)p.out + tok_i * p.ts + int64_t(h) * p.hs;
#pragma unroll
  for (int nd = 0; nd < ND; ++nd)
#pragma unroll
    for (int v = 0; v < 16; ++v) op[32 * nd + acc_row(v, g)] = TR::from_f(O[nd][v] * inv);
  if (g == 0) p.lse[int64_t(h) * T_ + tok_i] = ok ? (m + log2f(lt)) * kLn2 : -INFINITY;
}

template <int DT, int D, bool NARROW>
void launch_fwd_d(const Params& p, hipStream_t st) {
  dim3 grid(unsigned((p.Lmax + 127) / 128), unsigned(p.H), unsigned(p.nseq));
  constexpr int NKT = (DT == DF_FP32_T && D == 128) ? 1 : 2;
  fwd_kernel<DT, D, NKT, NARROW><<<grid, 256, 0, st>>>(p);
}

template <int DT, int D>
void launch_fwd_n(const Params& p, hipStream_t st) {
  if (p.narrow)
    launch_fwd_d<DT, D, true>(p, st);
  else
    launch_fwd_d<DT, D, false>(p, st);
}

template <int DT>
void launch_fwd_dt(const Params& p, hipStream_t st) {
  switch (p.D) {
    case 32: launch_fwd_n<DT, 32>(p, st); break;
    case 64: launch_fwd_n<DT, 64>(p, st); break;
    default: launch_fwd_n<DT, 128>(p, st); break;
  }
}

}  // namespace

hipError_t launch_fwd(const Params& p, hipStream_t st) {
  switch (p.dtype) {
    case DF_BF16_T: launch_fwd_dt<DF_BF16_T>(p, st); break;
    case DF_FP16_T: launch_fwd_dt<DF_FP16_T>(p, st); break;
    default: launch_fwd_dt<DF_FP32_T>(p, st); break;
  }
  return hipGetLastError();
}

}  // namespace dfa
