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
// band tile stages each query's C2P strip window in LDS (the lanes gather
// from different rows) and reads the P2C terms straight from the strip,
// which stays in L2 (for a fixed key the 32 lanes of a half read one
// contiguous run of its row). Both gathers are issued ahead of the score
// MFMAs and joined with one packed dot product. When the tables can skip
// rows, both terms come from global memory.
//
// The tile body is compiled once per tile class (band / far), so each class
// runs as straight-line code that the scheduler can interleave.
#include "band.hpp"
#include "pipe.hpp"

namespace dfa {

namespace {

constexpr float kMaxSlack = 8.f;

template <int DT, int D, int NKT, bool NARROW, bool DROP>
__global__ __launch_bounds__(256, (D <= 64 && DT != DF_FP32_T) ? 2 : 1) void fwd_kernel(Params p) {
  using TR = Tr<DT>;
  using T = typename TR::T;
  using frag = typename TR::frag;
  constexpr int E = TR::E, KS = TR::KS, NQ = D / KS, ND = D / 32, ES = int(sizeof(T));
  constexpr bool DMA = ES == 2;  // 16-bit tiles go global -> LDS without registers
  constexpr int BM = 128, BN = 32 * NKT, NL = BM + BN - 1;
  constexpr int KP = RowPitch<T, D>::rows, VP = RowPitch<T, D>::cols;
  constexpr int WC = BN + 8, WCP = WinPitch<T, WC>::v;
  static_assert(NL <= 256, "one table entry per thread");
  using KTile = RowTile<T, BN, D, 256>;

  // the two buffers of each tile are distinct LDS objects and every access
  // names its buffer at compile time (the loop is unrolled by two): reads of
  // the current buffer then provably do not alias the copy into the other
  // one, so the compiler does not make them wait for that copy
  __shared__ __align__(16) T Ks0[BN * KP];
  __shared__ __align__(16) T Ks1[BN * KP];
  __shared__ __align__(16) T Vs0[BN * VP];
  __shared__ __align__(16) T Vs1[BN * VP];
  __shared__ __align__(16) float bj_s[2][BN];
  __shared__ uint32_t lut_s[2][NL];
  // C2P windows of band tiles: two LDS-DMA buffers filled one tile ahead
  // (16-bit), or one buffer staged when the tile starts (fp32)
  using Win = C2PWindowDma<uint16_t, BM, 256>;
  constexpr bool AWIN = NARROW && DMA;
  __shared__ __align__(16) T Wc0[AWIN ? Win::ELEMS : (NARROW ? BM * WCP : 1)];
  __shared__ __align__(16) T Wc1[AWIN ? Win::ELEMS : 1];

  const int lane = threadIdx.x & 63, g = lane >> 5, li = lane & 31, wave = threadIdx.x >> 6;
  const int tid = threadIdx.x;
  const AttnBlock blk = attn_block((p.Lmax + 127) / 128, p.H);
  const SeqRange sq = seq_range(p.cu, blk.z, p.Lmax);
  const int h = blk.h;
  const int i0 = blk.x * BM;
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

  // buffer views of this sequence's rows (reads past its end return zero)
  // and this thread's fixed offsets into them: issuing a tile's loads then
  // needs no address arithmetic
  const uint32_t seq_bytes = uint32_t(sq.len) * uint32_t(p.ts * ES);
  const BufView kview = buf_view(kbase, seq_bytes), vview = buf_view(vbase, seq_bytes);
  [[maybe_unused]] DmaRows<T, BN, D, KP, 256> kdma;
  [[maybe_unused]] DmaRows<T, BN, D, VP, 256> vdma;
  if constexpr (DMA) {
    kdma.init(p.ts);
    vdma.init(p.ts);
  }
  const BufView lview = buf_view(p.lutp, uint32_t(2 * p.Lmax - 1 + 2 * kLutPad) * 4u);
  // table slice entry tid of tile kb is packed entry (i0 - kb*BN - BN + 1 + tid) + Lmax - 1 + kLutPad
  const int lvoff = (i0 - BN + 1 + tid + p.Lmax - 1 + kLutPad) * 4;
  const BufView mview = buf_view(kmask, kmask ? uint32_t(sq.len) : 0u);
  const BufView eview_l = buf_view(ends + p2c_end_of(TILE_FAR_LEFT) * HT + sq.start, uint32_t(sq.len) * ES);
  const BufView eview_r = buf_view(ends + p2c_end_of(TILE_FAR_RIGHT) * HT + sq.start, uint32_t(sq.len) * ES);

  // ---- next-tile registers
  KTile kt, vt;
  kt.init();
  vt.init();
  // the next tile's per-key values and table slice, loaded raw and only
  // used when the tile is committed, so nothing waits for them (or for the
  // tile copy issued after them) before then; key mask and end values past
  // the sequence read 0 (the key is masked there anyway)
  T e_raw = TR::from_f(0.f);
  uint32_t m_raw = 1u, l_raw = 0u;

  // Issue the loads of tile kb into buffer Q (free since the last barrier).
  auto prefetch = [&](int kb, auto q_c) {
    constexpr int Q = decltype(q_c)::value;
    const int j0 = kb * BN;
    const int cls = cls_of(kb);
    if (tid < BN) {
      if (kmask) m_raw = buf_load_u8(mview, j0 + tid);
      e_raw = buf_load<T>(cls == TILE_FAR_LEFT ? eview_l : eview_r, tid * ES, j0 * ES);
    }
    if (tid < NL) l_raw = buf_load<uint32_t>(lview, lvoff - j0 * 4, 0);
    if constexpr (DMA) {
      kdma.issue(Q ? Ks1 : Ks0, kview, j0 * int(p.ts) * ES);
      vdma.issue(Q ? Vs1 : Vs0, vview, j0 * int(p.ts) * ES);
    } else {
      kt.load(kbase, p.ts, j0, sq.len);
      vt.load(vbase, p.ts, j0, sq.len);
    }
  };

  auto commit = [&](int kb, auto q_c) {
    constexpr int Q = decltype(q_c)::value;
    const int j0 = kb * BN;
    const int cls = cls_of(kb);
    if constexpr (!DMA) {
      kt.template store<KP>(Q ? Ks1 : Ks0);
      vt.template store<VP>(Q ? Vs1 : Vs0);
    }
    if (tid < BN) {
      const bool ok = j0 + tid < sq.len && m_raw != 0u;
      bj_s[Q][tid] = ok ? (cls != TILE_BAND ? TR::to_f(e_raw) : 0.f) : -INFINITY;
    }
    // both 16-bit halves scale to byte offsets at once (narrow: (R-1)*ES fits 16 bits)
    if (tid < NL) lut_s[Q][tid] = NARROW ? l_raw * ES : l_raw;
  };

  f32x16 O[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) O[nd] = zero16();
  float m = -INFINITY, l = 0.f;

  const int nkb = (sq.len + BN - 1) / BN;
  [[maybe_unused]] Win win;
  if constexpr (AWIN) {
    // window of tile 0 now, row starts of tile 1 for the first iteration
    if (cls_of(0) == TILE_BAND) {
      win.load_starts(p, i0 - BN + 1);
      win.issue(Wc0, c2pstrip, RP, i0, sq.len);
    }
    if (nkb > 1 && cls_of(1) == TILE_BAND) win.load_starts(p, i0 - BN - BN + 1);
  }
  prefetch(0, IntC<0>{});
  commit(0, IntC<0>{});
  wait_vmem();
  __syncthreads();

  // one tile; P = kb & 1 is the buffer it reads
  auto iter = [&](int kb, auto p_c) __attribute__((always_inline)) {
    constexpr int P = decltype(p_c)::value;
    constexpr int buf = P;
    const T* const Kc = P ? Ks1 : Ks0;
    const T* const Vc = P ? Vs1 : Vs0;
    const int j0 = kb * BN;
    const int cls = cls_of(kb);
    // loads for the next tiles: the next band tile's window into the other
    // buffer (free since the last barrier), the row starts of the band tile
    // after it, the next K/V tile
    auto issue_next = [&]() {
      if constexpr (AWIN) {
        if (kb + 1 < nkb && cls_of(kb + 1) == TILE_BAND) win.issue(P ? Wc0 : Wc1, c2pstrip, RP, i0, sq.len);
        if (kb + 2 < nkb && cls_of(kb + 2) == TILE_BAND) win.load_starts(p, i0 - (kb + 2) * BN - BN + 1);
      }
      if (kb + 1 < nkb) prefetch(kb + 1, IntC<P ^ 1>{});
    };

    // the score part of the tile body (relative terms, S MFMAs, softmax),
    // compiled once per tile class as straight-line code; it leaves the
    // packed probabilities, their row sum and the rescale factor
    issue_next();
    frag pf[NKT][32 / KS];
    float alpha, ls;
    auto body = [&](auto band_c) {
      constexpr bool BAND = decltype(band_c)::value;
      if constexpr (BAND && NARROW && !AWIN) {
        stage_window<T, WC, WCP, 256>(Wc0, c2pstrip, RP, BM, i0, sq.len,
                                      [&](int r) { return win_start_bytes<ES>(lut_c(lut_s[buf][r])) / ES; });
        __syncthreads();
      }
      const float a = BAND ? 0.f : (cls == TILE_FAR_LEFT ? a_end1 : a_end0);

      // relative terms (log2 domain) of this lane's 16*NKT keys. Band tiles
      // gather them before the score MFMAs so the LDS latency overlaps them.
      float rel[NKT][16];
      if constexpr (BAND) {
        const uint32_t* lrow = &lut_s[buf][il + BN - 1];  // entry of key jl: lrow[-jl]
        if constexpr (NARROW) {
          // C2P from this row's LDS window; P2C straight from the strip in
          // L2 (for a fixed key the 32 lanes of a half read one contiguous
          // run of its strip row; keys past the sequence end read zero)
          const char* wc = reinterpret_cast<const char*>(AWIN && P ? Wc1 : Wc0) +
                           (AWIN ? Win::row_offset(il) : il * WCP) * ES - win_start_bytes<ES>(lut_c(lut_s[buf][il]));
          const BufView prow = buf_view(p2cstrip, uint32_t(sq.len) * uint32_t(RP * ES));
          const int soff = j0 * RP * ES;
#pragma unroll
          for (int t = 0; t < NKT; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int jl = 32 * t + acc_row(v, g);
              const uint32_t e = lrow[-jl];
              rel[t][v] = TR::add2(*reinterpret_cast<const T*>(wc + lut_c(e)),
                                   buf_load<T>(prow, jl * RP * ES + lut_p(e), soff), bj_s[buf][jl]);
            }
        } else {
          const T* crow = c2pstrip + int64_t(qin ? iw : sq.len - 1) * RP;
#pragma unroll
          for (int t = 0; t < NKT; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int jl = 32 * t + acc_row(v, g);
              const uint32_t e = lrow[-jl];
              const int jj = min(j0 + jl, sq.len - 1);
              rel[t][v] = TR::add2(crow[lut_c(e)], p2cstrip[int64_t(jj) * RP + lut_p(e)], bj_s[buf][jl]);
            }
        }
      } else {
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
          for (int v = 0; v < 16; ++v) rel[t][v] = bj_s[buf][32 * t + acc_row(v, g)];
      }

      float y[NKT][16];
#pragma unroll
      for (int t = 0; t < NKT; ++t) {
        f32x16 acc = zero16();
#pragma unroll
        for (int q = 0; q < NQ; ++q) acc = TR::mma(ld_row<TR>(Kc, KP, 32 * t + li, q * KS + g * E), Qf[q], acc);
#pragma unroll
        for (int v = 0; v < 16; ++v) y[t][v] = fmaf(acc[v], p.scale_log2, rel[t][v]);
      }
      // online softmax (log2 domain); a is this tile's per-row C2P value
      float mt = -INFINITY;
#pragma unroll
      for (int t = 0; t < NKT; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) mt = fmaxf(mt, y[t][v]);
      mt = fmaxf(mt, xor32(mt)) + a;
      // the running max moves only when the tile's max exceeds it by more
      // than kMaxSlack (log2 units): otherwise the probabilities are taken
      // against the old max (at most 2^kMaxSlack, exact in fp32 sums and at
      // full relative precision in the 16-bit P operand) and O needs no
      // rescale; O / l and the LSE are the same either way
      const float mnew = mt > m + kMaxSlack ? mt : m;
      const float msafe = mnew == -INFINITY ? 0.f : mnew;
      const float m_old = m;
      const float shift = msafe - a;
#pragma unroll
      for (int t = 0; t < NKT; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) y[t][v] = fast_exp2(y[t][v] - shift);
      m = mnew;
      alpha = fast_exp2(m_old - msafe);
      // the row sum adds the same rounded P the MFMA uses
      ls = 0.f;
#pragma unroll
      for (int t = 0; t < NKT; ++t)
#pragma unroll
        for (int q = 0; q < 32 / KS; ++q) {
          pf[t][q] = TR::pack(&y[t][q * E]);
          ls = TR::sum(pf[t][q], ls);
        }
      if constexpr (DROP) {
        // the row sum above is of the undropped P; P V takes the dropped P
        // (kept or zero, unscaled: the 1 / (1 - p) factor multiplies O once
        // at the end, so the 16-bit operand never holds P / (1 - p)).
        // Registers 4k..4k+3 of a subtile hold four consecutive keys, one
        // Philox call.
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4) {
            const int j = j0 + 32 * t + acc_row(4 * k4, g);
            const Philox4 r = philox4x32_10(uint32_t(j) >> 2, uint32_t(iw), uint32_t(blk.z * p.H + h), p.drop_off,
                                            p.seed_lo, p.seed_hi);
#pragma unroll
            for (int e = 0; e < 4; ++e) y[t][4 * k4 + e] = r.w[e] >= p.drop_thr ? y[t][4 * k4 + e] : 0.f;
          }
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
          for (int q = 0; q < 32 / KS; ++q) pf[t][q] = TR::pack(&y[t][q * E]);
      }
    };
    if (cls == TILE_BAND)
      body(BoolC<true>{});
    else
      body(BoolC<false>{});

    // O^T += V^T P^T after the lazy rescale (same code for both classes, so
    // the accumulators are updated in place)
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int nd = 0; nd < ND; ++nd)
#pragma unroll
        for (int v = 0; v < 16; ++v) O[nd][v] *= alpha;
    }
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int q = 0; q < 32 / KS; ++q)
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) O[nd] = TR::mma(ld_col<TR>(Vc, VP, 32 * t, 32 * nd, q), pf[t][q], O[nd]);
    l = l * alpha + ls;

    if (kb + 1 < nkb) commit(kb + 1, IntC<P ^ 1>{});
    wait_vmem();
    __syncthreads();
  };
  for (int kb = 0; kb < nkb; kb += 2) {
    iter(kb, IntC<0>{});
    if (kb + 1 < nkb) iter(kb + 1, IntC<1>{});
  }

  const float lt = l + xor32(l);
  if (!qin) return;
  const bool ok = qvalid && lt > 0.f;
  const float inv = ok ? (DROP ? p.drop_scale : 1.f) / lt : 0.f;
  T* op = (T*)p.out + tok_i * p.ts + int64_t(h) * p.hs;
#pragma unroll
  for (int nd = 0; nd < ND; ++nd)
#pragma unroll
    for (int v = 0; v < 16; ++v) op[32 * nd + acc_row(v, g)] = TR::from_f(O[nd][v] * inv);
  if (g == 0 && p.lse) p.lse[int64_t(h) * T_ + tok_i] = ok ? (m + log2f(lt)) * kLn2 : -INFINITY;
}

template <int DT, int D, bool NARROW>
void launch_fwd_d(const Params& p, hipStream_t st) {
  dim3 grid(unsigned((p.Lmax + 127) / 128 * p.H * p.nseq));
  constexpr int NKT = (DT == DF_FP32_T && D == 128) ? 1 : 2;
  if (p.drop)
    fwd_kernel<DT, D, NKT, NARROW, true><<<grid, 256, 0, st>>>(p);
  else
    fwd_kernel<DT, D, NKT, NARROW, false><<<grid, 256, 0, st>>>(p);
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
