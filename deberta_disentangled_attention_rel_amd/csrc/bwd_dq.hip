// Backward, query side: dQ and the dense dC2P strip (DisentangledFlash 1.1.1
// page, "Hugging Face usage": an independently selected dQ kernel;
// "Performance": scores are recomputed in the backward).
//
// Work item: one sequence, one head, 128 queries (4 waves x 32 queries,
// resident in registers). The loop walks BN = 32*NKT keys at a time; the next
// tile (K and V rows, per-key P2C far-field values with the key mask folded
// in, table slice) is loaded into registers during the current one and
// written to the other half of a double-buffered LDS area (one barrier per
// tile); the K^T operand is read with transposing LDS reads. Each wave computes
// S^T = K Q^T and dP^T = V dO^T, so lane l owns query l % 32; P and dS are
// lane-local per query:
//   P = exp2(s log2e QK + rel - LSE log2e),  dS = P (dP - Delta)
//   dQ^T += K^T dS^T
//   dC2P[i, r] = sum_{j: delta(i,j) = r} dS[i, j]
// The strip row of query i is written by an ordered walk over the keys (one
// step per tile in the far field, where the whole tile shares one row). Once
// a wave's strip rows are complete, the same kernel adds the relative term
// dC2P K_r to its dQ accumulators (rel_epilogue) and writes dq. No atomics.
//
// The key tiles fall into three contiguous ranges (far-left, band,
// far-right), each with its own loop and its own copy of the tile body. Far
// tiles start the score accumulator at the per-key P2C end value and dP at
// -Delta, so P and dS take one FMA, one exp2 and one multiply per pair. Band
// tiles recompute the relative terms as the forward does: C2P from the
// query's LDS strip window, P2C straight from the strip in L2, both issued
// ahead of the score MFMAs.
#include "band.hpp"
#include "pipe.hpp"
#include "walk.hpp"

namespace dfa {

namespace {

template <int DT, int D, int NKT, bool NARROW, bool DROP>
__global__ __launch_bounds__(256, (DT != DF_FP32_T && (D <= 64 || NKT == 1)) ? 2 : 1) void dq_kernel(Params p) {
  using TR = Tr<DT>;
  using T = typename TR::T;
  using frag = typename TR::frag;
  constexpr int E = TR::E, KS = TR::KS, NQ = D / KS, ND = D / 32, ES = int(sizeof(T));
  constexpr int BM = 128, BN = 32 * NKT, NL = BM + BN - 1;
  constexpr int KP = RowPitch<T, D>::rows;
  constexpr int WC = BN + 8, WCP = WinPitch<T, WC>::v;
  static_assert(NL <= 256, "one table entry per thread");
  using KTile = RowTile<T, BN, D, 256, true>;  // keys half-major (walk order)

  __shared__ __align__(16) T Ks[2][BN * KP];
  __shared__ __align__(16) T Vs[2][BN * KP];
  __shared__ __align__(16) float bj_s[2][BN];
  __shared__ uint32_t lut_s[2][NL];
  __shared__ __align__(16) T Wc[NARROW ? BM * WCP : 1];

  const int lane = threadIdx.x & 63, g = lane >> 5, li = lane & 31, wave = threadIdx.x >> 6;
  const int tid = threadIdx.x;
  const AttnBlock blk = attn_block((p.Lmax + 127) / 128, p.H);
  const SeqRange sq = seq_range(p.cu, blk.z, p.Lmax);
  const int h = blk.h;
  const int i0 = blk.x * BM;
  if (i0 >= sq.len) return;
  const int64_t T_ = p.T, HT = int64_t(p.H) * p.T;
  const int R = p.R, RP = p.RP;
  const int d_hi = p.d_hi, d_lo = p.d_lo;

  const int il = wave * 32 + li;
  const int iw = i0 + il;
  const bool qin = iw < sq.len;
  const int64_t tok_i = sq.start + (qin ? iw : sq.len - 1);
  const bool qvalid = qin && (!p.kmask || p.kmask[tok_i]);

  frag Qf[NQ], dOf[NQ];
  {
    const T* qp = (const T*)p.q + tok_i * p.ts + int64_t(h) * p.hs;
    const T* dp = (const T*)p.dout + tok_i * p.ts + int64_t(h) * p.hs;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      Qf[q] = TR::ld(qp + q * KS + g * E);
      dOf[q] = TR::ld(dp + q * KS + g * E);
    }
  }
  // masked query: P = 0 through an infinite LSE
  const float lse2 = qvalid ? p.lse[int64_t(h) * T_ + tok_i] * kLog2e : INFINITY;
  const float dlt = qvalid ? p.delta[int64_t(h) * T_ + tok_i] : 0.f;
  const float inv_sl = 1.f / p.scale_log2;
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

  KTile kt, vt;
  kt.init();
  vt.init();
  // buffer views of this sequence's rows (reads past its end return zero),
  // so that a tile's loads take a scalar row offset and no branch
  const uint32_t seq_bytes = uint32_t(sq.len) * uint32_t(p.ts * ES);
  const BufView kview = buf_view(kbase, seq_bytes), vview = buf_view(vbase, seq_bytes);
  const BufView lview = buf_view(p.lutp, uint32_t(2 * p.Lmax - 1 + 2 * kLutPad) * 4u);
  // table slice entry tid of key tile kb is packed entry (i0 - kb*BN - BN + 1 + tid) + Lmax - 1 + kLutPad
  const int lvoff = (i0 - BN + 1 + tid + p.Lmax - 1 + kLutPad) * 4;
  const BufView mview = buf_view(kmask, kmask ? uint32_t(sq.len) : 0u);
  const BufView eview_l = buf_view(ends + p2c_end_of(TILE_FAR_LEFT) * HT + sq.start, uint32_t(sq.len) * ES);
  const BufView eview_r = buf_view(ends + p2c_end_of(TILE_FAR_RIGHT) * HT + sq.start, uint32_t(sq.len) * ES);
  // the next tile's per-key values and table slice, loaded raw and used when
  // the tile is committed (past the sequence end they read 0; such keys are
  // masked)
  T e_raw = TR::from_f(0.f);
  uint32_t m_raw = 1u, lreg = 0;

  auto prefetch = [&](int kb) {
    const int j0 = kb * BN;
    const int cls = cls_of(kb);
    kt.load_buf(kview, p.ts, j0 * int(p.ts) * ES);
    vt.load_buf(vview, p.ts, j0 * int(p.ts) * ES);
    if (tid < BN) {
      if (kmask) m_raw = buf_load_u8(mview, j0 + tid);
      e_raw = buf_load<T>(cls == TILE_FAR_LEFT ? eview_l : eview_r, tid * ES, j0 * ES);
    }
    if (cls == TILE_BAND && tid < NL) lreg = buf_load<uint32_t>(lview, lvoff - j0 * 4, 0);
  };

  auto commit = [&](int kb) {
    const int buf = kb & 1;
    const int j0 = kb * BN;
    const int cls = cls_of(kb);
    kt.template store<KP>(Ks[buf]);
    vt.template store<KP>(Vs[buf]);
    // per key: far tiles its P2C end value divided by s log2 e (it seeds the
    // score accumulator), band tiles 0; -inf if masked
    if (tid < BN) {
      const bool ok = j0 + tid < sq.len && m_raw != 0u;
      bj_s[buf][tid] = ok ? (cls != TILE_BAND ? TR::to_f(e_raw) * inv_sl : 0.f) : -INFINITY;
    }
    // both 16-bit halves scale to byte offsets at once (narrow: (R-1)*ES fits 16 bits)
    if (tid < NL) lut_s[buf][tid] = NARROW ? lreg * ES : lreg;
  };

  f32x16 dQt[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) dQt[nd] = zero16();
  T* wrow = (T*)p.dc2p + (int64_t(h) * T_ + tok_i) * RP;  // this query's dC2P row
  // the dC2P rows of this work-group's queries, for the band-tile walk steps
  const BufView wview = buf_view((T*)p.dc2p + (int64_t(h) * T_ + sq.start + i0) * RP,
                                 uint32_t(min(BM, sq.len - i0)) * uint32_t(RP * ES));
  const int wbase = il * RP * ES;
  int rc = R;                                                // open run (half 0): none yet
  float sc = 0.f;
  if constexpr (NARROW) {
    rc = lut_c(lut_entry(p, qin ? iw : 0));  // row of key 0
    if (qin && g == 0) walk_open<TR>(wrow, R, rc);
  }

  const int nkb = (sq.len + BN - 1) / BN;
  // the key tiles fall into three contiguous ranges: far-left (tile kb with
  // i0 - kb*BN - BN + 1 >= d_hi), band, far-right (i0 + BM - 1 - kb*BN <=
  // d_lo); each range runs its own loop, so the far loops carry none of the
  // band tiles' gathers, windows and walk state
  const int nl = i0 - BN + 1 - d_hi;
  const int kb_band = min(nkb, nl >= 0 ? nl / BN + 1 : 0);
  const int kb_right = max(kb_band, min(nkb, (i0 + BM - 1 - d_lo + BN - 1) / BN));
  prefetch(0);
  commit(0);
  __syncthreads();

  auto iter = [&](int kb, auto band_c) __attribute__((always_inline)) {
    const int buf = kb & 1;
    const int j0 = kb * BN;
    const int cls = decltype(band_c)::value ? TILE_BAND : cls_of(kb);
    // band tiles: the C2P window is staged before the next tile's loads are
    // issued (a wave's vector memory operations complete in order, so the
    // staging's wait then does not wait for those)
    if constexpr (decltype(band_c)::value && NARROW) {
      stage_window<T, WC, WCP, 256>(Wc, c2pstrip, RP, BM, i0, sq.len,
                                    [&](int r) { return win_start_bytes<ES>(lut_c(lut_s[buf][r])) / ES; });
      __syncthreads();
    }
    if (kb + 1 < nkb) prefetch(kb + 1);

    // the tile body, compiled once per tile class as straight-line code
    auto body = [&](auto band_c) {
      constexpr bool BAND = decltype(band_c)::value;
      const float w = (BAND ? 0.f : (cls == TILE_FAR_LEFT ? a_end1 : a_end0)) - lse2;

      // relative terms (log2 domain) of this lane's keys; band tiles gather
      // them before the score MFMAs so the gather latency overlaps them
      float rel[NKT][16];
      if constexpr (BAND) {
        const uint32_t* lrow = &lut_s[buf][il + BN - 1];  // entry of key jl: lrow[-jl]
        if constexpr (NARROW) {
          // C2P from this row's LDS window; P2C straight from the strip in L2
          // (for a fixed key the lanes of a half read one contiguous run)
          const char* wc = reinterpret_cast<const char*>(Wc) + il * WCP * ES - win_start_bytes<ES>(lut_c(lut_s[buf][il]));
          const BufView prow = buf_view(p2cstrip, uint32_t(sq.len) * uint32_t(RP * ES));
          const int soff = j0 * RP * ES;
#pragma unroll
          for (int t = 0; t < NKT; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int jl = half_major_partner<NKT>(t, g, v);
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
              const int jl = half_major_partner<NKT>(t, g, v);
              const uint32_t e = lrow[-jl];
              const int jj = min(j0 + jl, sq.len - 1);
              rel[t][v] = TR::add2(crow[lut_c(e)], p2cstrip[int64_t(jj) * RP + lut_p(e)], bj_s[buf][jl]);
            }
        }
      }

      // band tiles: each lane group walks its own half of the keys (the tile
      // is stored half-major, so those are its 16*NKT registers in order)
      WalkHalf wk = walk_begin(g, rc, sc, -1);
      if constexpr (BAND)
        wk = walk_begin(g, rc, sc,
                        j0 + 16 * NKT < sq.len ? lut_c(lut_s[buf][il - 16 * NKT + BN - 1]) / (NARROW ? ES : 1) : -1);
      float rowsum = 0.f;
#pragma unroll
      for (int t = 0; t < NKT; ++t) {
        // far tiles: the per-key terms seed the score accumulator and -Delta
        // the dP one (P = exp2(fma(S, s log2 e, w)), dS = P dP)
        f32x16 S = BAND ? zero16() : seq16(&bj_s[buf][half_major_partner<NKT>(t, g, 0)]);
        f32x16 dP = (BAND || DROP) ? zero16() : splat16(-dlt);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          S = TR::mma(ld_row<TR>(Ks[buf], KP, 32 * t + li, q * KS + g * E), Qf[q], S);
          dP = TR::mma(ld_row<TR>(Vs[buf], KP, 32 * t + li, q * KS + g * E), dOf[q], dP);
        }
        float dS[16];
        if constexpr (DROP) {
          // dS = P (F dP - Delta), F = keep / (1 - p). The keys are
          // half-major: registers 8c .. 8c+7 hold the eight keys of one
          // Philox block, so each lane computes its own two calls
          const int jb = j0 + half_major_partner<NKT>(t, g, 0);  // a multiple of 16
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const Philox4 r = philox4x32_10(uint32_t(jb >> 3) + uint32_t(c), uint32_t(iw), uint32_t(blk.z * p.H + h),
                                            p.drop_off, p.seed_lo, p.seed_hi);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int v = 8 * c + e;
              const float P = BAND ? fast_exp2(fmaf(S[v], p.scale_log2, rel[t][v]) + w)
                                   : fast_exp2(fmaf(S[v], p.scale_log2, w));
              const bool keep = (e & 1) ? keep_hi(r.w[e >> 1], p.drop_thr) : keep_lo(r.w[e >> 1], p.drop_thr);
              dS[v] = P * fmaf(dP[v], keep ? p.drop_scale : 0.f, -dlt);
            }
          }
        } else {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            if constexpr (BAND) {
              const float P = fast_exp2(fmaf(S[v], p.scale_log2, rel[t][v]) + w);
              dS[v] = P * (dP[v] - dlt);
            } else {
              dS[v] = fast_exp2(fmaf(S[v], p.scale_log2, w)) * dP[v];
            }
          }
        }
        // the subtile's K fragments first, so their reads share the waits
        frag fk[32 / KS][ND];
#pragma unroll
        for (int q = 0; q < 32 / KS; ++q)
#pragma unroll
          for (int nd = 0; nd < ND; ++nd) fk[q][nd] = ld_col<TR>(Ks[buf], KP, 32 * t, 32 * nd, q);
#pragma unroll
        for (int q = 0; q < 32 / KS; ++q) {
          const frag sb = TR::pack(&dS[q * E]);
          // far tiles: this lane's part of the row sum (of the rounded dS the
          // MFMA uses)
          if constexpr (!BAND) rowsum = TR::sum(sb, rowsum);
#pragma unroll
          for (int nd = 0; nd < ND; ++nd) dQt[nd] = TR::mma(fk[q][nd], sb, dQt[nd]);
        }
        if constexpr (BAND) {
          // dC2P: this half's keys of the subtile, in order (a block of its
          // own, so the scheduler keeps it apart from the next subtile)
          if (qin) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int jl = half_major_partner<NKT>(t, g, v);
              const int r = lut_c(lut_s[buf][il - jl + BN - 1]) / (NARROW ? ES : 1);
              if constexpr (NARROW)
                walk_step_narrow<TR>(wview, wbase, wk, r, dS[v], j0 + jl < sq.len);
              else
                walk_step<TR, false>(wrow, R, wk, r, dS[v], j0 + jl < sq.len);
            }
          }
        }
      }
      if constexpr (!BAND) {
        rowsum += xor32(rowsum);  // the query's two lane halves
        if (qin && g == 0) {
          walk_step<TR, NARROW>(wrow, R, wk, cls == TILE_FAR_LEFT ? R - 1 : 0, rowsum);
          rc = wk.r;
          sc = wk.s;
        }
      } else {
        walk_merge<TR>(wrow, R, g, wk, rc, sc, qin);
      }
    };
    body(band_c);

    if (kb + 1 < nkb) commit(kb + 1);
    __syncthreads();
  };
  int kb = 0;
  for (; kb < kb_band; ++kb) iter(kb, BoolC<false>{});
  for (; kb < kb_right; ++kb) iter(kb, BoolC<true>{});
  for (; kb < nkb; ++kb) iter(kb, BoolC<false>{});

  // close this query's dC2P row, then add the relative term dC2P K_r: the
  // wave's rows are complete once its own stores are (no other wave writes
  // them, and no cache above L2 holds them)
  if (qin && g == 0) walk_finish<TR>(wrow, R, RP, rc, sc);
  wait_vmem();
  rel_epilogue<TR, ND>(dQt, wview, wbase, buf_view((const T*)p.krT + int64_t(h) * D * RP, uint32_t(D * RP * ES)), RP);
  if (!qin) return;
  T* dqp = (T*)p.dq + tok_i * p.ts + int64_t(h) * p.hs;
#pragma unroll
  for (int nd = 0; nd < ND; ++nd)
#pragma unroll
    for (int v = 0; v < 16; ++v) dqp[32 * nd + acc_row(v, g)] = TR::from_f(dQt[nd][v] * p.scale);
}

template <int DT, int D, bool NARROW>
void launch_d(const Params& p, hipStream_t st) {
  dim3 grid(unsigned((p.Lmax + 127) / 128 * p.H * p.nseq));
  // D=128: 32-key tiles, which fit two work-groups per CU (two waves per
  // SIMD); a 64-key tile needs one per CU
  constexpr int NKT = D == 128 ? 1 : 2;
  if (p.drop)
    dq_kernel<DT, D, NKT, NARROW, true><<<grid, 256, 0, st>>>(p);
  else
    dq_kernel<DT, D, NKT, NARROW, false><<<grid, 256, 0, st>>>(p);
}

template <int DT, int D>
void launch_n(const Params& p, hipStream_t st) {
  if (p.narrow)
    launch_d<DT, D, true>(p, st);
  else
    launch_d<DT, D, false>(p, st);
}

template <int DT>
void launch_dt(const Params& p, hipStream_t st) {
  switch (p.D) {
    case 32: launch_n<DT, 32>(p, st); break;
    case 64: launch_n<DT, 64>(p, st); break;
    default: launch_n<DT, 128>(p, st); break;
  }
}

}  // namespace

hipError_t launch_bwd_dq(const Params& p, hipStream_t st) {
  switch (p.dtype) {
    case DF_BF16_T: launch_dt<DF_BF16_T>(p, st); break;
    case DF_FP16_T: launch_dt<DF_FP16_T>(p, st); break;
    default: launch_dt<DF_FP32_T>(p, st); break;
  }
  return hipGetLastError();
}

}  // namespace dfa
