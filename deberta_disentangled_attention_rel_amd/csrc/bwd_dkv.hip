// Backward, key side: dK, dV and the dense dP2C strip (DisentangledFlash
// 1.1.1 page, "Hugging Face usage": an independently selected dK/dV kernel;
// "Performance": the backward recomputes the score products). Determinism
// follows the FastFlashAttention page ("Determinism"): every output element is
// written once, by its owner, with no atomics.
//
// Work item: one sequence, one head, 128 keys (4 waves x 32 keys, resident
// in registers). The loop walks BM = 32*NQT queries at a time; the next query
// tile (Q and dO rows, per-query LSE/Delta/C2P-end values, table slice) is
// loaded into registers during the current one and written to the other half
// of a double-buffered LDS area (one barrier per tile); the Q^T and dO^T
// operands are read with transposing LDS reads. Each wave computes S = Q K^T and
// dP = dO V^T with 32x32 MFMAs, so lane l owns key l % 32 and holds 16 of
// every 32 queries:
//   P = exp2(s log2e QK + rel - LSE log2e),  dS = P (dP - Delta)
//   dV^T += dO^T P,   dK^T += Q^T dS
//   dP2C[j, r] = sum_{i: delta(j,i) = r} dS[i, j]
// The strip row of key j is written by an ordered walk over the queries (one
// step per tile in the far field). Once a wave's strip rows are complete, the
// same kernel adds the relative term dP2C Q_r to its dK accumulators
// (rel_epilogue) and writes dk.
//
// The query tiles fall into three contiguous ranges (far-right, band,
// far-left), each with its own loop and its own copy of the tile body (the
// dropout bodies, which need more registers, keep one loop that decides the
// class per tile). Far tiles start the score accumulator at the per-query
// (C2P end - LSE log2e) / (s log2e) and dP at -Delta. Band tiles gather both
// relative terms from LDS strip windows (one C2P row per query, one P2C row
// per key); the table slice holds byte offsets, so a gather address is one
// add, and the two values and the per-key mask term are joined with one
// packed dot product.
#include "band.hpp"
#include "pipe.hpp"
#include "walk.hpp"

namespace dfa {

namespace {

template <int DT, int D, int NQT, bool NARROW, bool DROP>
__global__ __launch_bounds__(256, (D <= 64 && DT != DF_FP32_T) ? 2 : 1) void dkv_kernel(Params p) {
  using TR = Tr<DT>;
  using T = typename TR::T;
  using frag = typename TR::frag;
  constexpr int E = TR::E, KS = TR::KS, NQ = D / KS, ND = D / 32, ES = int(sizeof(T));
  constexpr bool DMA = ES == 2;  // 16-bit tiles go global -> LDS without registers
  constexpr int BN = 128, BM = 32 * NQT, NL = BM + BN - 1;
  constexpr int QP = RowPitch<T, D>::rows;
  constexpr int WC = BN + 8, WCP = WinPitch<T, WC>::v;   // C2P window: one row per query
  constexpr int WPW = BM + 8, WPP = WinPitch<T, WPW>::v;  // P2C window: one row per key
  static_assert(NL <= 256, "one table entry per thread");
  using QTile = RowTile<T, BM, D, 256, true>;  // queries half-major (walk order)

  __shared__ __align__(16) T Qs[2][BM * QP];
  __shared__ __align__(16) T dOs[2][BM * QP];
  // per query: ((C2P end) - LSE*log2e) / (s*log2e) (-inf if masked), the
  // start of its score accumulator; and -Delta, the start of its dP
  // accumulator
  __shared__ __align__(16) float uq_s[2][BM];
  __shared__ __align__(16) float dlt_s[2][BM];
  __shared__ uint32_t lut_s[2][NL];
  // strip windows of band tiles: 16-bit types copy the next band tile's
  // windows by LDS-DMA halfway through the current tile, as soon as its last
  // gather is done; fp32 stages them when the tile starts
  constexpr bool AWIN = NARROW && DMA;
  using WcW = WinDma<uint16_t, BM, WC / 8, false, 256>;  // one row per query (lanes read along it)
  using WpW = WinDma<uint16_t, BN, WPW / 8, true, 256>;  // one row per key (lanes read across rows)
  __shared__ __align__(16) T Wc[AWIN ? WcW::ELEMS : (NARROW ? BM * WCP : 1)];
  __shared__ __align__(16) T Wp[AWIN ? WpW::ELEMS : (NARROW ? BN * WPP : 1)];
  __shared__ int cb_s[NARROW ? BM : 1];  // per query: byte base of its C2P window row

  const int lane = threadIdx.x & 63, g = lane >> 5, li = lane & 31, wave = threadIdx.x >> 6;
  const int tid = threadIdx.x;
  const AttnBlock blk = attn_block((p.Lmax + 127) / 128, p.H);
  const SeqRange sq = seq_range(p.cu, blk.z, p.Lmax);
  const int h = blk.h;
  const int j0 = blk.x * BN;
  if (j0 >= sq.len) return;
  const int64_t T_ = p.T, HT = int64_t(p.H) * p.T;
  const int RP = p.RP;
  const int d_hi = p.d_hi, d_lo = p.d_lo;

  const int jl = wave * 32 + li;  // this lane's key within the block
  const int jw = j0 + jl;
  const bool jin = jw < sq.len;
  const int64_t tok_j = sq.start + (jin ? jw : sq.len - 1);
  const bool kvalid = jin && (!p.kmask || p.kmask[tok_j]);

  frag Kf[NQ], Vf[NQ];
  {
    const T* kp = (const T*)p.k + tok_j * p.ts + int64_t(h) * p.hs;
    const T* vp = (const T*)p.v + tok_j * p.ts + int64_t(h) * p.hs;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      Kf[q] = TR::ld(kp + q * KS + g * E);
      Vf[q] = TR::ld(vp + q * KS + g * E);
    }
  }
  const T* ends = (const T*)p.ends + int64_t(h) * T_;
  const float kbias = kvalid ? 0.f : -INFINITY;
  const float inv_sl = 1.f / p.scale_log2;
  const float b_end0 = TR::to_f(ends[2 * HT + tok_j]) + kbias;  // P2C column 0
  const float b_end1 = TR::to_f(ends[3 * HT + tok_j]) + kbias;  // P2C column R-1
  const T* c2pstrip = (const T*)p.c2ps + (int64_t(h) * T_ + sq.start) * RP;
  const T* p2cstrip = (const T*)p.p2cs + (int64_t(h) * T_ + sq.start) * RP;
  const T* qbase = (const T*)p.q + sq.start * p.ts + int64_t(h) * p.hs;
  const T* dobase = (const T*)p.dout + sq.start * p.ts + int64_t(h) * p.hs;
  const float* lse = p.lse + int64_t(h) * T_ + sq.start;
  const float* dlt = p.delta + int64_t(h) * T_ + sq.start;
  const uint8_t* kmask = p.kmask ? p.kmask + sq.start : nullptr;

  auto cls_of = [&](int qb) {
    const int i0 = qb * BM;
    return tile_class(i0 - j0 - BN + 1, i0 + BM - 1 - j0, d_hi, d_lo);
  };

  QTile qt, ot;
  qt.init();
  ot.init();
  // buffer views of this sequence's rows (reads past its end return zero)
  // and this thread's fixed offsets into them, so that issuing a query tile
  // takes no address arithmetic
  const uint32_t seq_bytes = uint32_t(sq.len) * uint32_t(p.ts * ES);
  const BufView qview = buf_view(qbase, seq_bytes), oview = buf_view(dobase, seq_bytes);
  [[maybe_unused]] DmaRows<T, BM, D, QP, 256, true> qdma;  // half-major, the same offsets for Q and dO
  if constexpr (DMA) qdma.init(p.ts);
  const BufView lview = buf_view(p.lutp, uint32_t(2 * p.Lmax - 1 + 2 * kLutPad) * 4u);
  // table slice entry tid of query tile qb is packed entry (qb*BM - j0 - BN + 1 + tid) + Lmax - 1 + kLutPad
  const int lvoff = (tid - j0 - BN + 1 + p.Lmax - 1 + kLutPad) * 4;
  const BufView mview = buf_view(kmask, kmask ? uint32_t(sq.len) : 0u);
  const BufView lsev = buf_view(lse, uint32_t(sq.len) * 4u), dltv = buf_view(dlt, uint32_t(sq.len) * 4u);
  const BufView eview_l = buf_view(ends + c2p_end_of(TILE_FAR_LEFT) * HT + sq.start, uint32_t(sq.len) * ES);
  const BufView eview_r = buf_view(ends + c2p_end_of(TILE_FAR_RIGHT) * HT + sq.start, uint32_t(sq.len) * ES);
  // the next tile's per-query values and table slice, loaded raw and only
  // used when the tile is committed
  T a_raw = TR::from_f(0.f);
  float lse_raw = 0.f, dlt_raw = 0.f;
  uint32_t m_raw = 1u, lreg = 0;

  auto prefetch = [&](int qb) {
    const int i0 = qb * BM;
    const int cls = cls_of(qb);
    if constexpr (DMA) {
      // straight into the free LDS buffer (last read two tiles ago)
      qdma.issue(Qs[qb & 1], qview, i0 * int(p.ts) * ES);
      qdma.issue(dOs[qb & 1], oview, i0 * int(p.ts) * ES);
    } else {
      qt.load(qbase, p.ts, i0, sq.len);
      ot.load(dobase, p.ts, i0, sq.len);
    }
    if (tid < BM) {
      // past the sequence end all of these read 0 (the row is masked there)
      if (kmask) m_raw = buf_load_u8(mview, i0 + tid);
      a_raw = buf_load<T>(cls == TILE_FAR_LEFT ? eview_l : eview_r, tid * ES, i0 * ES);
      lse_raw = buf_load<float>(lsev, tid * 4, i0 * 4);
      dlt_raw = buf_load<float>(dltv, tid * 4, i0 * 4);
    }
    if (cls == TILE_BAND && tid < NL) lreg = buf_load<uint32_t>(lview, lvoff + i0 * 4, 0);
  };
  auto commit = [&](int qb) {
    const int buf = qb & 1;
    const int i0 = qb * BM;
    const int cls = cls_of(qb);
    if constexpr (!DMA) {
      qt.template store<QP>(Qs[buf]);
      ot.template store<QP>(dOs[buf]);
    }
    if (tid < BM) {
      const bool ok = i0 + tid < sq.len && m_raw != 0u;
      const float a = cls != TILE_BAND ? TR::to_f(a_raw) : 0.f;
      uq_s[buf][tid] = ok ? (a - lse_raw * kLog2e) * inv_sl : -INFINITY;
      dlt_s[buf][tid] = ok ? -dlt_raw : 0.f;
    }
    // both 16-bit halves scale to byte offsets at once (narrow: (R-1)*ES fits 16 bits)
    if (tid < NL) lut_s[buf][tid] = NARROW ? lreg * ES : lreg;
  };

  f32x16 dVt[ND], dKt[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) {
    dVt[nd] = zero16();
    dKt[nd] = zero16();
  }
  const int R = p.R;
  T* wrow = (T*)p.dp2c + (int64_t(h) * T_ + tok_j) * RP;  // this key's dP2C row
  // the dP2C rows of this work-group's keys, for the band-tile walk steps
  const BufView wview = buf_view((T*)p.dp2c + (int64_t(h) * T_ + sq.start + j0) * RP,
                                 uint32_t(min(BN, sq.len - j0)) * uint32_t(RP * ES));
  const int wbase = jl * RP * ES;
  int rc = R;                                                // open run (half 0): none yet
  float sc = 0.f;
  if constexpr (NARROW) {
    rc = lut_p(lut_entry(p, -(jin ? jw : 0)));  // row of query 0
    if (jin && g == 0) walk_open<TR>(wrow, R, rc);
  }

  // the sequence's strip rows of this head, for the window copies
  const BufView c2pview = buf_view(c2pstrip, uint32_t(sq.len) * uint32_t(RP * ES));
  const BufView p2cview = buf_view(p2cstrip, uint32_t(sq.len) * uint32_t(RP * ES));
  // windows of the band tile whose table slice is in lut_s[lb]
  [[maybe_unused]] auto issue_windows = [&](int lb, int i0n) {
    if constexpr (AWIN) {
      WcW::issue(reinterpret_cast<uint16_t*>(Wc), c2pview, RP, i0n, sq.len,
                 [&](int, int r) { return win_start_bytes<ES>(lut_c(lut_s[lb][r])) / ES; });
      WpW::issue(reinterpret_cast<uint16_t*>(Wp), p2cview, RP, j0, sq.len,
                 [&](int, int r) { return win_start_bytes<ES>(lut_p(lut_s[lb][NL - 1 - r])) / ES; });
      if (tid < BM) cb_s[tid] = WcW::row_offset(tid) * ES - win_start_bytes<ES>(lut_c(lut_s[lb][tid]));
    }
  };

  const int nqb = (sq.len + BM - 1) / BM;
  // the query tiles fall into three contiguous ranges: far-right (tile qb
  // with qb*BM + BM - 1 - j0 <= d_lo), band, far-left (qb*BM - j0 - BN + 1
  // >= d_hi); each range runs its own loop, so the far loops carry none of
  // the band tiles' gathers, windows and walk state
  const int nr = d_lo + j0 - BM + 1;
  const int qb_band = min(nqb, nr >= 0 ? nr / BM + 1 : 0);
  const int qb_left = max(qb_band, min(nqb, (j0 + BN - 1 + d_hi + BM - 1) / BM));
  prefetch(0);
  commit(0);
  wait_vmem();
  __syncthreads();
  if constexpr (AWIN) {
    if (qb_band == 0 && qb_left > 0) {
      issue_windows(0, 0);
      wait_vmem();
      __syncthreads();
    }
  }

  // body of one query tile; mode: 0 far, 1 band (both compiled for that
  // class alone), 2 decided per tile
  auto iter = [&](int qb, auto mode_c) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode_c)::value;
    const int buf = qb & 1;
    const int i0 = qb * BM;
    const bool BAND = MODE == 2 ? (qb >= qb_band && qb < qb_left) : MODE == 1;
    [[maybe_unused]] const bool next_band = qb + 1 >= qb_band && qb + 1 < qb_left;
    if (qb + 1 < nqb) prefetch(qb + 1);
    if (NARROW && !AWIN && BAND) {
      stage_window<T, WC, WCP, 256>(Wc, c2pstrip, RP, BM, i0, sq.len,
                                    [&](int r) { return win_start_bytes<ES>(lut_c(lut_s[buf][r])) / ES; });
      stage_window<T, WPW, WPP, 256>(Wp, p2cstrip, RP, BN, j0, sq.len,
                                     [&](int r) { return win_start_bytes<ES>(lut_p(lut_s[buf][NL - 1 - r])) / ES; });
      if (tid < BM) cb_s[tid] = tid * WCP * ES - win_start_bytes<ES>(lut_c(lut_s[buf][tid]));
      __syncthreads();
    }

    // far tiles: the per-key P2C term of the tile's class
    const bool left = qb >= qb_left;
    const float bj = left ? b_end0 : b_end1;
    // byte base of this key's P2C window row
    [[maybe_unused]] const char* wp =
        reinterpret_cast<const char*>(Wp) + (AWIN ? WpW::row_offset(jl) : jl * WPP) * ES -
        (NARROW && BAND ? win_start_bytes<ES>(lut_p(lut_s[buf][NL - 1 - jl])) : 0);

    // band tiles: each lane group walks its own half of the queries (the
    // tile is stored half-major, so those are its 16*NQT registers in order)
    WalkHalf wk = walk_begin(g, rc, sc, -1);
    if (BAND) {
      const int r1 = i0 + 16 * NQT < sq.len ? lut_p(lut_s[buf][16 * NQT - jl + BN - 1]) / (NARROW ? ES : 1) : -1;
      wk = walk_begin(g, rc, sc, r1);
    }
    float colsum = 0.f;
#pragma unroll
    for (int u = 0; u < NQT; ++u) {
      // band tiles: the gathered C2P + P2C terms of this subtile's pairs (one
      // block per subtile, so the 16 gathers are in flight together); the
      // per-query C2P value minus the LSE seeds the score accumulator
      [[maybe_unused]] float rel[16];
      if (BAND) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int il = half_major_partner<NQT>(u, g, v);
          const uint32_t e = lut_s[buf][il - jl + BN - 1];
          if constexpr (NARROW) {
            rel[v] = TR::add2(*reinterpret_cast<const T*>(reinterpret_cast<const char*>(Wc) + cb_s[il] + lut_c(e)),
                              *reinterpret_cast<const T*>(wp + lut_p(e)), kbias);
          } else {
            const int ii = min(i0 + il, sq.len - 1);
            rel[v] = TR::add2(c2pstrip[int64_t(ii) * RP + lut_c(e)],
                              p2cstrip[int64_t(jin ? jw : sq.len - 1) * RP + lut_p(e)], kbias);
          }
        }
      }
      if constexpr (AWIN && MODE != 0) {
        if (u == NQT - 1 && next_band) {
          // this tile's last gather is issued: publish the next tile's table
          // slice and wait for every wave to be done with the windows; the
          // next tile's windows are copied once this tile's MFMAs have read
          // their operands (an LDS-DMA copy in flight makes the compiler
          // hold back the transposing reads that follow it)
          if (tid < NL) lut_s[buf ^ 1][tid] = NARROW ? lreg * ES : lreg;
          __syncthreads();
        }
      }
      // registers v of this lane group hold the subtile's queries ib + v
      const int ib = half_major_partner<NQT>(u, g, 0);
      f32x16 S = seq16(&uq_s[buf][ib]);
      f32x16 dP = DROP ? zero16() : seq16(&dlt_s[buf][ib]);  // dP - Delta without dropout
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        S = TR::mma(ld_row<TR>(Qs[buf], QP, 32 * u + li, q * KS + g * E), Kf[q], S);
        dP = TR::mma(ld_row<TR>(dOs[buf], QP, 32 * u + li, q * KS + g * E), Vf[q], dP);
      }
      float P[16], dS[16];
      [[maybe_unused]] uint32_t wd[8];
      if constexpr (DROP) {
        // This lane's key takes 16 bits of the call for (query, key block
        // jw / 8), and the eight lanes 8m .. 8m+7 hold the eight keys of one
        // block and the same 16 queries (slots v, queries ib + v). Lane e of
        // the eight computes the calls of slots 2e and 2e + 1 and packs, for
        // each lane d of the eight, the bits of key d of both calls into one
        // word (low half slot 2e, high half slot 2e + 1); an 8 x 8 transpose
        // of those words (an exchange with lane e ^ 4, then a 4 x 4
        // transpose in each quad) leaves wd[s] = key jw's bits of slots 2s
        // (low half) and 2s + 1 (high half).
        const int e = lane & 7;
        const uint32_t i2 = uint32_t(i0 + ib + 2 * e);
        const Philox4 r0 = philox4x32_10(uint32_t(jw) >> 3, i2, uint32_t(blk.z * p.H + h), p.drop_off, p.seed_lo,
                                         p.seed_hi);
        const Philox4 r1 = philox4x32_10(uint32_t(jw) >> 3, i2 + 1u, uint32_t(blk.z * p.H + h), p.drop_off,
                                         p.seed_lo, p.seed_hi);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // key 2k: low halves of word k, key 2k + 1: high halves
          wd[2 * k] = (r0.w[k] & 0xFFFFu) | (r1.w[k] << 16);
          wd[2 * k + 1] = (r0.w[k] >> 16) | (r1.w[k] & 0xFFFF0000u);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) xor4_swap(wd[k], wd[k + 4]);
        quad_transpose(wd[0], wd[1], wd[2], wd[3], e & 3);
        quad_transpose(wd[4], wd[5], wd[6], wd[7], e & 3);
      }
      if (BAND) {
#pragma unroll
        for (int v = 0; v < 16; ++v) P[v] = fast_exp2(fmaf(S[v], p.scale_log2, rel[v]));
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) P[v] = fast_exp2(fmaf(S[v], p.scale_log2, bj));
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        if constexpr (DROP) {
          // dS = P (F dP - Delta), F = keep / (1 - p); dV takes P keep (the
          // 1 / (1 - p) factor multiplies dV once at the end)
          const bool keep = (v & 1) ? keep_hi(wd[v >> 1], p.drop_thr) : keep_lo(wd[v >> 1], p.drop_thr);
          dS[v] = P[v] * fmaf(dP[v], keep ? p.drop_scale : 0.f, dlt_s[buf][ib + v]);
          P[v] = keep ? P[v] : 0.f;
        } else {
          dS[v] = P[v] * dP[v];
        }
      }
      float cs = 0.f;  // far tiles: this lane's part of the column sum (of the rounded dS the MFMA uses)
#pragma unroll
      for (int q = 0; q < 32 / KS; ++q) {
        // the step's dO and Q fragments first, so their reads share one wait
        frag fo[ND], fq[ND];
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) {
          fo[nd] = ld_col<TR>(dOs[buf], QP, 32 * u, 32 * nd, q);
          fq[nd] = ld_col<TR>(Qs[buf], QP, 32 * u, 32 * nd, q);
        }
        const frag pb = TR::pack(&P[q * E]);
        const frag sb = TR::pack(&dS[q * E]);
        if (!BAND) cs = TR::sum(sb, cs);
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) {
          dVt[nd] = TR::mma(fo[nd], pb, dVt[nd]);
          dKt[nd] = TR::mma(fq[nd], sb, dKt[nd]);
        }
      }
      if (!BAND) {
        // far tiles: one row, one sum per tile
        colsum += cs;
      } else {
        if constexpr (AWIN && MODE != 0) {
          // the next band tile's windows, after this tile's last transposing
          // reads and before its last walk stores (in the band loop the 16
          // stores that follow the copy let the tile's end wait for the
          // copies alone)
          if (u == NQT - 1 && next_band) issue_windows(buf ^ 1, i0 + BM);
          __builtin_amdgcn_sched_barrier(0);  // the walk stores stay after the copies
        }
        // dP2C: this half's queries of the subtile, in order (their rows
        // are read in one batch, so the walk waits on LDS once)
        int wr[16];
#pragma unroll
        for (int v = 0; v < 16; ++v)
          wr[v] = lut_p(lut_s[buf][half_major_partner<NQT>(u, g, v) - jl + BN - 1]) / (NARROW ? ES : 1);
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if constexpr (NARROW)
            walk_step_narrow<TR>(wview, wbase, wk, wr[v], dS[v], jin && i0 + half_major_partner<NQT>(u, g, v) < sq.len);
          else
            walk_step<TR, false>(wrow, R, wk, wr[v], dS[v], jin && i0 + half_major_partner<NQT>(u, g, v) < sq.len);
      }
    }
    if constexpr (AWIN) {
      if (next_band) {
        if constexpr (MODE == 0) {
          // a far tile reads no window: the hand-over waits until its
          // subtiles are done, so they stay one straight-line block
          if (tid < NL) lut_s[buf ^ 1][tid] = NARROW ? lreg * ES : lreg;
          __syncthreads();
          issue_windows(buf ^ 1, i0 + BM);
        } else if (!BAND) {
          issue_windows(buf ^ 1, i0 + BM);  // (band tiles issued it before their last walk)
        }
      }
    }
    if (!BAND) {
      colsum += xor32(colsum);  // the key's two lane halves
      if (jin && g == 0) {
        WalkHalf wf = walk_begin(0, rc, sc, -1);
        walk_step<TR, NARROW>(wrow, R, wf, left ? 0 : R - 1, colsum);
        rc = wf.r;
        sc = wf.s;
      }
    } else {
      walk_merge<TR>(wrow, R, g, wk, rc, sc, jin);
    }
    if (qb + 1 < nqb) commit(qb + 1);
    // this tile's copies (the next query tile, the next band tile's windows)
    // must land before the barrier publishes them. A tile of the band loop
    // issues 16 walk stores (one per step, always issued) after its last
    // copy, and a wave's vector memory operations complete in order, so it
    // need not wait for those stores
    if constexpr (AWIN && MODE == 1)
      wait_vmem_keep<16>();
    else
      wait_vmem();
    __syncthreads();
  };
  if constexpr (DROP) {
    // the dropout bodies need more registers: one loop, the class decided
    // per tile (with the ranges apart they spill)
    for (int qb = 0; qb < nqb; ++qb) iter(qb, IntC<2>{});
  } else {
    int qb = 0;
    for (; qb < qb_band; ++qb) iter(qb, IntC<0>{});
    for (; qb < qb_left; ++qb) iter(qb, IntC<1>{});
    for (; qb < nqb; ++qb) iter(qb, IntC<0>{});
  }

  // close this key's dP2C row, then add the relative term dP2C Q_r (the
  // wave's rows are complete once its own stores are)
  if (jin && g == 0) walk_finish<TR>(wrow, R, RP, rc, sc);
  wait_vmem();
  rel_epilogue<TR, ND>(dKt, wview, wbase, buf_view((const T*)p.qrT + int64_t(h) * D * RP, uint32_t(D * RP * ES)), RP);
  if (!jin) return;
  T* dvp = (T*)p.dv + tok_j * p.ts + int64_t(h) * p.hs;
  T* dkp = (T*)p.dk + tok_j * p.ts + int64_t(h) * p.hs;
#pragma unroll
  for (int nd = 0; nd < ND; ++nd)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int c = 32 * nd + acc_row(v, g);
      dvp[c] = TR::from_f(DROP ? dVt[nd][v] * p.drop_scale : dVt[nd][v]);
      dkp[c] = TR::from_f(dKt[nd][v] * p.scale);
    }
}

template <int DT, int D, bool NARROW>
void launch_d(const Params& p, hipStream_t st) {
  dim3 grid(unsigned((p.Lmax + 127) / 128 * p.H * p.nseq));
  constexpr int NQT = (DT == DF_FP32_T) ? 1 : 2;
  if (p.drop)
    dkv_kernel<DT, D, NQT, NARROW, true><<<grid, 256, 0, st>>>(p);
  else
    dkv_kernel<DT, D, NQT, NARROW, false><<<grid, 256, 0, st>>>(p);
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

hipError_t launch_bwd_dkv(const Params& p, hipStream_t st) {
  switch (p.dtype) {
    case DF_BF16_T: launch_dt<DF_BF16_T>(p, st); break;
    case DF_FP16_T: launch_dt<DF_FP16_T>(p, st); break;
    default: launch_dt<DF_FP32_T>(p, st); break;
  }
  return hipGetLastError();
}

}  // namespace dfa
