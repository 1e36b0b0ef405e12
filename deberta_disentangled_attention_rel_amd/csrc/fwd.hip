// Fused forward: output and log-sum-exp of disentangled attention without
// the L x L matrix (DisentangledFlash 1.1.1 page, "Status" and "Hugging Face
// usage": the LSE-producing training forward).
//
// Work item: one sequence, one head, 128 query rows (4 waves x 32). The key
// loop walks BN = 32*NKT keys at a time. Each wave computes S^T = K Q^T with
// 32x32 MFMAs, so lane l owns query row l % 32 and holds 16 of every 32 keys
// (the other 16 sit in lane l ^ 32). Row max and row sum are lane-local plus
// one exchange; the output is accumulated transposed, O^T = V^T P^T, so the
// rescale is lane-local and P feeds the MFMA straight from registers.
//
// Scores are in the log2 domain: y = s*log2(e)*QK + (relative terms). The
// key tiles of a query block fall into three contiguous ranges: far-left
// tiles (every pair beyond +span: one C2P value per query, one P2C value per
// key), band tiles, and far-right tiles (every pair beyond -span). In a far
// tile the per-key P2C value is added in the same FMA as the scale and the
// per-query C2P value a is folded into the row max (exp2(y - (m - a))). A
// band tile gathers each query's C2P terms from an LDS window of its strip
// row (the lanes read different rows) and the P2C terms straight from the
// strip, which stays in L2 (for a fixed key the 32 lanes of a half read one
// contiguous run of its row); when the tables can skip rows, both terms come
// from global memory.
//
// Far ranges run a software pipeline in which the matrix and vector units of
// one wave work at the same time. Iteration kb holds the scores of tile kb
// (computed in the previous iteration) and runs two straight-line stages,
// their instructions interleaved explicitly (scheduling group barriers):
//   A: the softmax of tile kb (exp2, packing, row sum)  alongside  the
//      S MFMAs of tile kb+1;
//   B: the P V MFMAs of tile kb  alongside  the scale FMAs and the row max
//      of tile kb+1.
// K rows and per-key values are therefore loaded two tiles ahead and V one
// tile ahead, each into the buffer that the tile two (one) back freed, so two
// buffers of each suffice and one barrier per tile publishes them. The band
// range keeps a plain loop (loads one tile ahead, a straight-line band
// tile body), so the gathered relative terms, windows and table slices never
// raise the register pressure of the far pipeline. Each range drains its
// loads before the next one starts.
#include "band.hpp"
#include "pipe.hpp"

namespace dfa {

namespace {

constexpr float kMaxSlack = 8.f;

// Scheduling-group masks (AMDGPU sched_group_barrier).
constexpr int kSgMfma = 0x008, kSgValu = 0x002, kSgDsRead = 0x100;

// Dropout of one 32-key subtile of P (lane = query i; register 4b + e holds
// key jt + 8b + 4g + e, so block b of the subtile's four 8-key blocks has its
// keys 0..3 in lane group 0 and 4..7 in lane group 1). Lane group g computes
// the calls of blocks 2g and 2g + 1; v_permlane32_swap (lanes 32..63 of the
// first operand with lanes 0..31 of the second) swaps words 0, 1 of one
// group's calls with words 2, 3 of the other's, which leaves each lane the two
// words of its four keys in every block. Dropped values become 0.
__device__ __forceinline__ void drop_subtile(float (&y)[16], int jt, int g, uint32_t i, uint32_t stream,
                                             const Params& p) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const Philox4 r = philox4x32_10(uint32_t(jt >> 3) + uint32_t(2 * g + c), i, stream, p.drop_off, p.seed_lo,
                                    p.seed_hi);
    const auto s0 = __builtin_amdgcn_permlane32_swap(r.w[0], r.w[2], false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(r.w[1], r.w[3], false, false);
    // s*[0]: block c, s*[1]: block 2 + c
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int b = 4 * (c + 2 * h);
      y[b] = keep_lo(s0[h], p.drop_thr) ? y[b] : 0.f;
      y[b + 1] = keep_hi(s0[h], p.drop_thr) ? y[b + 1] : 0.f;
      y[b + 2] = keep_lo(s1[h], p.drop_thr) ? y[b + 2] : 0.f;
      y[b + 3] = keep_hi(s1[h], p.drop_thr) ? y[b + 3] : 0.f;
    }
  }
}

template <int DT, int D, int NKT, bool NARROW, bool DROP>
__global__ __launch_bounds__(256, (DT != DF_FP32_T && (D <= 64 || NKT == 1)) ? 2 : 1) void fwd_kernel(Params p) {
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
  // names its buffer at compile time (the loops are unrolled by two): reads
  // of one buffer then provably do not alias the copy into the other, so the
  // compiler does not make them wait for that copy
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
  const int nkb = (sq.len + BN - 1) / BN;

  auto cls_of = [&](int kb) {
    const int j0 = kb * BN;
    return tile_class(i0 - j0 - BN + 1, i0 + BM - 1 - j0, d_hi, d_lo);
  };
  // the three ranges: tile kb is far-left iff i0 - kb*BN - BN + 1 >= d_hi,
  // far-right iff i0 + BM - 1 - kb*BN <= d_lo
  const int nl = i0 - BN + 1 - d_hi;
  const int kb_band = min(nkb, nl >= 0 ? nl / BN + 1 : 0);
  const int kb_right = max(kb_band, min(nkb, (i0 + BM - 1 - d_lo + BN - 1) / BN));

  // buffer views of this sequence's rows (reads past its end return zero)
  // and this thread's fixed offsets into them: issuing a tile's loads then
  // needs no address arithmetic
  const uint32_t seq_bytes = uint32_t(sq.len) * uint32_t(p.ts * ES);
  const BufView kview = buf_view(kbase, seq_bytes), vview = buf_view(vbase, seq_bytes);
  [[maybe_unused]] DmaRows<T, BN, D, KP, 256> kdma;
  [[maybe_unused]] DmaRows<T, BN, D, VP, 256, false, true> vdma;  // rows interleaved for the transposing reads
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

  // Register staging (fp32 K/V tiles; per-key values and table slice of
  // every type) is loaded raw and committed to LDS at the end of an
  // iteration, so nothing waits for it before then; key mask and end values
  // past the sequence read 0 (the key is masked there anyway).
  KTile kt, vt;
  kt.init();
  vt.init();
  T e_raw = TR::from_f(0.f);
  uint32_t m_raw = 1u, l_raw = 0u;

  f32x16 O[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) O[nd] = zero16();
  float m = -INFINITY, l = 0.f;
  const float inv_sl = 1.f / p.scale_log2;

  auto load_k = [&](int n, auto kb_c) {
    constexpr int KB = decltype(kb_c)::value;
    if constexpr (DMA)
      kdma.issue(KB ? Ks1 : Ks0, kview, n * BN * int(p.ts) * ES);
    else
      kt.load(kbase, p.ts, n * BN, sq.len);
  };
  auto load_v = [&](int n, auto vb_c) {
    constexpr int VB = decltype(vb_c)::value;
    if constexpr (DMA)
      vdma.issue(VB ? Vs1 : Vs0, vview, n * BN * int(p.ts) * ES);
    else
      vt.load(vbase, p.ts, n * BN, sq.len);
  };
  auto commit_k = [&](auto kb_c) {
    constexpr int KB = decltype(kb_c)::value;
    if constexpr (!DMA) kt.template store<KP>(KB ? Ks1 : Ks0);
  };
  auto commit_v = [&](auto vb_c) {
    constexpr int VB = decltype(vb_c)::value;
    if constexpr (!DMA) vt.template store<VP>(VB ? Vs1 : Vs0);
  };
  // per-key values of tile n (raw), and their commit: the far value of the
  // tile's class, 0 in band tiles, -inf for masked or absent keys
  auto load_keyvals = [&](int n, int cls) {
    if (tid < BN) {
      if (kmask) m_raw = buf_load_u8(mview, n * BN + tid);
      e_raw = buf_load<T>(cls == TILE_FAR_LEFT ? eview_l : eview_r, tid * ES, n * BN * ES);
    }
  };
  // (far ranges store the value divided by s log2 e: it seeds the score
  // accumulator)
  auto commit_keyvals = [&](int n, int cls, auto kb_c, bool unscaled = false) {
    constexpr int KB = decltype(kb_c)::value;
    if (tid < BN) {
      const bool ok = n * BN + tid < sq.len && m_raw != 0u;
      const float b = cls != TILE_BAND ? TR::to_f(e_raw) : 0.f;
      bj_s[KB][tid] = ok ? (unscaled ? b * inv_sl : b) : -INFINITY;
    }
  };

  // =========================================================================
  // Far range [kb0, kb1) of class CLS: the software pipeline.
  auto far_range = [&](int kb0, int kb1, auto cls_c) {
    constexpr int CLS = decltype(cls_c)::value;
    const float a = CLS == TILE_FAR_LEFT ? a_end1 : a_end0;  // per-query C2P value
    // y: raw scores QK + b/(s log2 e) of the current tile (the per-key P2C
    // term rides in the accumulator: the MFMAs start from it), so the
    // log2-domain score is y * s log2 e
    float y[NKT][16];
    float mt;
    // S^T of the tile in buffer KB on top of its per-key terms
    auto score_mma = [&](auto kb_c, f32x16 (&acc)[NKT]) {
      constexpr int KB = decltype(kb_c)::value;
      const T* const Kc = KB ? Ks1 : Ks0;
#pragma unroll
      for (int t = 0; t < NKT; ++t) {
        acc[t] = bias16(&bj_s[KB][32 * t], g);
#pragma unroll
        for (int q = 0; q < NQ; ++q) acc[t] = TR::mma(ld_row<TR>(Kc, KP, 32 * t + li, q * KS + g * E), Qf[q], acc[t]);
      }
    };
    // the tile's row max (log2 domain, + a)
    auto finish = [&](auto, const f32x16 (&acc)[NKT]) {
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < NKT; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          y[t][v] = acc[t][v];
          mx = fmaxf(mx, y[t][v]);
        }
      mt = fmaf(fmaxf(mx, xor32(mx)), p.scale_log2, a);
    };

    // prologue: K and per-key values of the first two tiles, V of the first;
    // then the scores of the first tile
    auto prologue = [&](auto p_c) {
      constexpr int P = decltype(p_c)::value;
      load_k(kb0, IntC<P>{});
      load_keyvals(kb0, CLS);
      load_v(kb0, IntC<P>{});
      commit_k(IntC<P>{});
      commit_v(IntC<P>{});
      commit_keyvals(kb0, CLS, IntC<P>{}, true);
      if (kb0 + 1 < kb1) {
        load_k(kb0 + 1, IntC<P ^ 1>{});
        load_keyvals(kb0 + 1, CLS);
        commit_k(IntC<P ^ 1>{});
        commit_keyvals(kb0 + 1, CLS, IntC<P ^ 1>{}, true);
      }
      wait_vmem();
      __syncthreads();
      f32x16 acc[NKT];
      score_mma(IntC<P>{}, acc);
      finish(IntC<P>{}, acc);
    };
    if (kb0 & 1)
      prologue(IntC<1>{});
    else
      prologue(IntC<0>{});

    // iteration kb, P = kb & 1: K[P^1] and the per-key values [P^1] hold tile
    // kb+1, V[P] tile kb; the loads go to K[P] (tile kb+2) and V[P^1] (tile
    // kb+1), which the previous iteration freed
    auto iter = [&](int kb, auto p_c) __attribute__((always_inline)) {
      constexpr int P = decltype(p_c)::value;
      const int j0 = kb * BN;
      const bool has1 = kb + 1 < kb1, has2 = kb + 2 < kb1;
      if (has2) {
        load_keyvals(kb + 2, CLS);
        load_k(kb + 2, IntC<P>{});
      }
      if (has1) load_v(kb + 1, IntC<P ^ 1>{});

      // online softmax of tile kb. The running max moves only when the
      // tile's max exceeds it by more than kMaxSlack (log2 units): otherwise
      // the probabilities are taken against the old max (at most
      // 2^kMaxSlack, exact in fp32 sums and at full relative precision in
      // the 16-bit P operand) and O needs no rescale; O / l and the LSE are
      // the same either way
      const float mnew = mt > m + kMaxSlack ? mt : m;
      const float msafe = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = fast_exp2(m - msafe);
      const float shift = msafe - a;
      m = mnew;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int nd = 0; nd < ND; ++nd)
#pragma unroll
          for (int v = 0; v < 16; ++v) O[nd][v] *= alpha;
      }

      // stage A: P of tile kb (exp2, dropout, packing, row sum) alongside
      // the S MFMAs of tile kb+1 (on the last tile they read a stale buffer
      // and are discarded)
      frag pf[NKT][32 / KS];
      float ls = 0.f;
      f32x16 acc[NKT];
#pragma unroll
      for (int t = 0; t < NKT; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) y[t][v] = fast_exp2(fmaf(y[t][v], p.scale_log2, -shift));
      if constexpr (DROP) {
        // the row sum is of the undropped P; P V takes the dropped P (kept
        // or zero, unscaled: 1 / (1 - p) multiplies O once at the end)
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
          for (int q = 0; q < 32 / KS; ++q) ls = TR::sum(TR::pack(&y[t][q * E]), ls);
#pragma unroll
        for (int t = 0; t < NKT; ++t) drop_subtile(y[t], j0 + 32 * t, g, uint32_t(iw), uint32_t(blk.z * p.H + h), p);
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
          for (int q = 0; q < 32 / KS; ++q) pf[t][q] = TR::pack(&y[t][q * E]);
      } else {
        // the row sum adds the same rounded P the MFMA uses
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
          for (int q = 0; q < 32 / KS; ++q) {
            pf[t][q] = TR::pack(&y[t][q * E]);
            ls = TR::sum(pf[t][q], ls);
          }
      }
      score_mma(IntC<P ^ 1>{}, acc);
      if constexpr (ES == 2 && !DROP) {
        // one MFMA, ~12 vector instructions and the fragment read of the
        // MFMA after next at a time
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
#pragma unroll
        for (int k = 0; k < NKT * NQ; ++k) {
          __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSgValu, 12, 0);
          __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
        }
      }
      l = l * alpha + ls;

      // stage B: O^T += V^T P^T for tile kb alongside the scores of tile kb+1
      const T* const Vc = P ? Vs1 : Vs0;
#pragma unroll
      for (int t = 0; t < NKT; ++t)
#pragma unroll
        for (int q = 0; q < 32 / KS; ++q)
#pragma unroll
          for (int nd = 0; nd < ND; ++nd) O[nd] = TR::mma(ld_col<TR, DMA>(Vc, VP, 32 * t, 32 * nd, q), pf[t][q], O[nd]);
      finish(IntC<P ^ 1>{}, acc);
      if constexpr (ES == 2) {
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 6, 0);
#pragma unroll
        for (int k = 0; k < NKT * (32 / KS) * ND; ++k) {
          __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSgValu, 3, 0);
          __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
        }
      }

      if (has2) {
        commit_k(IntC<P>{});
        commit_keyvals(kb + 2, CLS, IntC<P>{}, true);
      }
      if (has1) commit_v(IntC<P ^ 1>{});
      wait_vmem();
      __syncthreads();
    };
    int kb = kb0;
    if (kb < kb1 && (kb & 1)) {
      iter(kb, IntC<1>{});
      ++kb;
    }
    for (; kb < kb1; kb += 2) {
      iter(kb, IntC<0>{});
      if (kb + 1 < kb1) iter(kb + 1, IntC<1>{});
    }
  };

  // =========================================================================
  // Band range [kb0, kb1) (every tile of it a band tile): loads one tile
  // ahead, the tile body straight-line code.
  auto band_range = [&](int kb0, int kb1) {
    auto prefetch = [&](int kb, auto q_c) {
      constexpr int Q = decltype(q_c)::value;
      const int cls = cls_of(kb);
      load_keyvals(kb, cls);
      if (tid < NL) l_raw = buf_load<uint32_t>(lview, lvoff - kb * BN * 4, 0);
      load_k(kb, IntC<Q>{});
      load_v(kb, IntC<Q>{});
    };
    auto commit = [&](int kb, auto q_c) {
      constexpr int Q = decltype(q_c)::value;
      commit_k(IntC<Q>{});
      commit_v(IntC<Q>{});
      commit_keyvals(kb, cls_of(kb), IntC<Q>{});
      // both 16-bit halves scale to byte offsets at once (narrow: (R-1)*ES fits 16 bits)
      if (tid < NL) lut_s[Q][tid] = NARROW ? l_raw * ES : l_raw;
    };

    [[maybe_unused]] Win win;
    auto start = [&](auto p_c) {
      constexpr int P = decltype(p_c)::value;
      if constexpr (AWIN) {
        // window of the first tile now, row starts of the second for the
        // first iteration
        win.load_starts(p, i0 - kb0 * BN - BN + 1);
        win.issue(P ? Wc1 : Wc0, c2pstrip, RP, i0, sq.len);
        if (kb0 + 1 < kb1) win.load_starts(p, i0 - (kb0 + 1) * BN - BN + 1);
      }
      prefetch(kb0, IntC<P>{});
      commit(kb0, IntC<P>{});
      wait_vmem();
      __syncthreads();
    };
    if (kb0 & 1)
      start(IntC<1>{});
    else
      start(IntC<0>{});

    // one tile; P = kb & 1 is the buffer it reads
    auto iter = [&](int kb, auto p_c) __attribute__((always_inline)) {
      constexpr int P = decltype(p_c)::value;
      constexpr int buf = P;
      const T* const Kc = P ? Ks1 : Ks0;
      const T* const Vc = P ? Vs1 : Vs0;
      const int j0 = kb * BN;
      const int cls = cls_of(kb);
      // with dropout, this tile's P2C terms are loaded first, before the
      // next tiles' copies: a wave's vector memory operations complete in
      // order, so their first use then waits for them alone (dropout step
      // 5.42 -> 4.99 ms); without dropout that order is slightly slower
      // (0.651 -> 0.663 ms), and the loads stay next to their use
      constexpr bool EARLY_P2C = NARROW && DROP;
      [[maybe_unused]] T p2c_raw[NKT][16];
      if constexpr (EARLY_P2C) {
        const uint32_t* lrow = &lut_s[buf][il + BN - 1];  // entry of key jl: lrow[-jl]
        const BufView prow = buf_view(p2cstrip, uint32_t(sq.len) * uint32_t(RP * ES));
        const int soff = j0 * RP * ES;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int jl = 32 * t + acc_row(v, g);
            p2c_raw[t][v] = buf_load<T>(prow, jl * RP * ES + lut_p(lrow[-jl]), soff);
          }
      }
      // loads for the next tiles: the next band tile's window into the
      // other buffer (free since the last barrier), the row starts of the
      // band tile after it, the next K/V tile
      if constexpr (AWIN) {
        if (kb + 1 < kb1) win.issue(P ? Wc0 : Wc1, c2pstrip, RP, i0, sq.len);
        if (kb + 2 < kb1) win.load_starts(p, i0 - (kb + 2) * BN - BN + 1);
      }
      if (kb + 1 < kb1) prefetch(kb + 1, IntC<P ^ 1>{});

      // the score part of the tile body (relative terms, S MFMAs, softmax)
      // as straight-line code; it leaves the packed probabilities, their row
      // sum and the rescale factor
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

        // relative terms (log2 domain) of this lane's 16*NKT keys, gathered
        // before the score MFMAs so the gather latency overlaps them
        float rel[NKT][16];
        if constexpr (BAND) {
          const uint32_t* lrow = &lut_s[buf][il + BN - 1];  // entry of key jl: lrow[-jl]
          if constexpr (NARROW) {
            // C2P from this row's LDS window; P2C straight from the strip in
            // L2 (keys past the sequence end read zero)
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
                T pv;
                if constexpr (EARLY_P2C)
                  pv = p2c_raw[t][v];
                else
                  pv = buf_load<T>(prow, jl * RP * ES + lut_p(e), soff);
                rel[t][v] = TR::add2(*reinterpret_cast<const T*>(wc + lut_c(e)), pv, bj_s[buf][jl]);
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
        // online softmax with the same lazy running max as the far ranges
        float mt = -INFINITY;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
          for (int v = 0; v < 16; ++v) mt = fmaxf(mt, y[t][v]);
        mt = fmaxf(mt, xor32(mt)) + a;
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
          // P V takes the dropped P (kept or zero, unscaled)
#pragma unroll
          for (int t = 0; t < NKT; ++t)
            drop_subtile(y[t], j0 + 32 * t, g, uint32_t(iw), uint32_t(blk.z * p.H + h), p);
#pragma unroll
          for (int t = 0; t < NKT; ++t)
#pragma unroll
            for (int q = 0; q < 32 / KS; ++q) pf[t][q] = TR::pack(&y[t][q * E]);
        }
      };
      body(BoolC<true>{});

      // O^T += V^T P^T after the lazy rescale (same code for both classes,
      // so the accumulators are updated in place)
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
          for (int nd = 0; nd < ND; ++nd) O[nd] = TR::mma(ld_col<TR, DMA>(Vc, VP, 32 * t, 32 * nd, q), pf[t][q], O[nd]);
      l = l * alpha + ls;

      if (kb + 1 < kb1) commit(kb + 1, IntC<P ^ 1>{});
      wait_vmem();
      __syncthreads();
    };
    int kb = kb0;
    if (kb < kb1 && (kb & 1)) {
      iter(kb, IntC<1>{});
      ++kb;
    }
    for (; kb < kb1; kb += 2) {
      iter(kb, IntC<0>{});
      if (kb + 1 < kb1) iter(kb + 1, IntC<1>{});
    }
  };

  if (kb_band > 0) far_range(0, kb_band, IntC<TILE_FAR_LEFT>{});
  if (kb_right > kb_band) band_range(kb_band, kb_right);
  if (nkb > kb_right) far_range(kb_right, nkb, IntC<TILE_FAR_RIGHT>{});

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
  // D=128: 32-key tiles, which fit two work-groups per CU (two waves per
  // SIMD) in registers and LDS; a 64-key tile needs one per CU
  constexpr int NKT = D == 128 ? 1 : 2;
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
