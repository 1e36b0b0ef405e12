// Fused forward: output and log-sum-exp of disentangled attention without
// the L x L matrix (DisentangledFlash 1.1.1 page, "Status" and "Hugging Face
// usage": the LSE-producing training forward).
//
// Work item: one sequence, one head, 128 query rows (4 waves x 32). The key
// loop walks 32*NKT keys at a time; K and V^T tiles are staged in LDS.
//
// Layout: each wave computes S^T = K Q^T with 32x32 MFMAs, so lane l owns
// query row l % 32 and holds 16 of every 32 keys; the other 16 sit in lane
// l ^ 32. Row max and row sum are lane-local plus one exchange. The output is
// accumulated transposed, O^T = V^T P^T, so the per-row rescale is lane-local
// too and P feeds the MFMA straight from the score registers.
//
// Scores are formed in the log2 domain: x = s*log2(e)*QK + C2P + P2C with the
// strips pre-scaled. A tile whose pairs all sit in the saturated far field
// (both index tables constant and at an end row) adds a per-row C2P value and
// a per-key P2C value; any other tile gathers both terms per pair through the
// index tables staged in LDS.
#include "tiles.hpp"

namespace dfa {

namespace {

template <int DT, int D, int NKT>
__global__ __launch_bounds__(256) void fwd_kernel(Params p) {
  using TR = Tr<DT>;
  using T = typename TR::T;
  using frag = typename TR::frag;
  constexpr int E = TR::E, KS = TR::KS, NQ = D / KS, ND = D / 32;
  constexpr int BM = 128, BN = 32 * NKT;
  constexpr int KP = Pitch<T, D>::rm, VP = Pitch<T, BN>::tr;
  constexpr int NL = BM + BN - 1;

  __shared__ __align__(16) T Ks[BN * KP];
  __shared__ __align__(16) T Vt[D * VP];
  __shared__ int lutc[NL], lutp[NL];
  __shared__ __align__(16) float bj_s[BN];
  __shared__ __align__(16) float kb_s[BN];

  const int lane = threadIdx.x & 63, g = lane >> 5, li = lane & 31, wave = threadIdx.x >> 6;
  const SeqRange sq = seq_range(p.cu, blockIdx.z, p.Lmax);
  const int h = blockIdx.y;
  const int i0 = blockIdx.x * BM;
  if (i0 >= sq.len) return;
  const int64_t T_ = p.T, HT = int64_t(p.H) * p.T;
  const int R = p.R, RP = p.RP, off = p.Lmax - 1;

  const int iw = i0 + wave * 32 + li;  // this lane's query (local index)
  const bool qin = iw < sq.len;
  const int64_t tok_i = sq.start + (qin ? iw : sq.len - 1);
  const bool qvalid = qin && (!p.kmask || p.kmask[tok_i]);

  frag Qf[NQ];
  {
    const T* qp = (const T*)p.q + tok_i * p.ts + int64_t(h) * p.hs;
#pragma unroll
    for (int q = 0; q < NQ; ++q) Qf[q] = TR::ld(qp + q * KS + g * E);
  }
  const T* ends = (const T*)p.ends;
  const float a_end0 = TR::to_f(ends[int64_t(h) * T_ + tok_i]);
  const float a_end1 = TR::to_f(ends[HT + int64_t(h) * T_ + tok_i]);
  const T* c2prow = (const T*)p.c2ps + (int64_t(h) * T_ + tok_i) * RP;
  const T* p2cbase = (const T*)p.p2cs + (int64_t(h) * T_ + sq.start) * RP;
  const T* kbase = (const T*)p.k + sq.start * p.ts + int64_t(h) * p.hs;
  const T* vbase = (const T*)p.v + sq.start * p.ts + int64_t(h) * p.hs;

  f32x16 O[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) O[nd] = zero16();
  float m = -INFINITY, l = 0.f;

  const int nkb = (sq.len + BN - 1) / BN;
  for (int kb = 0; kb < nkb; ++kb) {
    const int j0 = kb * BN;
    __syncthreads();
    stage_rows<T, D, BN, KP, 256>(Ks, kbase, p.ts, j0, sq.len);
    stage_rows_tr<T, D, BN, KP, VP, 256>(nullptr, Vt, vbase, p.ts, j0, sq.len);

    // tile class (uniform): are both tables constant at an end row?
    const int dlo = i0 - (j0 + BN - 1), dhi = i0 + BM - 1 - j0;
    auto cl = [&](int d) { return d < -off ? 0 : (d > off ? 2 * off : d + off); };
    const int clo = p.c2p[cl(dlo)], chi = p.c2p[cl(dhi)];
    const int plo = p.p2c[cl(dlo)], phi = p.p2c[cl(dhi)];
    const bool far = clo == chi && plo == phi && (clo == 0 || clo == R - 1) && (plo == 0 || plo == R - 1);

    bool kv_ok = true;
    if (threadIdx.x < BN) {
      const int j = j0 + threadIdx.x;
      const bool in = j < sq.len;
      const int64_t tj = sq.start + (in ? j : sq.len - 1);
      const bool ok = in && (!p.kmask || p.kmask[tj]);
      kb_s[threadIdx.x] = ok ? 0.f : -INFINITY;
      kv_ok = ok;
      if (far) bj_s[threadIdx.x] = TR::to_f(ends[(plo == 0 ? 2 : 3) * HT + int64_t(h) * T_ + tj]);
    }
    if (!far) {
      for (int n = threadIdx.x; n < NL; n += 256) {
        lutc[n] = p.c2p[cl(dlo + n)];
        lutp[n] = p.p2c[cl(dlo + n)];
      }
    }
    const bool all_keys = __syncthreads_and(kv_ok);
    const float a_far = clo == 0 ? a_end0 : a_end1;

    float x[NKT][16];
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      f32x16 acc = zero16();
#pragma unroll
      for (int q = 0; q < NQ; ++q) acc = TR::mma(TR::ld(&Ks[(32 * t + li) * KP + q * KS + g * E]), Qf[q], acc);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int jl = 32 * t + acc_row(v, g);
        float val = acc[v] * p.scale_log2;
        if (far) {
          val += a_far + bj_s[jl];
        } else {
          const int n = (iw - i0) - jl + BN - 1;
          const int jj = min(j0 + jl, sq.len - 1);
          val += TR::to_f(c2prow[lutc[n]]) + TR::to_f(p2cbase[int64_t(jj) * RP + lutp[n]]);
        }
        if (!all_keys) val += kb_s[jl];
        x[t][v] = val;
      }
    }
    // online softmax (log2 domain)
    float mt = -INFINITY;
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) mt = fmaxf(mt, x[t][v]);
    mt = fmaxf(mt, xor32(mt));
    const float mnew = fmaxf(m, mt);
    const float msafe = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = fast_exp2(m - msafe);
    float ls = 0.f;
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        x[t][v] = fast_exp2(x[t][v] - msafe);
        ls += x[t][v];
      }
    l = l * alpha + ls;
    m = mnew;
#pragma unroll
    for (int nd = 0; nd < ND; ++nd)
#pragma unroll
      for (int v = 0; v < 16; ++v) O[nd][v] *= alpha;
    // O^T += V^T P^T
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int q = 0; q < 32 / KS; ++q) {
        const frag pb = TR::pack(&x[t][q * E]);
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) {
          const T* vr = &Vt[(32 * nd + li) * VP + 32 * t];
          frag va;
          if constexpr (E == 8)
            va = TR::ld2x4(vr + 16 * q + 4 * g, vr + 16 * q + 8 + 4 * g);
          else
            va = TR::ld(vr + fed_row<E>(q, 0, g));
          O[nd] = TR::mma(va, pb, O[nd]);
        }
      }
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

template <int DT, int D>
void launch_fwd_d(const Params& p, hipStream_t st) {
  dim3 grid(unsigned((p.Lmax + 127) / 128), unsigned(p.H), unsigned(p.nseq));
  constexpr int NKT = (DT == DF_FP32_T && D == 128) ? 1 : 2;
  fwd_kernel<DT, D, NKT><<<grid, 256, 0, st>>>(p);
}

template <int DT>
void launch_fwd_dt(const Params& p, hipStream_t st) {
  switch (p.D) {
    case 32: launch_fwd_d<DT, 32>(p, st); break;
    case 64: launch_fwd_d<DT, 64>(p, st); break;
    default: launch_fwd_d<DT, 128>(p, st); break;
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
