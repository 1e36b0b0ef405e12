// Backward, query side: dQ and the dense dC2P strip (DisentangledFlash 1.1.1
// page, "Hugging Face usage": an independently selected dQ kernel;
// "Performance": scores are recomputed in the backward).
//
// Work item: one sequence, one head, 128 queries (4 waves x 32 queries,
// resident in registers). The loop walks 32*NKT keys at a time; K, V and K^T
// are staged in LDS. Each wave computes S^T = K Q^T and dP^T = V dO^T, so lane
// l owns query l % 32; P and dS are lane-local per query and
//   dQ^T += K^T dS^T
//   dC2P[i, r] = sum_{j: delta(i,j) = r} dS[i, j]
// with the strip row of query i written by an ordered walk over the keys
// (one step per tile in the far field). dQ here is the dS K part only; the
// dC2P K_r term is added by the relative-gradient GEMM.
#include "tiles.hpp"
#include "walk.hpp"

namespace dfa {

namespace {

template <int DT, int D, int NKT>
__global__ __launch_bounds__(256) void dq_kernel(Params p) {
  using TR = Tr<DT>;
  using T = typename TR::T;
  using frag = typename TR::frag;
  constexpr int E = TR::E, KS = TR::KS, NQ = D / KS, ND = D / 32;
  constexpr int BM = 128, BN = 32 * NKT;
  constexpr int KP = Pitch<T, D>::rm, KTP = Pitch<T, BN>::tr;
  constexpr int NL = BM + BN - 1;

  __shared__ __align__(16) T Ks[BN * KP];
  __shared__ __align__(16) T Vs[BN * KP];
  __shared__ __align__(16) T Kt[D * KTP];
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
  const float lse2 = qvalid ? p.lse[int64_t(h) * T_ + tok_i] * kLog2e : 0.f;
  const float dlt = qvalid ? p.delta[int64_t(h) * T_ + tok_i] : 0.f;
  const T* ends = (const T*)p.ends;
  const float a_end0 = TR::to_f(ends[int64_t(h) * T_ + tok_i]);
  const float a_end1 = TR::to_f(ends[HT + int64_t(h) * T_ + tok_i]);
  const T* c2prow = (const T*)p.c2ps + (int64_t(h) * T_ + tok_i) * RP;
  const T* p2cbase = (const T*)p.p2cs + (int64_t(h) * T_ + sq.start) * RP;
  const T* kbase = (const T*)p.k + sq.start * p.ts + int64_t(h) * p.hs;
  const T* vbase = (const T*)p.v + sq.start * p.ts + int64_t(h) * p.hs;

  f32x16 dQt[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) dQt[nd] = zero16();
  StripWalk<TR> walk;
  walk.init((T*)p.dc2p + (int64_t(h) * T_ + tok_i) * RP, R, RP);
  const bool walker = qin && g == 0;

  const int nkb = (sq.len + BN - 1) / BN;
  for (int kb = 0; kb < nkb; ++kb) {
    const int j0 = kb * BN;
    __syncthreads();
    stage_rows_tr<T, D, BN, KP, KTP, 256>(Ks, Kt, kbase, p.ts, j0, sq.len);
    stage_rows<T, D, BN, KP, 256>(Vs, vbase, p.ts, j0, sq.len);

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

    float rowsum = 0.f;
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      f32x16 S = zero16(), dP = zero16();
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        S = TR::mma(TR::ld(&Ks[(32 * t + li) * KP + q * KS + g * E]), Qf[q], S);
        dP = TR::mma(TR::ld(&Vs[(32 * t + li) * KP + q * KS + g * E]), dOf[q], dP);
      }
      float dS[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int jl = 32 * t + acc_row(v, g);
        float x = S[v] * p.scale_log2;
        if (far) {
          x += a_far + bj_s[jl];
        } else {
          const int n = il - jl + BN - 1;
          const int jj = min(j0 + jl, sq.len - 1);
          x += TR::to_f(c2prow[lutc[n]]) + TR::to_f(p2cbase[int64_t(jj) * RP + lutp[n]]);
        }
        if (!all_keys) x += kb_s[jl];
        const float P = qvalid ? fast_exp2(x - lse2) : 0.f;
        dS[v] = P * (dP[v] - dlt);
      }
#pragma unroll
      for (int q = 0; q < 32 / KS; ++q) {
        const frag sb = TR::pack(&dS[q * E]);
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) {
          const T* kr = &Kt[(32 * nd + li) * KTP + 32 * t];
          frag a;
          if constexpr (E == 8)
            a = TR::ld2x4(kr + 16 * q + 4 * g, kr + 16 * q + 8 + 4 * g);
          else
            a = TR::ld(kr + fed_row<E>(q, 0, g));
          dQt[nd] = TR::mma(a, sb, dQt[nd]);
        }
      }
      // dC2P: ordered walk over this subtile's keys
      if (far) {
        float rs = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) rs += dS[v];
        rowsum += rs + xor32(rs);
      } else {
        float other[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) other[v] = xor32(dS[v]);
        if (walker) {
#pragma unroll
          for (int k = 0; k < 32; ++k) {
            const int jl = 32 * t + k;
            if (j0 + jl >= sq.len) break;
            const float val = walk_grp(k) == 0 ? dS[walk_reg(k)] : other[walk_reg(k)];
            walk.step(lutc[il - jl + BN - 1], val);
          }
        }
      }
    }
    if (far && walker) walk.step(clo, rowsum);
  }

  if (!qin) return;
  float* dqp = p.dq_acc + (int64_t(h) * T_ + tok_i) * D;
#pragma unroll
  for (int nd = 0; nd < ND; ++nd)
#pragma unroll
    for (int v = 0; v < 16; ++v) dqp[32 * nd + acc_row(v, g)] = dQt[nd][v] * p.scale;
  if (g == 0) walk.finish();
}

template <int DT, int D>
void launch_d(const Params& p, hipStream_t st) {
  dim3 grid(unsigned((p.Lmax + 127) / 128), unsigned(p.H), unsigned(p.nseq));
  constexpr int NKT = (DT == DF_FP32_T && D == 128) ? 1 : 2;
  dq_kernel<DT, D, NKT><<<grid, 256, 0, st>>>(p);
}

template <int DT>
void launch_dt(const Params& p, hipStream_t st) {
  switch (p.D) {
    case 32: launch_d<DT, 32>(p, st); break;
    case 64: launch_d<DT, 64>(p, st); break;
    default: launch_d<DT, 128>(p, st); break;
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
