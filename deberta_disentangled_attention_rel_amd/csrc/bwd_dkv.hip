// Backward, key side: dK, dV and the dense dP2C strip (DisentangledFlash
// 1.1.1 page, "Hugging Face usage": an independently selected dK/dV kernel;
// "Performance": the backward recomputes the score products). Determinism
// follows the FastFlashAttention page ("Determinism"): every output element is
// written once, by its owner, with no atomics.
//
// Work item: one sequence, one head, 128 keys (4 waves x 32 keys, resident
// in registers). The loop walks 32*NQT queries at a time; Q, dO and their
// transposes are staged in LDS. Each wave computes S = Q K^T and
// dP = dO V^T with 32x32 MFMAs, so lane l owns key l % 32 and holds 16 of
// every 32 queries. P = exp2(x - LSE*log2 e) is recomputed from the saved LSE,
// dS = P (dP - Delta), and
//   dV^T += dO^T P,   dK^T += Q^T dS       (accumulators lane-local per key)
//   dP2C[j, r] = sum_{i: delta(j,i) = r} dS[i, j]
// The strip row of key j is owned by its lane and written by an ordered walk
// over the queries; in far-field tiles (both index tables constant) the walk
// takes the tile's column sum in one step. dK here is the dS^T Q part only;
// the dP2C Q_r term is added by the relative-gradient GEMM.
#include "tiles.hpp"
#include "walk.hpp"

namespace dfa {

namespace {

template <int DT, int D, int NQT>
__global__ __launch_bounds__(256) void dkv_kernel(Params p) {
  using TR = Tr<DT>;
  using T = typename TR::T;
  using frag = typename TR::frag;
  constexpr int E = TR::E, KS = TR::KS, NQ = D / KS, ND = D / 32;
  constexpr int BN = 128, BM = 32 * NQT;
  constexpr int QP = Pitch<T, D>::rm, QTP = Pitch<T, BM>::tr;
  constexpr int NL = BM + BN - 1;

  __shared__ __align__(16) T Qs[BM * QP];
  __shared__ __align__(16) T dOs[BM * QP];
  __shared__ __align__(16) T Qt[D * QTP];
  __shared__ __align__(16) T dOt[D * QTP];
  __shared__ int lutc[NL], lutp[NL];
  __shared__ __align__(16) float lse_s[BM];
  __shared__ __align__(16) float dlt_s[BM];
  __shared__ __align__(16) float aq_s[BM];
  __shared__ __align__(16) float qok_s[BM];

  const int lane = threadIdx.x & 63, g = lane >> 5, li = lane & 31, wave = threadIdx.x >> 6;
  const SeqRange sq = seq_range(p.cu, blockIdx.z, p.Lmax);
  const int h = blockIdx.y;
  const int j0 = blockIdx.x * BN;
  if (j0 >= sq.len) return;
  const int64_t T_ = p.T, HT = int64_t(p.H) * p.T;
  const int R = p.R, RP = p.RP, off = p.Lmax - 1;

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
  const T* ends = (const T*)p.ends;
  const float b_end0 = TR::to_f(ends[2 * HT + int64_t(h) * T_ + tok_j]);
  const float b_end1 = TR::to_f(ends[3 * HT + int64_t(h) * T_ + tok_j]);
  const T* p2crow = (const T*)p.p2cs + (int64_t(h) * T_ + tok_j) * RP;
  const T* c2pbase = (const T*)p.c2ps + (int64_t(h) * T_ + sq.start) * RP;
  const T* qbase = (const T*)p.q + sq.start * p.ts + int64_t(h) * p.hs;
  const T* dobase = (const T*)p.dout + sq.start * p.ts + int64_t(h) * p.hs;
  const float* lse = p.lse + int64_t(h) * T_ + sq.start;
  const float* dlt = p.delta + int64_t(h) * T_ + sq.start;

  f32x16 dVt[ND], dKt[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) {
    dVt[nd] = zero16();
    dKt[nd] = zero16();
  }
  StripWalk<TR> walk;
  walk.init((T*)p.dp2c + (int64_t(h) * T_ + tok_j) * RP, R, RP);
  const bool walker = jin && g == 0;

  const int nqb = (sq.len + BM - 1) / BM;
  for (int qb = 0; qb < nqb; ++qb) {
    const int i0 = qb * BM;
    __syncthreads();
    stage_rows_tr<T, D, BM, QP, QTP, 256>(Qs, Qt, qbase, p.ts, i0, sq.len);
    stage_rows_tr<T, D, BM, QP, QTP, 256>(dOs, dOt, dobase, p.ts, i0, sq.len);

    const int dlo = i0 - (j0 + BN - 1), dhi = i0 + BM - 1 - j0;
    auto cl = [&](int d) { return d < -off ? 0 : (d > off ? 2 * off : d + off); };
    const int clo = p.c2p[cl(dlo)], chi = p.c2p[cl(dhi)];
    const int plo = p.p2c[cl(dlo)], phi = p.p2c[cl(dhi)];
    const bool far = clo == chi && plo == phi && (clo == 0 || clo == R - 1) && (plo == 0 || plo == R - 1);

    if (threadIdx.x < BM) {
      const int i = i0 + threadIdx.x;
      const bool in = i < sq.len;
      const int ic = in ? i : sq.len - 1;
      const bool ok = in && (!p.kmask || p.kmask[sq.start + ic]);
      qok_s[threadIdx.x] = ok ? 1.f : 0.f;
      lse_s[threadIdx.x] = ok ? lse[ic] * kLog2e : 0.f;
      dlt_s[threadIdx.x] = ok ? dlt[ic] : 0.f;
      if (far) aq_s[threadIdx.x] = TR::to_f(ends[(clo == 0 ? 0 : 1) * HT + int64_t(h) * T_ + sq.start + ic]);
    }
    if (!far) {
      for (int n = threadIdx.x; n < NL; n += 256) {
        lutc[n] = p.c2p[cl(dlo + n)];
        lutp[n] = p.p2c[cl(dlo + n)];
      }
    }
    __syncthreads();
    const float b_far = plo == 0 ? b_end0 : b_end1;

    float colsum = 0.f;
#pragma unroll
    for (int u = 0; u < NQT; ++u) {
      f32x16 S = zero16(), dP = zero16();
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        S = TR::mma(TR::ld(&Qs[(32 * u + li) * QP + q * KS + g * E]), Kf[q], S);
        dP = TR::mma(TR::ld(&dOs[(32 * u + li) * QP + q * KS + g * E]), Vf[q], dP);
      }
      float P[16], dS[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int il = 32 * u + acc_row(v, g);
        float x = S[v] * p.scale_log2;
        if (far) {
          x += aq_s[il] + b_far;
        } else {
          const int n = il - jl + BN - 1;
          const int ii = min(i0 + il, sq.len - 1);
          x += TR::to_f(c2pbase[int64_t(ii) * RP + lutc[n]]) + TR::to_f(p2crow[lutp[n]]);
        }
        const bool ok = kvalid && qok_s[il] != 0.f;
        P[v] = ok ? fast_exp2(x - lse_s[il]) : 0.f;
        dS[v] = P[v] * (dP[v] - dlt_s[il]);
      }
#pragma unroll
      for (int q = 0; q < 32 / KS; ++q) {
        const frag pb = TR::pack(&P[q * E]);
        const frag sb = TR::pack(&dS[q * E]);
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) {
          const T* dr = &dOt[(32 * nd + li) * QTP + 32 * u];
          const T* qr = &Qt[(32 * nd + li) * QTP + 32 * u];
          frag a_do, a_q;
          if constexpr (E == 8) {
            a_do = TR::ld2x4(dr + 16 * q + 4 * g, dr + 16 * q + 8 + 4 * g);
            a_q = TR::ld2x4(qr + 16 * q + 4 * g, qr + 16 * q + 8 + 4 * g);
          } else {
            a_do = TR::ld(dr + fed_row<E>(q, 0, g));
            a_q = TR::ld(qr + fed_row<E>(q, 0, g));
          }
          dVt[nd] = TR::mma(a_do, pb, dVt[nd]);
          dKt[nd] = TR::mma(a_q, sb, dKt[nd]);
        }
      }
      // dP2C: ordered walk over this subtile's queries
      if (far) {
        float cs = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) cs += dS[v];
        colsum += cs + xor32(cs);
      } else {
        float other[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) other[v] = xor32(dS[v]);
        if (walker) {
#pragma unroll
          for (int k = 0; k < 32; ++k) {
            const int il = 32 * u + k;
            if (i0 + il >= sq.len) break;
            const float val = walk_grp(k) == 0 ? dS[walk_reg(k)] : other[walk_reg(k)];
            walk.step(lutp[il - jl + BN - 1], val);
          }
        }
      }
    }
    if (far && walker) walk.step(plo, colsum);
  }

  if (!jin) return;
  T* dvp = (T*)p.dv + tok_j * p.ts + int64_t(h) * p.hs;
  float* dkp = p.dk_acc + (int64_t(h) * T_ + tok_j) * D;
#pragma unroll
  for (int nd = 0; nd < ND; ++nd)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int c = 32 * nd + acc_row(v, g);
      dvp[c] = TR::from_f(dVt[nd][v]);
      dkp[c] = dKt[nd][v] * p.scale;
    }
  if (g == 0) walk.finish();
}

template <int DT, int D>
void launch_d(const Params& p, hipStream_t st) {
  dim3 grid(unsigned((p.Lmax + 127) / 128), unsigned(p.H), unsigned(p.nseq));
  constexpr int NQT = (DT == DF_FP32_T && D == 128) ? 1 : 2;
  dkv_kernel<DT, D, NQT><<<grid, 256, 0, st>>>(p);
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

hipError_t launch_bwd_dkv(const Params& p, hipStream_t st) {
  switch (p.dtype) {
    case DF_BF16_T: launch_dt<DF_BF16_T>(p, st); break;
    case DF_FP16_T: launch_dt<DF_FP16_T>(p, st); break;
    default: launch_dt<DF_FP32_T>(p, st); break;
  }
  return hipGetLastError();
}

}  // namespace dfa
