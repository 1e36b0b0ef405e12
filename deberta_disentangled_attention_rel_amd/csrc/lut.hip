// Relative-position index tables (DeBERTa-v2/v3 relative index with optional
// log buckets; DisentangledFlash 1.1.1 page, "Status": v2/v3-style C2P/P2C).
//
//   c2p[d] = clamp(bucket(d) + att, 0, R-1)    row of K_r for query i, key j, d = i - j
//   p2c[d] = clamp(bucket(-d) + att, 0, R-1)   row of Q_r for key j, query i
//
// bucket(d) = d for |d| <= mid (or no buckets); otherwise
// sign(d) * (mid + ceil(x)), x = (mid-1) * ln(|d|/mid) / ln((span-1)/mid).
// x is evaluated in fp64. When it lies within 1e-9 of an integer n, whether x
// equals n exactly is decided in integers: x = n  <=>  (a/mid)^(mid-1) =
// (b/mid)^n (a = |d|, b = span-1), compared prime by prime on the exponents.
#include "common.hpp"

namespace dfa {

namespace {

__device__ int strip_factor(long long& x, long long p) {
  int e = 0;
  while (x % p == 0) {
    x /= p;
    ++e;
  }
  return e;
}

// (a/m)^(m-1) == (b/m)^n exactly?  <=>  for every prime p:
// (m-1) * (v_p(a) - v_p(m)) == n * (v_p(b) - v_p(m)).
__device__ bool exact_power_tie(long long a, long long b, long long m, long long n) {
  long long x[3] = {a, b, m};
  for (long long p = 2;; ++p) {
    long long mx = x[0] > x[1] ? x[0] : x[1];
    mx = mx > x[2] ? mx : x[2];
    if (p * p > mx) break;
    int ea = strip_factor(x[0], p), eb = strip_factor(x[1], p), em = strip_factor(x[2], p);
    if ((m - 1) * (ea - em) != n * (eb - em)) return false;
  }
  // what is left of each number is 1 or a prime
  for (int t = 0; t < 3; ++t) {
    long long q = x[t];
    if (q <= 1) continue;
    int ea = x[0] == q, eb = x[1] == q, em = x[2] == q;
    if ((m - 1) * (ea - em) != n * (eb - em)) return false;
  }
  return true;
}

__device__ int bucket_of(int d, int span, int buckets) {
  if (buckets <= 0) return d;
  const int mid = buckets / 2;
  const int a = d < 0 ? -d : d;
  if (a <= mid) return d;
  const double x = double(mid - 1) * log(double(a) / double(mid)) / log(double(span - 1) / double(mid));
  const double n = rint(x);
  long long k;
  if (fabs(x - n) <= 1e-9 * fmax(1.0, fabs(x)) && exact_power_tie(a, span - 1, mid, (long long)n))
    k = (long long)n;
  else
    k = (long long)ceil(x);
  const int b = mid + int(k);
  return d < 0 ? -b : b;
}

__global__ void lut_kernel(int Lmax, int span, int buckets, int32_t* __restrict__ c2p,
                           int32_t* __restrict__ p2c) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= 2 * Lmax - 1) return;
  const int d = n - (Lmax - 1);
  const int att = buckets > 0 ? buckets : span;
  const int R = 2 * att;
  int c = bucket_of(d, span, buckets) + att;
  int p = bucket_of(-d, span, buckets) + att;
  c2p[n] = c < 0 ? 0 : (c > R - 1 ? R - 1 : c);
  p2c[n] = p < 0 ? 0 : (p > R - 1 ? R - 1 : p);
}

}  // namespace

hipError_t launch_lut(int Lmax, int span, int buckets, int32_t* c2p, int32_t* p2c, hipStream_t st) {
  const int n = 2 * Lmax - 1;
  lut_kernel<<<(n + 255) / 256, 256, 0, st>>>(Lmax, span, buckets, c2p, p2c);
  return hipGetLastError();
}

}  // namespace dfa
