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
// (b/mid)^n (a = |d|, b = span-1), checked on the reduced numerators and
// denominators through integer roots (a few operations, so the waves that
// meet such a d do not hold the kernel up).
#include "common.hpp"

namespace dfa {

namespace {

__device__ unsigned gcd_u(unsigned a, unsigned b) {
  while (b) {
    const unsigned t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// w^e == target, computed exactly (stops as soon as the power passes target)
__device__ bool power_is(unsigned long long w, unsigned e, unsigned long long target) {
  unsigned long long x = 1;
  for (unsigned i = 0; i < e; ++i) {
    x *= w;
    if (x > target) return false;
  }
  return x == target;
}

// u^k == v^j for positive integers, k, j >= 1. With g = gcd(k, j) this holds
// iff u = w^(j/g) and v = w^(k/g) for one integer w (unique factorisation).
__device__ bool powers_equal(unsigned u, unsigned v, unsigned k, unsigned j) {
  if (u == 1 || v == 1) return u == v;
  const unsigned g = gcd_u(k, j), kk = k / g, jj = j / g;
  const double w0 = rint(exp(log(double(u)) / double(jj)));
  for (int dw = -1; dw <= 1; ++dw) {
    const double w = w0 + dw;
    if (w < 2.0) continue;
    const unsigned long long wi = (unsigned long long)w;
    if (power_is(wi, jj, u)) return power_is(wi, kk, v);
  }
  return false;
}

// (a/m)^(m-1) == (b/m)^n exactly? Both fractions in lowest terms; the
// equality holds iff it holds for the numerators and the denominators apart.
__device__ bool exact_power_tie(unsigned a, unsigned b, unsigned m, long long n) {
  if (n <= 0) return false;
  const unsigned ga = gcd_u(a, m), gb = gcd_u(b, m);
  const unsigned k = m - 1, j = unsigned(n);
  return powers_equal(a / ga, b / gb, k, j) && powers_equal(m / ga, m / gb, k, j);
}

__device__ int bucket_of(int d, int span, int buckets) {
  if (buckets <= 0) return d;
  const int mid = buckets / 2;
  const int a = d < 0 ? -d : d;
  if (a <= mid) return d;
  const double x = double(mid - 1) * log(double(a) / double(mid)) / log(double(span - 1) / double(mid));
  const double n = rint(x);
  long long k;
  if (fabs(x - n) <= 1e-9 * fmax(1.0, fabs(x)) && exact_power_tie(unsigned(a), unsigned(span - 1), unsigned(mid), (long long)n))
    k = (long long)n;
  else
    k = (long long)ceil(x);
  const int b = mid + int(k);
  return d < 0 ? -b : b;
}

__global__ void lut_kernel(int Lmax, int span, int buckets, int p2c_shared, int32_t* __restrict__ c2p,
                           int32_t* __restrict__ p2c, uint32_t* __restrict__ packed) {
  // with `packed`, thread n also writes entry n of the padded packed table
  // (kLutPad entries on each side repeat the end entries)
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  const int pad = packed ? kLutPad : 0;
  if (n >= 2 * Lmax - 1 + 2 * pad) return;
  int d = n - pad - (Lmax - 1);
  d = d < -(Lmax - 1) ? -(Lmax - 1) : (d > Lmax - 1 ? Lmax - 1 : d);
  const int att = buckets > 0 ? buckets : span;
  const int R = 2 * att;
  // bucket is odd, so the P2C row needs no second evaluation
  const int b = bucket_of(d, span, buckets);
  int c = b + att;
  // literal P2C row delta(j, i) = att - bucket(d); the shared convention's
  // row delta(i, j) in reversed coordinates R - 1 - (att + bucket(d))
  int p = p2c_shared ? att - 1 - b : att - b;
  c = c < 0 ? 0 : (c > R - 1 ? R - 1 : c);
  p = p < 0 ? 0 : (p > R - 1 ? R - 1 : p);
  const int m = n - pad;
  if (m >= 0 && m < 2 * Lmax - 1) {
    c2p[m] = c;
    p2c[m] = p;
  }
  if (packed) packed[n] = uint32_t(c) | (uint32_t(p) << 16);
}

}  // namespace

hipError_t launch_lut(int Lmax, int span, int buckets, int p2c_shared, int32_t* c2p, int32_t* p2c, uint32_t* packed,
                      hipStream_t st) {
  const int n = 2 * Lmax - 1 + (packed ? 2 * kLutPad : 0);
  lut_kernel<<<(n + 255) / 256, 256, 0, st>>>(Lmax, span, buckets, p2c_shared, c2p, p2c, packed);
  return hipGetLastError();
}

// dst[h][r][:] = src[h][R - 1 - r][:] for contiguous [H][R][D] rows (the
// shared P2C convention's reversed q_r), 16 bytes per thread.
namespace {
__global__ void reverse_rows_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int H, int R,
                                    int chunks_per_row) {
  const int64_t n = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = int64_t(H) * R * chunks_per_row;
  if (n >= total) return;
  const int64_t row = n / chunks_per_row, c = n % chunks_per_row;
  const int64_t h = row / R, r = row % R;
  dst[n] = src[(h * R + (R - 1 - r)) * chunks_per_row + c];
}
}  // namespace

hipError_t launch_reverse_rows(const void* src, void* dst, int H, int R, int D, int elem_bytes, hipStream_t st) {
  const int cpr = D * elem_bytes / 16;
  const int64_t total = int64_t(H) * R * cpr;
  if (total == 0) return hipSuccess;
  reverse_rows_kernel<<<unsigned((total + 255) / 256), 256, 0, st>>>((const uint4*)src, (uint4*)dst, H, R, cpr);
  return hipGetLastError();
}

// The relative rows transposed for the backward kernels' epilogue, in
// 16-byte chunks: dst[h][r / CE][d][r % CE] = src[h][r][d] for r < R, 0 for
// R <= r < RP, CE = 16 bytes of elements. A chunk of one row d holds the
// 16 bytes one lane loads, and the chunks of consecutive rows d are adjacent,
// so the 32 rows a load instruction reads are one contiguous 512-byte run.
namespace {
template <typename T>
__global__ void transpose_rows_kernel(const T* __restrict__ src, T* __restrict__ dst, int H, int R, int RP, int D) {
  constexpr int CE = 16 / int(sizeof(T));
  const int64_t n = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (n >= int64_t(H) * D * RP) return;
  const int NC = RP / CE;
  int64_t t = n / CE;
  const int64_t e = n % CE, d = t % D;
  t /= D;
  const int64_t c = t % NC, h = t / NC;
  const int64_t r = c * CE + e;
  dst[n] = r < R ? src[(h * R + r) * D + d] : T(0);
}
}  // namespace

hipError_t launch_transpose_rows(const void* src, void* dst, int H, int R, int RP, int D, int elem_bytes,
                                 hipStream_t st) {
  const int64_t total = int64_t(H) * D * RP;
  if (total == 0) return hipSuccess;
  const unsigned nb = unsigned((total + 255) / 256);
  if (elem_bytes == 4)
    transpose_rows_kernel<uint32_t><<<nb, 256, 0, st>>>((const uint32_t*)src, (uint32_t*)dst, H, R, RP, D);
  else
    transpose_rows_kernel<uint16_t><<<nb, 256, 0, st>>>((const uint16_t*)src, (uint16_t*)dst, H, R, RP, D);
  return hipGetLastError();
}

}  // namespace dfa
