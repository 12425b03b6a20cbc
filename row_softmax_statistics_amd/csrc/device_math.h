// Inline fp64 log for the few exact scores a chunk needs (Gumbel values of
// candidate columns) and the row entropies, written from its series:
//   log x = k ln2 + 2 atanh(s),  x = m 2^k, m in [sqrt(1/2), sqrt(2)),
//           s = (m - 1) / (m + 1), atanh s = s + s^3/3 + s^5/5 + ...
// It is accurate to a few fp64 ulps, far below what any comparison here
// needs. The coefficients are read through a pointer the compiler cannot see
// through, so they are loaded at the point of use (scalar loads) instead of
// being kept in registers across the kernels' loops.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rowstats {

struct MathTable {
  double inv_odd[12];   // 1 / (2 i + 3), i = 0..11
  double ln2_hi;        // ln 2 to 32 significant bits: k * ln2_hi is exact
  double ln2_lo;        // ln 2 - ln2_hi
};

__constant__ const MathTable kMath = {
    {1.0 / 3, 1.0 / 5, 1.0 / 7, 1.0 / 9, 1.0 / 11, 1.0 / 13, 1.0 / 15, 1.0 / 17, 1.0 / 19,
     1.0 / 21, 1.0 / 23, 1.0 / 25},
    0x1.62e42fee00000p-1,
    0x1.a39ef35793c76p-33,
};

typedef const __attribute__((address_space(4))) MathTable *MathTablePtr;

__device__ __forceinline__ MathTablePtr math_table() {
  MathTablePtr t = (MathTablePtr)&kMath;
  __asm__ volatile("" : "+s"(t));
  return t;
}

// Natural log of a positive, finite, normal x.
__device__ __forceinline__ double log_d(double x) {
  MathTablePtr T = math_table();
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  int k = (int)((b >> 52) & 0x7FF) - 1023;
  double m = __longlong_as_double((long long)((b & 0x000FFFFFFFFFFFFFull) | 0x3FF0000000000000ull));
  if (m > 1.4142135623730951) {
    m *= 0.5;
    k += 1;
  }
  const double f = m - 1.0;  // exact: m is within a factor 2 of 1
  const double d = 2.0 + f;
  double r = __builtin_amdgcn_rcp(d);
  r = fma(fma(-d, r, 1.0), r, r);
  r = fma(fma(-d, r, 1.0), r, r);
  double s = f * r;
  s = fma(fma(-d, s, f), r, s);
  const double s2 = s * s;
  double p = T->inv_odd[11];
#pragma unroll
  for (int i = 10; i >= 0; --i) p = fma(p, s2, T->inv_odd[i]);
  const double ts = 2.0 * s;
  const double lm = fma(ts * s2, p, ts);
  const double kd = (double)k;
  return fma(kd, T->ln2_hi, fma(kd, T->ln2_lo, lm));
}

// Standard Gumbel variate of a 32-bit word: u = (w + 0.5) 2^-32 lies in
// (0, 1) and is exact in fp64; g = -log(-log u).
__device__ __forceinline__ double gumbel_of_word(uint32_t w) {
  const double u = ((double)w + 0.5) * 0x1p-32;
  return -log_d(-log_d(u));
}

// -log u of the same u in fp32, relative error below 2^-13, for the
// candidate filters only (never for a score).
__device__ __forceinline__ float neg_log_u_f32(uint32_t w) {
  constexpr float kLn2 = 0.693147180559945309f;
  if (w < 0x80000000u) {  // u < 1/2: log2 of the word itself is accurate
    return (32.0f - __builtin_amdgcn_logf((float)w + 0.5f)) * kLn2;
  }
  const float t = ((float)(~w) + 0.5f) * 0x1p-32f;  // 1 - u in (0, 1/2]
  if (t < 0x1p-10f) return t * (1.0f + t * (0.5f + t * (1.0f / 3.0f)));
  return -__builtin_amdgcn_logf(1.0f - t) * kLn2;
}

}  // namespace rowstats
