// encode_common.h -- the key radius code, shared by the bulk encode kernel
// and the append encode inside the query-prep kernel.
//
// [SPHERICAL KV, §2.1]: a key keeps a quantised radius beside its angle
// code.  r8 = largest m in 1..255 with |k|^2 >= 2^((m-64)/8), else 0.
#pragma once

#include "internal.h"

namespace dkv {

// Nearest doubles to 2^(f/8), f = 0..7.
static __constant__ double kEighthOctave[8] = {
    0x1.0000000000000p+0, 0x1.172b83c7d517bp+0, 0x1.306fe0a31b715p+0,
    0x1.4bfdad5362a27p+0, 0x1.6a09e667f3bcdp+0, 0x1.8ace5422aa0dbp+0,
    0x1.ae89f995ad3adp+0, 0x1.d5818dcfba487p+0};

// r8 from |k|^2: with r2 = M * 2^e, M in [1,2), the unclamped code is
// 64 + 8e + f where f is the largest index with M >= C[f].
static __device__ int radius_code(double r2) {
  if (!(r2 > 0.0)) return 0;
  int e;
  double mant = frexp(r2, &e); // r2 = mant * 2^e, mant in [0.5, 1)
  double M = mant * 2.0;
  e -= 1;
  int f = 0;
#pragma unroll
  for (int i = 1; i < 8; ++i)
    if (M >= kEighthOctave[i]) f = i;
  long m = 64L + 8L * e + f;
  if (m < 1) return 0;
  if (m > 255) return 255;
  return (int)m;
}

// The same code from an fp32 |k|^2 with fp32 thresholds (each within 2^-24
// of its double).  Only used to find codes whose value is certain: a caller
// compares the codes of r2 (1 - 2^-15) and r2 (1 + 2^-15), which a rounding
// of 2^-24 here cannot make equal when the exact code differs.
__device__ __forceinline__ int radius_code_f(float r2) {
  if (!(r2 > 0.f)) return 0;
  int e;
  const float M = 2.f * frexpf(r2, &e); // r2 = M * 2^(e-1), M in [1,2)
  e -= 1;
  int f = 0;
#pragma unroll
  for (int i = 1; i < 8; ++i)
    if (M >= (float)kEighthOctave[i]) f = i;
  const int m = 64 + 8 * e + f;
  return m < 1 ? 0 : (m > 255 ? 255 : m);
}

} // namespace dkv
