// qprep.hip -- int8 query codes for one decode step, and the matrix-core
// operand the score kernel multiplies them with.
//
// [DASH-KV, asymmetric hashing / dynamic mixed precision]: the query side
// keeps the deeper, higher-precision encoder.  Here: p_hj = q_h . P_:j in
// double precision, index order; one symmetric scale per (sequence, KV
// group): M = max |p| over the group's G heads and all b columns;
// q8 = round_half_even((p * 127) / M) clamped to +-127 (0 when M == 0).
//
// Score operand.  The score kernel computes, per key and query head,
//   D_h = sum_j q8_hj * bit_j   on a 16x16x128 fp8 x fp4 matrix core op,
// with s_h = 2 D_h - Q_h, Q_h = sum_j q8_hj.  The code bits enter as fp4
// nibbles (see score.hip: the nibble for bit j carries the value f_m, m =
// j mod 4, f = {0.5, 1, 2, 0.5}); the query enters as fp8 (e4m3) rows
// 2h (high part) and 2h+1 (low part) with q8 = 16*hi + lo, hi in [-8,7],
// lo in [0,15], each pre-multiplied by 2/f_m so every product is the exact
// even integer 2*hi*bit or 2*lo*bit.  All values are integers of at most
// four significant bits, so they are exact in e4m3 and every partial sum is
// exact in fp32.
//
// Register layout of the 16x16x128 f8f6f4 operation on gfx950 (measured):
//   fp8 operand: lane L holds row L%16; byte p of its 8 dwords is
//     k = 16*(L/16) + p (p < 16) or 64 + 16*(L/16) + (p-16) (p >= 16);
//   fp4 operand: lane L holds column L%16; nibble p of its 4 dwords is
//     k = 32*(L/16) + p;
//   result: lane L holds rows 4*(L/16)+i, i = 0..3, of column L%16.
// The code word (4*ks + L/16) of key L%16 expands into nibble slots
// p = 8m + e <-> bit j = 32*(4*ks + L/16) + 4e + m.
#include "internal.h"

namespace dkv {
namespace {

constexpr int kThreads = 256;

// e4m3 (bias 7) byte of a small integer v, |v| <= 60 with at most four
// significant bits (exactly representable).
__device__ __forceinline__ uint32_t e4m3_of_int(int v) {
  if (v == 0) return 0u;
  const uint32_t sign = v < 0 ? 0x80u : 0u;
  const uint32_t a = (uint32_t)(v < 0 ? -v : v);
  const int e = 31 - __clz(a);                 // floor(log2 a)
  const uint32_t mant = ((a << 3) >> e) - 8u;  // 3 fraction bits, exact
  return sign | ((uint32_t)(e + 7) << 3) | mant;
}

__global__ __launch_bounds__(kThreads) void qprep_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ proj,
    int8_t *__restrict__ q8, uint32_t *__restrict__ qop,
    float *__restrict__ qneg, int Hq, int Hkv, int G, int b, int KS) {
  const int unit = blockIdx.x;
  const int s = unit / Hkv;
  const int g = unit % Hkv;
  __shared__ double sQ[8 * kHeadDim];
  __shared__ uint16_t sP[kHeadDim * 256];
  __shared__ int sq8[8 * 256];
  __shared__ double sMax[kThreads / 64];
  __shared__ int sSum[8];

  const uint16_t *qg = q + ((int64_t)s * Hq + (int64_t)g * G) * kHeadDim;
  for (int i = threadIdx.x; i < G * kHeadDim; i += kThreads)
    sQ[i] = (double)bf16_to_float(qg[i]);
  for (int i = threadIdx.x; i < kHeadDim * b; i += kThreads) sP[i] = proj[i];
  if (threadIdx.x < 8) sSum[threadIdx.x] = 0;
  __syncthreads();

  const int npairs = G * b;
  double p[8];
  double mloc = 0.0;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int idx = threadIdx.x + r * kThreads;
    p[r] = 0.0;
    if (idx < npairs) {
      const int h = idx / b, j = idx % b;
      double acc = 0.0;
      for (int i = 0; i < kHeadDim; ++i)
        acc = fma(sQ[h * kHeadDim + i], (double)bf16_to_float(sP[i * b + j]), acc);
      p[r] = acc;
      mloc = fmax(mloc, fabs(acc));
    }
  }
  for (int off = 32; off > 0; off >>= 1) mloc = fmax(mloc, __shfl_xor(mloc, off));
  if ((threadIdx.x & 63) == 0) sMax[threadIdx.x >> 6] = mloc;
  __syncthreads();
  double M = sMax[0];
  for (int i = 1; i < kThreads / 64; ++i) M = fmax(M, sMax[i]);

  int8_t *qo = q8 + ((int64_t)s * Hq + (int64_t)g * G) * b;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int idx = threadIdx.x + r * kThreads;
    if (idx < npairs) {
      int v = 0;
      if (M != 0.0) {
        const double scaled = p[r] * 127.0;
        const double ratio = scaled / M;
        v = (int)fmin(127.0, fmax(-127.0, rint(ratio)));
      }
      qo[idx] = (int8_t)v;
      sq8[idx] = v;
      atomicAdd(&sSum[idx / b], v);
    }
  }
  __syncthreads();
  if (threadIdx.x < G)
    qneg[(int64_t)s * Hq + (int64_t)g * G + threadIdx.x] = -(float)sSum[threadIdx.x];

  // A operand dwords: [KS][64 lanes][8 dwords]
  uint32_t *dst = qop + (int64_t)unit * KS * 64 * 8;
  for (int t = threadIdx.x; t < KS * 64 * 8; t += kThreads) {
    const int ks = t / 512, la = (t / 8) % 64, di = t % 8;
    const int row = la % 16, gA = la / 16;
    const int h = row / 2, part = row % 2;
    uint32_t word = 0;
    if (h < G) {
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        const int pA = 4 * di + bi;
        const int kk = pA < 16 ? 16 * gA + pA : 64 + 16 * gA + (pA - 16);
        const int tt = kk / 32, pp = kk % 32, m = pp / 8, e = pp % 8;
        const int j = 32 * (4 * ks + tt) + 4 * e + m;
        int v = 0;
        if (j < b) {
          const int qv = sq8[h * b + j];
          const int x = part == 0 ? (qv >> 4) : (qv & 15);
          v = (m == 2) ? x : (m == 1 ? 2 * x : 4 * x);  // 2x / f_m
        }
        word |= e4m3_of_int(v) << (8 * bi);
      }
    }
    dst[t] = word;
  }
}

} // namespace

hipError_t launch_qprep(const DecodeDims &d, const uint16_t *q,
                        const uint16_t *proj, int8_t *q8, uint32_t *qop,
                        float *qneg, hipStream_t stream) {
  hipLaunchKernelGGL(qprep_kernel, dim3(d.B * d.Hkv), dim3(kThreads), 0,
                     stream, q, proj, q8, qop, qneg, d.Hq, d.Hkv, d.G, d.b,
                     d.KS);
  return hipGetLastError();
}

} // namespace dkv
