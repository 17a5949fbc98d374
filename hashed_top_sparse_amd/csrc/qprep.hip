// qprep.hip -- int8 query codes for one decode step.
//
// [DASH-KV, asymmetric hashing / dynamic mixed precision]: the query side
// keeps the deeper, higher-precision encoder.  Here: p_hj = q_h . P_:j in
// double precision, index order; one symmetric scale per (sequence, KV
// group): M = max |p| over the group's G heads and all b columns;
// q8 = round_half_even((p * 127) / M) clamped to +-127 (0 when M == 0).
//
// One workgroup per (sequence, KV head); each thread owns up to 8 (head,
// column) pairs (G*b <= 8*256).
#include "internal.h"

namespace dkv {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void qprep_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ proj,
    int8_t *__restrict__ q8, int Hq, int Hkv, int G, int b) {
  const int unit = blockIdx.x;
  const int s = unit / Hkv;
  const int g = unit % Hkv;
  __shared__ float sQ[8 * kHeadDim];
  __shared__ double sMax[kThreads / 64];
  const uint16_t *qg = q + ((int64_t)s * Hq + (int64_t)g * G) * kHeadDim;
  for (int i = threadIdx.x; i < G * kHeadDim; i += kThreads)
    sQ[i] = bf16_to_float(qg[i]);
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
        acc = fma((double)sQ[h * kHeadDim + i],
                  (double)bf16_to_float(proj[i * b + j]), acc);
      p[r] = acc;
      mloc = fmax(mloc, fabs(acc));
    }
  }
  // workgroup maximum of |p|
  for (int off = 32; off > 0; off >>= 1)
    mloc = fmax(mloc, __shfl_xor(mloc, off));
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
        double scaled = p[r] * 127.0;
        double ratio = scaled / M;
        double rr = rint(ratio);
        rr = fmin(127.0, fmax(-127.0, rr));
        v = (int)rr;
      }
      qo[idx] = (int8_t)v;
    }
  }
}

} // namespace

hipError_t launch_qprep(const DecodeDims &d, const uint16_t *q,
                        const uint16_t *proj, int8_t *q8, hipStream_t stream) {
  hipLaunchKernelGGL(qprep_kernel, dim3(d.B * d.Hkv), dim3(kThreads), 0,
                     stream, q, proj, q8, d.Hq, d.Hkv, d.G, d.b);
  return hipGetLastError();
}

} // namespace dkv
