// encode.hip -- key codes and radii at KV write time.
//
// [SPHERICAL KV, §2.1 / §2.3]: each key is stored as a quantised radius and
// a packed angle code, computed when the key is written to the paged cache.
// [DASH-KV, asymmetric hashing]: the key side takes the light encoder and
// its code is reused by every later query.
//
// Code bit j = [p_j > 0] with p_j = sum_i k_i * P_ij accumulated in double
// precision in index order (bf16 x bf16 products are exact in double, so a
// fused multiply-add equals a multiply then an add).  Radius code r8 =
// largest m in 1..255 with |k|^2 >= 2^((m-64)/8), else 0.
//
// Work mapping: one workgroup per (sequence, 16-token tile); one wave per
// (token, KV head) pair at a time; lane j owns projection columns
// j, j+64, ...; the 64 sign bits of a column chunk are packed with one
// wave ballot.  P is staged once per workgroup in LDS.
#include "internal.h"

namespace dkv {
namespace {

constexpr int kTile = 16;   // tokens per workgroup
constexpr int kThreads = 256;

// Nearest doubles to 2^(f/8), f = 0..7.
__constant__ double kEighthOctave[8] = {
    0x1.0000000000000p+0, 0x1.172b83c7d517bp+0, 0x1.306fe0a31b715p+0,
    0x1.4bfdad5362a27p+0, 0x1.6a09e667f3bcdp+0, 0x1.8ace5422aa0dbp+0,
    0x1.ae89f995ad3adp+0, 0x1.d5818dcfba487p+0};

// r8 from |k|^2: with r2 = M * 2^e, M in [1,2), the unclamped code is
// 64 + 8e + f where f is the largest index with M >= C[f].
__device__ int radius_code(double r2) {
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

__global__ __launch_bounds__(kThreads) void encode_kernel(
    const uint16_t *__restrict__ k_pool, int64_t num_blocks,
    const int32_t *__restrict__ block_table, int max_blocks,
    const int32_t *__restrict__ enc_start, const int32_t *__restrict__ enc_end,
    int max_encode_len, const uint16_t *__restrict__ proj, int Hkv, int b,
    uint32_t *__restrict__ codes, uint8_t *__restrict__ radii) {
  extern __shared__ uint16_t sP[]; // [kHeadDim][b]
  const int s = blockIdx.y;
  const int limit = kPage * max_blocks;
  const int start = clamp_int(enc_start[s], 0, limit);
  int end = clamp_int(enc_end[s], 0, limit);
  if (end - start > max_encode_len) end = start + max_encode_len;
  const int t0 = start + blockIdx.x * kTile;
  if (t0 >= end) return; // whole workgroup leaves together

  for (int i = threadIdx.x; i < kHeadDim * b; i += kThreads) sP[i] = proj[i];
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int W = b / 32;
  const int pairs = kTile * Hkv;
  for (int pr = wave; pr < pairs; pr += kThreads / 64) {
    const int t = t0 + pr / Hkv;
    const int h = pr % Hkv;
    if (t >= end) break;
    const int blk = block_table[(int64_t)s * max_blocks + t / kPage];
    if (blk < 0 || blk >= num_blocks) continue;
    const int slot = t % kPage;
    const uint16_t *krow = k_pool + (((int64_t)blk * kPage + slot) * Hkv + h) * kHeadDim;
    uint32_t *cw = codes + ((int64_t)blk * Hkv + h) * W * kPage + slot;
    for (int c = 0; c < b / 64; ++c) {
      const int j = c * 64 + lane;
      double acc = 0.0;
      for (int i = 0; i < kHeadDim; ++i) {
        double kv = (double)bf16_to_float(krow[i]);
        double pv = (double)bf16_to_float(sP[i * b + j]);
        acc = fma(kv, pv, acc);
      }
      const uint64_t mask = __ballot(acc > 0.0);
      if (lane == 0) {
        cw[(2 * c) * kPage] = (uint32_t)mask;
        cw[(2 * c + 1) * kPage] = (uint32_t)(mask >> 32);
      }
    }
    if (lane == 0) {
      double r2 = 0.0;
      for (int i = 0; i < kHeadDim; ++i) {
        double kv = (double)bf16_to_float(krow[i]);
        r2 = fma(kv, kv, r2);
      }
      radii[((int64_t)blk * Hkv + h) * kPage + slot] = (uint8_t)radius_code(r2);
    }
  }
}

} // namespace

hipError_t launch_encode(const uint16_t *k_pool, int64_t num_blocks,
                         const int32_t *block_table, int max_blocks, int batch,
                         const int32_t *enc_start, const int32_t *enc_end,
                         int max_encode_len, const uint16_t *proj, int Hkv,
                         int b, uint32_t *codes, uint8_t *radii,
                         hipStream_t stream) {
  if (max_encode_len <= 0 || batch <= 0) return hipSuccess;
  dim3 grid((max_encode_len + kTile - 1) / kTile, batch);
  size_t lds = sizeof(uint16_t) * kHeadDim * b;
  hipLaunchKernelGGL(encode_kernel, grid, dim3(kThreads), lds, stream, k_pool,
                     num_blocks, block_table, max_blocks, enc_start, enc_end,
                     max_encode_len, proj, Hkv, b, codes, radii);
  return hipGetLastError();
}

} // namespace dkv
