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
// Work mapping: one workgroup per (sequence, 16-token tile).  The tile's
// (token, KV head) pairs are taken in rounds of eight: the round's key rows
// are staged in LDS as doubles, wave v owns pairs v and v+4, and lane j
// keeps the projection chains of columns j, j+64, ... of both pairs, so
// every lane runs 2*b/64 independent index-order chains side by side.  The
// 64 sign bits of a column chunk are packed with one wave ballot.  Lanes 0
// and 1 also run the radius chains of the wave's two pairs.  P is staged
// once per workgroup in LDS.
#include "encode_common.h"

namespace dkv {
namespace {

constexpr int kTile = 16;    // tokens per workgroup
constexpr int kThreads = 256; // four waves
constexpr int kRound = 8;     // (token, KV head) pairs staged at a time

template <int C> // C = b / 64 column chunks
__global__ __launch_bounds__(kThreads) void encode_kernel(
    const uint16_t *__restrict__ k_pool, int64_t num_blocks,
    const int32_t *__restrict__ block_table, int max_blocks,
    const int32_t *__restrict__ enc_start, const int32_t *__restrict__ enc_end,
    int max_encode_len, const uint16_t *__restrict__ proj, int Hkv,
    uint32_t *__restrict__ codes, uint8_t *__restrict__ radii) {
  constexpr int b = 64 * C, W = b / 32;
  __shared__ __align__(16) uint16_t sP[kHeadDim * b]; // [i][j]
  __shared__ double sK[kRound][kHeadDim];
  __shared__ int sBlk[kRound];
  const int s = blockIdx.y;
  const int limit = kPage * max_blocks;
  const int start = clamp_int(enc_start[s], 0, limit);
  int end = clamp_int(enc_end[s], 0, limit);
  if (end - start > max_encode_len) end = start + max_encode_len;
  const int t0 = start + blockIdx.x * kTile;
  if (t0 >= end) return; // whole workgroup leaves together
  const int npairs = min(kTile, end - t0) * Hkv;

  { // proj is 16-byte aligned (checked on the host)
    const uint4 *src = reinterpret_cast<const uint4 *>(proj);
    uint4 *dst = reinterpret_cast<uint4 *>(sP);
    for (int i = threadIdx.x; i < kHeadDim * b / 8; i += kThreads) dst[i] = src[i];
  }

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int32_t *bt = block_table + (int64_t)s * max_blocks;
  for (int p0 = 0; p0 < npairs; p0 += kRound) {
    __syncthreads(); // sP staged / previous round's rows consumed
    {
      // thread -> (pair r, 4 consecutive elements)
      const int r = threadIdx.x >> 5, e = 4 * (threadIdx.x & 31);
      const int p = p0 + r;
      int blk = -1, slot = 0, h = 0;
      if (p < npairs) {
        const int t = t0 + p / Hkv;
        h = p % Hkv;
        slot = t % kPage;
        blk = bt[t / kPage];
        if (blk < 0 || blk >= num_blocks) blk = -1;
      }
      uint2 raw = make_uint2(0u, 0u);
      if (blk >= 0) {
        const uint16_t *krow =
            k_pool + (((int64_t)blk * kPage + slot) * Hkv + h) * kHeadDim;
        raw = *reinterpret_cast<const uint2 *>(krow + e);
      }
      sK[r][e + 0] = (double)bf16_to_float(raw.x & 0xFFFFu);
      sK[r][e + 1] = (double)bf16_to_float(raw.x >> 16);
      sK[r][e + 2] = (double)bf16_to_float(raw.y & 0xFFFFu);
      sK[r][e + 3] = (double)bf16_to_float(raw.y >> 16);
      if ((threadIdx.x & 31) == 0) sBlk[r] = blk;
    }
    __syncthreads();

    const int r0 = wave, r1 = wave + 4;
    double acc0[C], acc1[C];
#pragma unroll
    for (int c = 0; c < C; ++c) acc0[c] = acc1[c] = 0.0;
    double r2 = 0.0;
    const int rr = (lane & 1) ? r1 : r0; // radius chain of lane 0 / lane 1
#pragma unroll 8
    for (int i = 0; i < kHeadDim; ++i) {
      const double k0 = sK[r0][i], k1 = sK[r1][i], kr = sK[rr][i];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const double pv = (double)bf16_to_float(sP[i * b + 64 * c + lane]);
        acc0[c] = fma(k0, pv, acc0[c]);
        acc1[c] = fma(k1, pv, acc1[c]);
      }
      r2 = fma(kr, kr, r2);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = q ? r1 : r0;
      const int p = p0 + r;
      const int blk = sBlk[r];
      if (blk < 0) continue; // wave-uniform
      const int t = t0 + p / Hkv, h = p % Hkv, slot = t % kPage;
      uint32_t *cw = codes + (((int64_t)blk * Hkv + h) * kPage + slot) * W;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const uint64_t mask = __ballot((q ? acc1[c] : acc0[c]) > 0.0);
        if (lane < 2) cw[2 * c + lane] = lane ? (uint32_t)(mask >> 32) : (uint32_t)mask;
      }
      if (lane == q)
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
#define DKV_ENCODE_CASE(CV)                                                    \
  if (b == 64 * CV) {                                                          \
    hipLaunchKernelGGL(encode_kernel<CV>, grid, dim3(kThreads), 0, stream,     \
                       k_pool, num_blocks, block_table, max_blocks, enc_start, \
                       enc_end, max_encode_len, proj, Hkv, codes, radii);      \
    return hipGetLastError();                                                  \
  }
  DKV_ENCODE_CASE(1)
  DKV_ENCODE_CASE(2)
  DKV_ENCODE_CASE(4)
#undef DKV_ENCODE_CASE
  return hipErrorInvalidValue;
}

} // namespace dkv
