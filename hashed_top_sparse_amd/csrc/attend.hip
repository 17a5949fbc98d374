// attend.hip -- exact attention over the selected keys, split over the
// selection list, and the merge of the splits.
//
// [DySCO review, item 1]: attention is softmax(q k^T / sqrt(d)) v.
// [DeepSeek DSA]: the real attention only reads the selected history.
// Each split keeps an online-softmax state (m, l, acc[d]) per query head in
// fp32 (logits are scaled by log2(e)/sqrt(d) so exp2 is used); the combine
// kernel merges the split states:
//   m* = max m_p,  l* = sum l_p 2^(m_p - m*),  o = sum acc_p 2^(m_p - m*) / l*.
//
// Work mapping of the split kernel: 4 waves, each taking its quarter of the
// split's rows in tiles of 16.  Per tile:
//   - logits on the matrix cores: S = K Q^T with four 16x16x32 bf16 ops
//     (K rows as the 16 M rows, the G query heads as N columns, d = 128 in
//     four K-steps of 32).  For K-step c, lane L loads dims 32c + 8(L/16)
//     .. +8 of key row L%16 (so one load instruction reads 64 contiguous
//     bytes of each of 16 rows) and holds the same dims of query head
//     L%16, so both operands use one k order; bf16 x bf16 products are
//     exact in fp32.  S row r, head h ends in lane 16*(r/4) + h, element
//     r%4;
//   - the online softmax runs in that layout (the four lanes of a head are
//     combined with lane-row swaps), and hands the weights p and the
//     rescale factors to the value pass through a per-wave LDS tile;
//   - values on the vector units: 16-lane row groups, lane l holding dims
//     8l .. 8l+7 of rows g, g+4, g+8, g+12 of the tile.
// A wave requests all its tiles' key and value rows at once, then uses them
// in order (its row ids come with one load and are handed out by lane
// shuffles).  The selection list already holds physical row ids (page*16 +
// slot); all G query heads of the KV group share the rows.
#include "internal.h"

namespace dkv {
namespace {

constexpr int kThreads = 256;
constexpr int kPartStride = kHeadDim + 2; // m, l, acc[128]

__device__ __forceinline__ void unpack8(const uint4 &v, float (&f)[8]) {
  f[0] = __uint_as_float(v.x << 16);
  f[1] = __uint_as_float(v.x & 0xFFFF0000u);
  f[2] = __uint_as_float(v.y << 16);
  f[3] = __uint_as_float(v.y & 0xFFFF0000u);
  f[4] = __uint_as_float(v.z << 16);
  f[5] = __uint_as_float(v.z & 0xFFFF0000u);
  f[6] = __uint_as_float(v.w << 16);
  f[7] = __uint_as_float(v.w & 0xFFFF0000u);
}

// Merge online-softmax state (m2, l2, a2) into (m1, l1, a1).
__device__ __forceinline__ void merge_state(float &m1, float &l1, float *a1,
                                            float m2, float l2, const float *a2,
                                            int n) {
  const float m = fmaxf(m1, m2);
  const float c1 = (m1 == -INFINITY) ? 0.f : exp2f(m1 - m);
  const float c2 = (m2 == -INFINITY) ? 0.f : exp2f(m2 - m);
  l1 = l1 * c1 + l2 * c2;
  for (int i = 0; i < n; ++i) a1[i] = a1[i] * c1 + a2[i] * c2;
  m1 = m;
}

typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));
typedef float v4f32 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v8bf16 as_bf16x8(const uint4 &u) {
  return __builtin_bit_cast(v8bf16, u);
}

// max / sum over the four 16-lane rows (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float max_4rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_4rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

constexpr int kWaves = kThreads / 64;
constexpr int kTileRows = 16;
constexpr int kWaveRows = kAttnRows / kWaves;
constexpr int kTiles = kWaveRows / kTileRows;
static_assert(kTiles * kTileRows * kWaves == kAttnRows, "whole tiles");
static_assert(kWaveRows <= 64, "one row id per lane");
constexpr int kPStride = 8; // floats per row of the p tile (G <= 8)

template <int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 2, 8))) void attend_split_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_pool,
    const uint16_t *__restrict__ v_pool, const int32_t *__restrict__ rows,
    const int32_t *__restrict__ cnt, int cap, float *__restrict__ part, int Hq,
    int Hkv, int nsplit, float qscale) {
  const int split = blockIdx.x;
  const int unit = blockIdx.y;
  const int s = unit / Hkv, g = unit % Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int n = cnt[unit];
  const int r0 = split * kAttnRows;
  const int r1 = (r0 + kAttnRows < n) ? r0 + kAttnRows : n;

  // Every load below is issued by every lane, at a clamped in-bounds
  // address, and values that are not needed are dropped where they are
  // used: a load inside a lane-dependent branch makes the compiler wait for
  // it (and for every load issued before it) at the end of the branch.
  //
  // this wave's row ids, one per lane (handed out by lane shuffles); the
  // list is filled up to cap (-1 past the count)
  const int row0 = wave * kWaveRows;
  const int myid_raw = rows[(int64_t)unit * cap + min(r0 + row0 + lane, cap - 1)];
  const int myid = lane < kWaveRows && r0 + row0 + lane < r1 ? myid_raw : -1;

  // query operand: head lrow (zero past G); K-step c takes dims
  // 32c + 8*lgrp .. +8, the same dims the key rows give this lane
  uint4 qb[4];
  {
    const uint16_t *src = q + ((int64_t)s * Hq + (int64_t)g * G + min(lrow, G - 1)) * kHeadDim +
                          8 * lgrp;
#pragma unroll
    for (int c = 0; c < 4; ++c) qb[c] = *reinterpret_cast<const uint4 *>(src + 32 * c);
  }

  // per-wave hand-off tile: p[row][head] and the rescale factors
  __shared__ __attribute__((aligned(16))) float sp[kWaves][kTileRows][kPStride];
  __shared__ __attribute__((aligned(16))) float sc[kWaves][kPStride];

  float m = -INFINITY, l = 0.f; // state of head lrow (all four lane rows)
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[h][c] = 0.f;

  // A tile's key and value rows; a row past the list reads pool row 0 (in
  // bounds) and is dropped in use_tile.  vok bit i: value row lgrp + 4i is
  // a listed row.
  auto load_tile = [&](int t, uint4 (&kr)[4], uint4 (&vr)[4], uint32_t &kvalid,
                       uint32_t &vok) {
    const int base = t * kTileRows;
    const int kid = __shfl(myid, base + lrow);
    kvalid = kid >= 0;
    {
      // load c: the row's bytes 64c .. 64c+63, 16 per lane row group
      const uint16_t *src = k_pool + ((int64_t)max(kid, 0) * Hkv + g) * kHeadDim + 8 * lgrp;
#pragma unroll
      for (int c = 0; c < 4; ++c) kr[c] = *reinterpret_cast<const uint4 *>(src + 32 * c);
    }
    vok = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int vid = __shfl(myid, base + lgrp + 4 * i);
      vok |= (uint32_t)(vid >= 0) << i;
      vr[i] = *reinterpret_cast<const uint4 *>(
          v_pool + ((int64_t)max(vid, 0) * Hkv + g) * kHeadDim + 8 * lrow);
    }
  };
  auto use_tile = [&](const uint4 (&kr)[4], const uint4 (&vr)[4], uint32_t kvalid,
                      uint32_t vok) {
    if (lrow >= G) { // the operand's padding heads are zero
#pragma unroll
      for (int c = 0; c < 4; ++c) qb[c] = make_uint4(0u, 0u, 0u, 0u);
    }
    // ---- logits of the tile's 16 rows for every head
    v4f32 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[c]), as_bf16x8(qb[c]),
                                                  S, 0, 0, 0);
    // rows whose id is valid: bit r of the ballot (lanes r, r+16, ... agree)
    const uint32_t vmask = (uint32_t)__ballot(kvalid != 0) & 0xFFFFu;
    float x[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * lgrp + i;
      x[i] = ((vmask >> r) & 1u) ? S[i] * qscale : -INFINITY;
      tmax = fmaxf(tmax, x[i]);
    }
    tmax = max_4rows(tmax);
    const float mn = fmaxf(m, tmax);
    float corr = 1.f, psum = 0.f;
    float p[4];
    if (mn == -INFINITY) { // nothing valid yet for this head
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = 0.f;
    } else {
      corr = exp2f(m - mn);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = exp2f(x[i] - mn);
        psum += p[i];
      }
    }
    psum = sum_4rows(psum);
    l = l * corr + psum;
    m = mn;
    // ---- hand p and corr to the row groups
    if (lrow < G) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sp[wave][4 * lgrp + i][lrow] = p[i];
      if (lgrp == 0) sc[wave][lrow] = corr;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float cr[G];
#pragma unroll
    for (int h = 0; h < G; ++h) cr[h] = sc[wave][h];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[h][c] *= cr[h];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // a value row past the list counts as zeros (its p is 0 too; zeros
      // keep the stand-in row's values, whatever they are, out of the sums)
      float vf[8];
      unpack8(vr[i], vf);
      const bool vin = (vok >> i) & 1u;
#pragma unroll
      for (int c = 0; c < 8; ++c) vf[c] = vin ? vf[c] : 0.f;
      const int r = lgrp + 4 * i;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ph = sp[wave][r][h];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[h][c] = fmaf(ph, vf[c], acc[h][c]);
      }
    }
    // the tile is read before the next one is written
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  };
  {
    // every tile's rows are requested at once, then used in order
    uint4 kt[kTiles][4], vt[kTiles][4];
    uint32_t ok[kTiles], vok[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) load_tile(t, kt[t], vt[t], ok[t], vok[t]);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) use_tile(kt[t], vt[t], ok[t], vok[t]);
  }

  // The wave's state: m, l per head (lane lrow), acc per row group over its
  // rows, all relative to the same m: sum the four row groups.
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[h][c] = sum_4rows(acc[h][c]);
  __shared__ float sm[kWaves][G][kPartStride];
  if (lgrp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < 8; ++c) sm[wave][h][2 + 8 * lrow + c] = acc[h][c];
    if (lrow < G) {
      sm[wave][lrow][0] = m;
      sm[wave][lrow][1] = l;
    }
  }
  __syncthreads();
  // thread t < G*128 finalises (head t/128, dim t%128)
  for (int t = threadIdx.x; t < G * kHeadDim; t += kThreads) {
    const int h = t / kHeadDim, dim = t % kHeadDim;
    float mm = sm[0][h][0], ll = sm[0][h][1], aa = sm[0][h][2 + dim];
    for (int wv = 1; wv < kWaves; ++wv)
      merge_state(mm, ll, &aa, sm[wv][h][0], sm[wv][h][1], &sm[wv][h][2 + dim], 1);
    float *dst = part + (((int64_t)unit * nsplit + split) * G + h) * kPartStride;
    if (dim == 0) {
      dst[0] = mm;
      dst[1] = ll;
    }
    dst[2 + dim] = aa;
  }
}

// Merge of the split states: one workgroup of 128 threads (one per dim)
// per (sequence, query head).  Splits are taken 32 at a time: threads 0..31
// load the splits' (m, l) into LDS while every thread loads its dim of the
// splits' accumulators, all before any is used, so the loads overlap.
constexpr int kCombineChunk = 32;

__global__ __launch_bounds__(kHeadDim) void attend_combine_kernel(
    const float *__restrict__ part, float *__restrict__ out, int Hq, int Hkv,
    int G, int nsplit) {
  const int sh = blockIdx.x;
  const int s = sh / Hq, hq = sh % Hq;
  const int g = hq / G, h = hq % G;
  const int unit = s * Hkv + g;
  const int dim = threadIdx.x;
  const float *src0 = part + ((int64_t)unit * nsplit * G + h) * kPartStride;
  const int64_t stride = (int64_t)G * kPartStride;
  __shared__ float sml[2][kCombineChunk];
  float mm = -INFINITY, ll = 0.f, aa = 0.f;
  for (int p0 = 0; p0 < nsplit; p0 += kCombineChunk) {
    const int n = min(kCombineChunk, nsplit - p0);
    if (dim < kCombineChunk) {
      const float *src = src0 + (int64_t)(p0 + dim) * stride;
      sml[0][dim] = dim < n ? src[0] : -INFINITY;
      sml[1][dim] = dim < n ? src[1] : 0.f;
    }
    float ap[kCombineChunk];
#pragma unroll
    for (int i = 0; i < kCombineChunk; ++i)
      ap[i] = i < n ? src0[(int64_t)(p0 + i) * stride + 2 + dim] : 0.f;
    __syncthreads();
    float mc = -INFINITY;
#pragma unroll
    for (int i = 0; i < kCombineChunk; ++i) mc = fmaxf(mc, sml[0][i]);
    if (mc != -INFINITY) { // workgroup-uniform
      float lc = 0.f, ac = 0.f;
#pragma unroll
      for (int i = 0; i < kCombineChunk; ++i) {
        const float mp = sml[0][i];
        const float c = (mp == -INFINITY) ? 0.f : exp2f(mp - mc);
        lc = fmaf(sml[1][i], c, lc);
        ac = fmaf(ap[i], c, ac);
      }
      merge_state(mm, ll, &aa, mc, lc, &ac, 1);
    }
    __syncthreads(); // sml is rewritten by the next chunk
  }
  out[(int64_t)sh * kHeadDim + dim] = (ll > 0.f) ? aa / ll : 0.f;
}

} // namespace

hipError_t launch_attend(const DecodeDims &d, const uint16_t *q,
                         const uint16_t *k_pool, const uint16_t *v_pool,
                         const int32_t *rows, const int32_t *cnt, float *part,
                         hipStream_t stream) {
  // log2(e) / sqrt(128)
  const float qscale = 1.4426950408889634f * 0.08838834764831845f;
  dim3 grid(d.nsplit, d.B * d.Hkv);
#define DKV_ATTEND_CASE(GG)                                                    \
  case GG:                                                                     \
    hipLaunchKernelGGL(attend_split_kernel<GG>, grid, dim3(kThreads), 0,       \
                       stream, q, k_pool, v_pool, rows, cnt, d.cap, part,      \
                       d.Hq, d.Hkv, d.nsplit, qscale);                         \
    break;
  switch (d.G) {
    DKV_ATTEND_CASE(1)
    DKV_ATTEND_CASE(2)
    DKV_ATTEND_CASE(4)
    DKV_ATTEND_CASE(8)
  default:
    return hipErrorInvalidValue;
  }
#undef DKV_ATTEND_CASE
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeDims &d, const float *part, float *out,
                          hipStream_t stream) {
  hipLaunchKernelGGL(attend_combine_kernel, dim3(d.B * d.Hq), dim3(kHeadDim),
                     0, stream, part, out, d.Hq, d.Hkv, d.G, d.nsplit);
  return hipGetLastError();
}

} // namespace dkv
