// attend.hip -- exact attention over the selected keys, split over the
// selection list, and the merge of the splits.
//
// [DySCO review, item 1]: attention is softmax(q k^T / sqrt(d)) v.
// [DeepSeek DSA]: the real attention only reads the selected history.
// Each split keeps an online-softmax state (m, l, acc[d]) per query head in
// fp32 (logits are pre-multiplied by log2(e)/sqrt(d) so exp2 is used); the
// combine kernel merges the split states:
//   m* = max m_p,  l* = sum l_p 2^(m_p - m*),  o = sum acc_p 2^(m_p - m*) / l*.
//
// Work mapping of the split kernel: 256 threads = 16 row groups of 16 lanes;
// a row group reads a selected key row and value row (256 B each: 16 B per
// lane), four rows per batch with the next batch in flight, so a workgroup
// has up to 128 row pairs of gathers outstanding; the split's row ids are
// read once into LDS; the 16-lane dot-product sums use DPP row operations.  The selection list already holds physical row ids
// (page*16 + slot).  All G query heads of the KV group share the rows.
#include "internal.h"

namespace dkv {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerRow = 16;
constexpr int kRowGroups = kThreads / kLanesPerRow;
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

// Sum over the 16 lanes of a DPP row, in every lane of the row: quad xor 1,
// quad xor 2, half-row mirror (the other quad), row mirror (the other half).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum_row16(float x) {
  x += dpp_mov<0xB1>(x);  // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);  // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x); // row_half_mirror
  x += dpp_mov<0x140>(x); // row_mirror
  return x;
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

template <int G>
__global__ __launch_bounds__(kThreads) void attend_split_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_pool,
    const uint16_t *__restrict__ v_pool, const int32_t *__restrict__ rows,
    const int32_t *__restrict__ cnt, int cap, float *__restrict__ part, int Hq,
    int Hkv, int nsplit, float qscale) {
  const int split = blockIdx.x;
  const int unit = blockIdx.y;
  const int s = unit / Hkv, g = unit % Hkv;
  const int lane = threadIdx.x % kLanesPerRow;
  const int rg = threadIdx.x / kLanesPerRow;
  const int n = cnt[unit];
  const int r0 = split * kAttnRows;
  const int r1 = (r0 + kAttnRows < n) ? r0 + kAttnRows : n;

  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 raw = *reinterpret_cast<const uint4 *>(
        q + ((int64_t)s * Hq + (int64_t)g * G + h) * kHeadDim + lane * 8);
    unpack8(raw, qv[h]);
#pragma unroll
    for (int c = 0; c < 8; ++c) qv[h][c] *= qscale;
  }
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[h][c] = 0.f;
  }

  // the split's row ids, once, into LDS
  __shared__ int32_t sid[kAttnRows];
  for (int i = threadIdx.x; i < kAttnRows; i += kThreads) {
    const int r = r0 + i;
    sid[i] = r < r1 ? rows[(int64_t)unit * cap + r] : -1;
  }
  __syncthreads();

  // Row group rg takes rows rg, rg+16, ... of the split: four batches of
  // four, the next batch's loads issued before the current batch is used.
  constexpr int kBatch = 4;
  constexpr int kBatches = kAttnRows / (kBatch * kRowGroups);
  static_assert(kBatches * kBatch * kRowGroups == kAttnRows, "whole batches");
  auto load_batch = [&](int b, uint4 (&kr)[kBatch], uint4 (&vr)[kBatch], bool (&ok)[kBatch]) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int idx = sid[(b * kBatch + i) * kRowGroups + rg];
      ok[i] = idx >= 0;
      const int64_t off = ((int64_t)(ok[i] ? idx : 0) * Hkv + g) * kHeadDim + lane * 8;
      kr[i] = make_uint4(0, 0, 0, 0);
      vr[i] = make_uint4(0, 0, 0, 0);
      if (ok[i]) {
        kr[i] = *reinterpret_cast<const uint4 *>(k_pool + off);
        vr[i] = *reinterpret_cast<const uint4 *>(v_pool + off);
      }
    }
  };
  auto use_batch = [&](const uint4 (&kr)[kBatch], const uint4 (&vr)[kBatch],
                       const bool (&ok)[kBatch]) {
    float dot[G][kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      float kf[8];
      unpack8(kr[i], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) d = fmaf(qv[h][c], kf[c], d);
        dot[h][i] = ok[i] ? sum_row16(d) : -INFINITY;
      }
    }
    float vf[kBatch][8];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) unpack8(vr[i], vf[i]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mn = m[h];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) mn = fmaxf(mn, dot[h][i]);
      if (mn == -INFINITY) continue; // nothing valid yet (uniform per row group)
      const float corr = exp2f(m[h] - mn);
      float pr[kBatch];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        pr[i] = exp2f(dot[h][i] - mn);
        psum += pr[i];
      }
      l[h] = l[h] * corr + psum;
      m[h] = mn;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float a = acc[h][c] * corr;
#pragma unroll
        for (int i = 0; i < kBatch; ++i) a = fmaf(pr[i], vf[i][c], a);
        acc[h][c] = a;
      }
    }
  };
  {
    uint4 ka[kBatch], va[kBatch], kb[kBatch], vb[kBatch];
    bool oa[kBatch], ob[kBatch];
    load_batch(0, ka, va, oa);
#pragma unroll
    for (int b = 0; b < kBatches; b += 2) {
      if (b + 1 < kBatches) load_batch(b + 1, kb, vb, ob);
      use_batch(ka, va, oa);
      if (b + 2 < kBatches) load_batch(b + 2, ka, va, oa);
      if (b + 1 < kBatches) use_batch(kb, vb, ob);
    }
  }

  // Merge the 16 row groups: first the 4 groups of a wave (lanes l, l+16,
  // l+32, l+48 hold the same dims), then the 4 waves through LDS.
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int off2 = 16; off2 < 64; off2 <<= 1) {
      const float m2 = __shfl_xor(m[h], off2);
      const float l2 = __shfl_xor(l[h], off2);
      float a2[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) a2[c] = __shfl_xor(acc[h][c], off2);
      merge_state(m[h], l[h], acc[h], m2, l2, a2, 8);
    }
  }
  __shared__ float sm[4][G][kPartStride];
  const int wave = threadIdx.x / 64;
  if ((threadIdx.x & 63) < kLanesPerRow) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (lane == 0) {
        sm[wave][h][0] = m[h];
        sm[wave][h][1] = l[h];
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) sm[wave][h][2 + lane * 8 + c] = acc[h][c];
    }
  }
  __syncthreads();
  // thread t < G*128 finalises (head t/128, dim t%128)
  for (int t = threadIdx.x; t < G * kHeadDim; t += kThreads) {
    const int h = t / kHeadDim, dim = t % kHeadDim;
    float mm = sm[0][h][0], ll = sm[0][h][1], aa = sm[0][h][2 + dim];
    for (int wv = 1; wv < 4; ++wv)
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
// per (sequence, query head).  Splits are taken 16 at a time, all 16
// states loaded before any is used so the loads overlap.
constexpr int kCombineChunk = 16;

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
  float mm = -INFINITY, ll = 0.f, aa = 0.f;
  for (int p0 = 0; p0 < nsplit; p0 += kCombineChunk) {
    float mp[kCombineChunk], lp[kCombineChunk], ap[kCombineChunk];
#pragma unroll
    for (int i = 0; i < kCombineChunk; ++i) {
      const int p = p0 + i < nsplit ? p0 + i : p0;
      const float *src = src0 + p * stride;
      mp[i] = p0 + i < nsplit ? src[0] : -INFINITY;
      lp[i] = src[1];
      ap[i] = src[2 + dim];
    }
    float mc = -INFINITY;
#pragma unroll
    for (int i = 0; i < kCombineChunk; ++i) mc = fmaxf(mc, mp[i]);
    if (mc == -INFINITY) continue;
    float lc = 0.f, ac = 0.f;
#pragma unroll
    for (int i = 0; i < kCombineChunk; ++i) {
      const float c = (mp[i] == -INFINITY) ? 0.f : exp2f(mp[i] - mc);
      lc = fmaf(lp[i], c, lc);
      ac = fmaf(ap[i], c, ac);
    }
    merge_state(mm, ll, &aa, mc, lc, &ac, 1);
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
