// attend_common.h -- one wave's share of exact attention over tiles of 16
// listed K/V rows, and the merge of a workgroup's wave states.  Used by the
// split kernel (attend.hip) and by the query-prep launch (qprep.hip), whose
// extra workgroups attend over the sink and window rows.
//
// [DySCO review, item 1]: attention is softmax(q k^T / sqrt(d)) v.  Each
// wave keeps an online-softmax state (m, l, acc[d]) per query head in fp32
// (logits scaled by log2(e)/sqrt(d) so exp2 is used); states merge as
//   m* = max m_p,  l* = sum l_p 2^(m_p - m*),  o = sum acc_p 2^(m_p - m*) / l*.
//
// Per tile:
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
// A wave's row ids sit one per lane (lane i: the i-th row of the wave's
// tiles, -1 for none) and are handed out by lane shuffles.
#pragma once

#include "internal.h"

namespace dkv {

constexpr int kAttnTileRows = 16;
constexpr int kAttnPStride = 8;            // floats per row of the p tile (G <= 8)
constexpr int kAttnPartStride = kHeadDim + 2; // m, l, acc[128]

// log2(e) / sqrt(128)
constexpr float kAttnQScale = 1.4426950408889634f * 0.08838834764831845f;

__device__ __forceinline__ void attn_unpack8(const uint4 &v, float (&f)[8]) {
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
__device__ __forceinline__ void attn_merge_state(float &m1, float &l1, float *a1,
                                                 float m2, float l2, const float *a2,
                                                 int n) {
  const float m = fmaxf(m1, m2);
  const float c1 = (m1 == -INFINITY) ? 0.f : exp2f(m1 - m);
  const float c2 = (m2 == -INFINITY) ? 0.f : exp2f(m2 - m);
  l1 = l1 * c1 + l2 * c2;
  for (int i = 0; i < n; ++i) a1[i] = a1[i] * c1 + a2[i] * c2;
  m1 = m;
}

typedef __bf16 attn_v8bf16 __attribute__((ext_vector_type(8)));
typedef float attn_v4f32 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ attn_v8bf16 attn_as_bf16x8(const uint4 &u) {
  return __builtin_bit_cast(attn_v8bf16, u);
}

// max / sum over the four 16-lane rows (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float attn_max_4rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float attn_sum_4rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// A wave's attention state over the G heads of one KV group.
template <int G> struct AttnWave {
  uint4 qb[4];   // query operand: head lrow (zero past G), K-step c
  float m, l;    // state of head lrow (all four lane rows)
  float acc[G][8];
  int lrow, lgrp;
  float (*sp)[kAttnPStride]; // this wave's p tile [16][8] in LDS
  float *sc;                 // and its rescale factors [8]

  // q: the group's first query row ([G][d] bf16)
  __device__ __forceinline__ void init(const uint16_t *q, int lane, float (*sp_)[kAttnPStride],
                                       float *sc_) {
    lrow = lane & 15;
    lgrp = lane >> 4;
    sp = sp_;
    sc = sc_;
    const uint16_t *src = q + (int64_t)min(lrow, G - 1) * kHeadDim + 8 * lgrp;
#pragma unroll
    for (int c = 0; c < 4; ++c) qb[c] = *reinterpret_cast<const uint4 *>(src + 32 * c);
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[h][c] = 0.f;
  }

  // The key and value rows of the tile whose row ids lanes base .. base+15
  // of myid hold (KV head g of a pool row laid out [row][Hkv][d]).  A row
  // id of -1 reads pool row 0 (in bounds) and is dropped in use_tile.  vok
  // bit i: value row lgrp + 4i is a listed row.
  __device__ __forceinline__ void load_tile(int myid, int base, const uint16_t *k_pool,
                                            const uint16_t *v_pool, int Hkv, int g,
                                            uint4 (&kr)[4], uint4 (&vr)[4],
                                            uint32_t &kvalid, uint32_t &vok) const {
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
  }

  __device__ __forceinline__ void use_tile(const uint4 (&kr)[4], const uint4 (&vr)[4],
                                           uint32_t kvalid, uint32_t vok) {
    if (lrow >= G) { // the operand's padding heads are zero
#pragma unroll
      for (int c = 0; c < 4; ++c) qb[c] = make_uint4(0u, 0u, 0u, 0u);
    }
    // ---- logits of the tile's 16 rows for every head
    attn_v4f32 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(attn_as_bf16x8(kr[c]), attn_as_bf16x8(qb[c]),
                                                  S, 0, 0, 0);
    // rows whose id is valid: bit r of the ballot (lanes r, r+16, ... agree)
    const uint32_t vmask = (uint32_t)__ballot(kvalid != 0) & 0xFFFFu;
    float x[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * lgrp + i;
      x[i] = ((vmask >> r) & 1u) ? S[i] * kAttnQScale : -INFINITY;
      tmax = fmaxf(tmax, x[i]);
    }
    tmax = attn_max_4rows(tmax);
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
    psum = attn_sum_4rows(psum);
    l = l * corr + psum;
    m = mn;
    // ---- hand p and corr to the row groups
    if (lrow < G) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sp[4 * lgrp + i][lrow] = p[i];
      if (lgrp == 0) sc[lrow] = corr;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float cr[G];
#pragma unroll
    for (int h = 0; h < G; ++h) cr[h] = sc[h];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[h][c] *= cr[h];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // a value row past the list counts as zeros (its p is 0 too; zeros
      // keep the stand-in row's values, whatever they are, out of the sums)
      float vf[8];
      attn_unpack8(vr[i], vf);
      const bool vin = (vok >> i) & 1u;
#pragma unroll
      for (int c = 0; c < 8; ++c) vf[c] = vin ? vf[c] : 0.f;
      const int r = lgrp + 4 * i;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ph = sp[r][h];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[h][c] = fmaf(ph, vf[c], acc[h][c]);
      }
    }
    // the tile is read before the next one is written
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }

  // The wave's m, l per head and acc per row group are all relative to the
  // same m: sum the four row groups and leave the state in sm[G][2 + d].
  __device__ __forceinline__ void store(float (*sm)[kAttnPartStride]) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[h][c] = attn_sum_4rows(acc[h][c]);
    if (lgrp == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int c = 0; c < 8; ++c) sm[h][2 + 8 * lrow + c] = acc[h][c];
      if (lrow < G) {
        sm[lrow][0] = m;
        sm[lrow][1] = l;
      }
    }
  }
};

// After a barrier that follows every wave's store: the merge of NW wave
// states sm[NW][G][2 + d] into dst[G][2 + d] (global), thread t < G*128
// finishing (head t/128, dim t%128).
template <int G, int NW, int NT>
__device__ __forceinline__ void attn_merge_waves(const float (*sm)[G][kAttnPartStride],
                                                 float *dst) {
  for (int t = threadIdx.x; t < G * kHeadDim; t += NT) {
    const int h = t / kHeadDim, dim = t % kHeadDim;
    float mm = sm[0][h][0], ll = sm[0][h][1], aa = sm[0][h][2 + dim];
    for (int wv = 1; wv < NW; ++wv)
      attn_merge_state(mm, ll, &aa, sm[wv][h][0], sm[wv][h][1], &sm[wv][h][2 + dim], 1);
    float *o = dst + h * kAttnPartStride;
    if (dim == 0) {
      o[0] = mm;
      o[1] = ll;
    }
    o[2 + dim] = aa;
  }
}

// Sink and window rows of a (sequence, KV head) with N cached tokens: the
// list entries [0, base) are positions [0, ns), then [ws, N).
struct SinkWindow {
  int ns, ws, base;
  __device__ __forceinline__ SinkWindow(int N, int w, int sigma) {
    ns = sigma < N ? sigma : N;
    ws = (N - w > ns) ? N - w : ns;
    base = ns + (N - ws);
  }
  __device__ __forceinline__ int pos(int r) const { return r < ns ? r : ws + (r - ns); }
};

} // namespace dkv
