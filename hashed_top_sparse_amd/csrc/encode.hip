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
// largest m in 1..255 with |k|^2 >= 2^((m-64)/8), else 0.  The kernel below
// reaches exactly these values through fp32 matrix ops whose signs are
// certified, with the fp64 chains only where they are not.

#include <algorithm>

#include "encode_common.h"

namespace dkv {
namespace {

// ---------------------------------------------------------------------------
// Matrix-core encode.  p = k.P runs as bf16 x bf16 matrix ops (16 keys x 16
// columns x 32 dims each; the products are exact in fp32, the sums are fp32).
// A sign is certain when |p32| exceeds a bound on the fp32 summation error
// in any order (Cauchy-Schwarz: sum |k_i P_ij| <= |k| |P_j|):
//   |p32 - p| <= 2 (d+1) 2^-23 |k| |P_j| + 2^-100,
// four times the classic (d+1) 2^-24 bound (headroom for the fp32 norms
// themselves; the 2^-100 term covers products that underflow).  Uncertain
// bits are recomputed with the index-order fp64 chain of the definition.
// Likewise |k|^2: an fp32 sum gives the radius code unless it lies within
// 2^-15 (relative) of a code threshold; then the fp64 chain decides.
//
// Work: persistent waves, each keeping its P fragments (64 columns) in
// registers; a tile is (sequence, page, KV head) and a 64-column part of the
// code.  Lane L loads 64 contiguous bytes (dims 32q..32q+31,
// q = L/16) of key row L%16; matrix K-step c pairs dims 32q+8c..32q+8c+7 of
// the row with the same dims of column L%16 of P, so every dim is used
// once.  The next tile's rows are loaded while the current one is scored.
typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));
typedef float v4f32 __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));

constexpr int kMmThreads = 256; // four waves
constexpr int kRangeLds = 1024; // sequences whose encode range sits in LDS
constexpr int kQueue = 64;      // uncertain signs queued per wave

__device__ __forceinline__ uint32_t lanes_below_u64(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ v8bf16 as_v8bf16(const uint4 &u) {
  return __builtin_bit_cast(v8bf16, u);
}

// Index-order fp64 projection of a key row (bf16, staged in LDS) on column
// n of P (LDS, transposed: sPt[n][i]).
__device__ double project_fp64(const uint16_t *krow, const uint16_t *pcol) {
  double acc = 0.0;
#pragma unroll 4
  for (int i = 0; i < kHeadDim; ++i)
    acc = fma((double)bf16_to_float(krow[i]), (double)bf16_to_float(pcol[i]), acc);
  return acc;
}

__device__ double sq_norm_fp64(const uint16_t *krow) {
  double acc = 0.0;
#pragma unroll 4
  for (int i = 0; i < kHeadDim; ++i) {
    const double x = (double)bf16_to_float(krow[i]);
    acc = fma(x, x, acc);
  }
  return acc;
}

// NB: 16-column blocks per wave (64 columns: 64 VGPRs of fragments, two
// waves per SIMD); HALVES: b/64 column parts, each taken by its own
// workgroups (the parts of one tile load the same rows, from L2).
template <int NB, int HALVES>
__global__ __launch_bounds__(kMmThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void encode_mfma_kernel(const uint16_t *__restrict__ k_pool, int64_t num_blocks,
                        const int32_t *__restrict__ block_table, int max_blocks,
                        int batch, const int32_t *__restrict__ enc_start,
                        const int32_t *__restrict__ enc_end, int max_encode_len,
                        int pages_max, const uint16_t *__restrict__ proj, int Hkv,
                        uint32_t *__restrict__ codes, uint8_t *__restrict__ radii) {
  constexpr int b = 16 * NB * HALVES, W = b / 32;
  constexpr int NCOL = 16 * NB;    // columns of this workgroup
  constexpr int WH = NB / 2;       // code words per key in one half
  __shared__ __align__(16) uint16_t sPt[NCOL][kHeadDim]; // P^T of the half
  __shared__ uint64_t sBal[kMmThreads / 64][NB][4]; // sign masks of (cb, i)
  __shared__ uint64_t sUnc[kMmThreads / 64][NB][4]; // uncertain entries
  __shared__ uint4 sQ[kMmThreads / 64][kQueue];      // queued fp64 chains
  __shared__ float sR2[kMmThreads / 64][16];
  __shared__ int2 sRange[kRangeLds];
  // tiles before each sequence's first (balanced mode): sPre[s] =
  // Hkv-free count of the pages the ranges of sequences 0..s-1 meet
  __shared__ int sPre[kRangeLds + 1];
  __shared__ uint32_t sScan[kMmThreads / 64];
  // a tile's key rows, staged only when an fp64 chain has to run
  __shared__ __align__(16) uint16_t sRow[kMmThreads / 64][kPage][kHeadDim];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, col = lane & 15;
  const int half = HALVES > 1 ? (int)(blockIdx.x % HALVES) : 0;
  const int col0 = half * NCOL;
  // positions a block table row reaches (the host keeps max_blocks at or
  // below DKV_MAX_SEQ_LEN / 16, so this fits an int)
  const int limit = (int)min((int64_t)kPage * max_blocks, (int64_t)DKV_MAX_SEQ_LEN);
  // a sequence's encode range [start, end), clamped
  auto range_of = [&](int s_) {
    const int st = clamp_int(enc_start[s_], 0, limit);
    int en = clamp_int(enc_end[s_], 0, limit);
    if (en - st > max_encode_len) en = st + max_encode_len;
    return make_int2(st, en);
  };
  // stage the half's columns of P transposed, and the first sequences'
  // ranges
  for (int e = threadIdx.x; e < kHeadDim * NCOL; e += kMmThreads) {
    const int i = e / NCOL, j = e % NCOL;
    sPt[j][i] = proj[(int64_t)i * b + col0 + j];
  }
  for (int i = threadIdx.x; i < batch && i < kRangeLds; i += kMmThreads) sRange[i] = range_of(i);
  __syncthreads();
  // Balanced mode (every sequence's range in LDS): only the pages the
  // ranges meet are tiles, numbered sequence by sequence, so the waves'
  // runs hold equal work in ragged batches.  Otherwise every sequence has
  // pages_max tile slots, the ones past its range empty.
  const bool bal = batch <= kRangeLds; // workgroup-uniform
  auto pages_met = [](int2 rg) { return rg.y > rg.x ? (rg.y - 1) / kPage - rg.x / kPage + 1 : 0; };
  if (bal) {
    constexpr int kPer = kRangeLds / kMmThreads; // sequences per thread
    const int i0 = (int)threadIdx.x * kPer;
    uint32_t local = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (i0 + u < batch) local += (uint32_t)pages_met(sRange[i0 + u]);
    uint32_t total;
    uint32_t run = wg_exclusive_scan<kMmThreads>(local, sScan, &total);
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (i0 + u < batch) {
        sPre[i0 + u] = (int)run;
        run += (uint32_t)pages_met(sRange[i0 + u]);
      }
    if (threadIdx.x == 0) sPre[batch] = (int)total;
    __syncthreads();
  }
  const __amdgpu_buffer_rsrc_t bt_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t *>(block_table), 0, (uint32_t)(batch * max_blocks) * 4u,
      0x00020000u);
  // this lane's B fragments and column norms
  v8bf16 bfr[NB][4];
  float cn[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const uint16_t *pc = sPt[16 * cb + col];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      bfr[cb][c] = as_v8bf16(*reinterpret_cast<const uint4 *>(pc + 32 * q + 8 * c));
    // |P_col|^2 from the fragments (each dim once across the row's lanes)
    float n2 = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (float)bfr[cb][c][e];
        n2 = fmaf(x, x, n2);
      }
    n2 += __shfl_xor(n2, 16);
    n2 += __shfl_xor(n2, 32);
    cn[cb] = sqrtf(n2) * (1.f + 0x1p-20f);
  }
  // tiles t = ((s * pages_max + pi) * Hkv + h): the heads of a page are
  // neighbours; each wave walks a contiguous run of them (a carry step per
  // tile, no divisions) -- the parts of one tile walk the same runs
  const int ntiles = bal ? sPre[batch] * Hkv : batch * pages_max * Hkv;
  const int nstream = (int)(gridDim.x / HALVES) * (kMmThreads / 64);
  const int chunk = (ntiles + nstream - 1) / nstream;
  const int wid = (int)(blockIdx.x / HALVES) * (kMmThreads / 64) + wave;
  const int t_begin = wid * chunk, t_end = min(ntiles, t_begin + chunk);
  if (t_begin >= t_end) return; // no barriers below

  struct Tile {
    int s, pi, h, start, end, p, blk;
    bool any; // inside the wave's run
  };
  auto set_seq = [&](Tile &T) {
    const int2 rg = T.s < kRangeLds ? sRange[T.s] : range_of(T.s);
    T.start = rg.x;
    T.end = rg.y;
  };
  auto tile_at = [&](int t, Tile &T) {
    T.h = t % Hkv;
    const int r = t / Hkv;
    if (bal) { // the last sequence whose first page slot is at or before r
      int lo = 0, hi = batch; // sPre[lo] <= r < sPre[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sPre[mid] <= r) lo = mid;
        else hi = mid;
      }
      T.s = lo;
      T.pi = r - sPre[lo];
    } else {
      T.pi = r % pages_max;
      T.s = r / pages_max;
    }
    set_seq(T);
    T.p = T.start / kPage + T.pi;
    T.any = t < t_end;
    T.blk = -1;
  };
  auto step = [&](Tile &T, int t_next) { // T becomes tile t_next = its id + 1
    if (++T.h == Hkv) {
      T.h = 0;
      if (bal) {
        if (++T.pi == sPre[T.s + 1] - sPre[T.s]) { // next sequence with pages
          T.pi = 0;
          do
            ++T.s;
          while (T.s < batch && sPre[T.s + 1] == sPre[T.s]);
          if (T.s < batch) set_seq(T);
        }
      } else if (++T.pi == pages_max) {
        T.pi = 0;
        if (++T.s < batch) set_seq(T);
      }
      T.p = T.start / kPage + T.pi;
    }
    T.any = t_next < t_end;
    T.blk = -1;
  };
  // the tile's block id by a vector load (a scalar load would stall the
  // wave where it is used; this one is issued a tile ahead), or -1 when the
  // page is past the range
  auto blk_load = [&](const Tile &T) -> int {
    if (!T.any || T.p * kPage >= T.end) return -1;
    return __builtin_amdgcn_raw_buffer_load_b32(
        bt_rsrc, (T.s * max_blocks + T.p) * 4, 0, 0);
  };
  auto set_blk = [&](Tile &T, int v) {
    const int blk = __builtin_amdgcn_readfirstlane(v);
    T.blk = (blk >= 0 && blk < num_blocks) ? blk : -1;
  };
  auto row_ptr = [&](const Tile &T, int r) {
    return k_pool + (((int64_t)T.blk * kPage + r) * Hkv + T.h) * kHeadDim;
  };
  auto load_rows = [&](const Tile &T, uint4 (&a)[4]) {
    if (T.blk >= 0) {
      const uint4 *src = reinterpret_cast<const uint4 *>(row_ptr(T, col) + 32 * q);
#pragma unroll
      for (int c = 0; c < 4; ++c) a[c] = src[c];
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) a[c] = make_uint4(0u, 0u, 0u, 0u);
    }
  };

  // the queue of uncertain signs: (key row, code word, column | bit << 8)
  uint32_t qn = 0;
  auto flush = [&]() {
    // the words these entries patch were stored by this wave: let those
    // stores complete first
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if ((uint32_t)lane < qn) {
      const uint4 ent = sQ[wave][lane];
      const uint4 *krow = reinterpret_cast<const uint4 *>(k_pool + (int64_t)ent.x * kHeadDim);
      const uint16_t *pcol = sPt[ent.z & 0xFFu];
      double v = 0.0; // the index-order chain
      for (int c = 0; c < kHeadDim / 8; ++c) {
        const uint4 k8 = krow[c];
        const uint32_t kw[4] = {k8.x, k8.y, k8.z, k8.w};
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t kb16 = (u & 1) ? (kw[u / 2] >> 16) : (kw[u / 2] & 0xFFFFu);
          v = fma((double)bf16_to_float(kb16), (double)bf16_to_float(pcol[8 * c + u]), v);
        }
      }
      const uint32_t bit = 1u << (ent.z >> 8);
      if (v > 0.0)
        atomicOr(&codes[ent.y], bit);
      else
        atomicAnd(&codes[ent.y], ~bit);
    }
    qn = 0;
  };

  // four stages: the block id of tile k+3, the rows of tiles k+2 and k+1
  // (two tiles of rows in flight) and the scoring of tile k overlap
  Tile cur, nxt, nx2;
  tile_at(t_begin, cur);
  set_blk(cur, blk_load(cur));
  nxt = cur;
  step(nxt, t_begin + 1);
  set_blk(nxt, blk_load(nxt));
  nx2 = nxt;
  step(nx2, t_begin + 2);
  int bn2 = blk_load(nx2);
  uint4 a[4], an[4];
  load_rows(cur, a);
  load_rows(nxt, an);
  for (int t = t_begin; t < t_end; ++t) {
    Tile nn = nx2;
    step(nn, t + 3);
    const int bnn = blk_load(nn);
    // the rows two tiles ahead are requested before this one is scored
    uint4 an2[4];
    set_blk(nx2, bn2);
    load_rows(nx2, an2);
    if (cur.blk >= 0) { // wave-uniform
      // |k|^2 of row `col` in fp32, two bf16 squares per dot2 (the four
      // lanes of a row combined)
      float r2 = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t wv[4] = {a[c].x, a[c].y, a[c].z, a[c].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const v2bf16 x = __builtin_bit_cast(v2bf16, wv[u]);
          r2 = __builtin_amdgcn_fdot2_f32_bf16(x, x, r2, false);
        }
      }
      r2 += __shfl_xor(r2, 16);
      r2 += __shfl_xor(r2, 32);
      if (lane < 16) sR2[wave][lane] = r2;
      // (read back below by other lanes of the wave)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // the projections
      v4f32 acc[NB];
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) acc[cb] = v4f32{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int cb = 0; cb < NB; ++cb)
          acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf16(a[c]), bfr[cb][c],
                                                            acc[cb], 0, 0, 0);
      // the matrix ops stay in wave-uniform control flow
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) asm volatile("" : "+v"(acc[cb][0]), "+v"(acc[cb][1]), "+v"(acc[cb][2]), "+v"(acc[cb][3]));
      // result lane L: keys 4q+i, column 16cb + col
      float kb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        kb[i] = (float)(2 * (kHeadDim + 1)) * 0x1p-23f * sqrtf(sR2[wave][4 * q + i] * (1.f + 0x1p-20f));
      // rows of the tile inside the encode range (result layout: 4q + i)
      const int base = cur.p * kPage;
      uint64_t inr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = base + 4 * q + i;
        inr[i] = __ballot(pos >= cur.start && pos < cur.end);
      }
      // signs and uncertain entries of (cb, i) as wave masks, to LDS
      uint32_t n_unc = 0;
#pragma unroll
      for (int cb = 0; cb < NB; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = acc[cb][i];
          const uint64_t pos = __ballot(p > 0.f);
          const uint64_t unc =
              __ballot(!(fabsf(p) > fmaf(kb[i], cn[cb], 0x1p-100f))) & inr[i];
          n_unc += (uint32_t)__popcll(unc);
          if (lane == 0) {
            sBal[wave][cb][i] = pos;
            sUnc[wave][cb][i] = unc;
          }
        }
      // radius code of row `lane` from the fp32 sum, unless near a threshold
      int r8 = 0;
      bool runc = false;
      if (lane < kPage) {
        const float r2f = sR2[wave][lane];
        r8 = radius_code_f(r2f * (1.f - 0x1p-15f));
        runc = r8 != radius_code_f(r2f * (1.f + 0x1p-15f));
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // Uncertain signs: the fp32 sign is written now and the entry joins
      // the wave's queue, whose fp64 chains run 64 at a time (one per lane)
      // and patch the written words; a tile with more entries than the
      // queue holds runs its chains here.
      const bool inline_fix = n_unc > (uint32_t)kQueue;
      if (n_unc != 0 && !inline_fix) {
        if (qn + n_unc > (uint32_t)kQueue) flush();
        for (int e = 0; e < NB * 4; ++e) {
          const int cb = e >> 2, i = e & 3;
          const uint64_t unc = sUnc[wave][cb][i];
          if (unc == 0) continue; // wave-uniform
          if ((unc >> lane) & 1u) {
            const int kk = 4 * q + i;
            sQ[wave][qn + lanes_below_u64(unc)] = make_uint4(
                (uint32_t)(((int64_t)cur.blk * kPage + kk) * Hkv + cur.h),
                (uint32_t)((((int64_t)cur.blk * Hkv + cur.h) * kPage + kk) * W + half * WH + cb / 2),
                (uint32_t)(16 * cb + col) | ((uint32_t)(16 * (cb & 1) + col) << 8), 0u);
          }
          qn += (uint32_t)__popcll(unc);
        }
      }
      if (inline_fix || __ballot(runc)) { // rare: the fp64 chains decide
        // the rows go to LDS (lane L holds dims 32q.. of row L%16)
        uint4 *dst = reinterpret_cast<uint4 *>(&sRow[wave][col][32 * q]);
#pragma unroll
        for (int c = 0; c < 4; ++c) dst[c] = a[c];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int e = 0; inline_fix && e < NB * 4; ++e) {
          const int cb = e >> 2, i = e & 3;
          const uint64_t unc = sUnc[wave][cb][i];
          if (unc == 0) continue; // wave-uniform
          const bool mine = (unc >> lane) & 1u;
          double v = 0.0;
          if (mine) v = project_fp64(sRow[wave][4 * q + i], sPt[16 * cb + col]);
          const uint64_t fixed = __ballot(mine && v > 0.0);
          if (lane == 0) sBal[wave][cb][i] = (sBal[wave][cb][i] & ~unc) | fixed;
        }
        if (runc) r8 = radius_code(sq_norm_fp64(sRow[wave][lane]));
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      // code words of this part: lane = key * WH + word
      if (lane < kPage * WH) {
        const int kk = lane / WH, w = lane % WH;
        const int pos = base + kk;
        const int qq = kk >> 2, ii = kk & 3;
        const uint32_t lo = (uint32_t)(sBal[wave][2 * w][ii] >> (16 * qq)) & 0xFFFFu;
        const uint32_t hi = (uint32_t)(sBal[wave][2 * w + 1][ii] >> (16 * qq)) & 0xFFFFu;
        if (pos >= cur.start && pos < cur.end)
          codes[(((int64_t)cur.blk * Hkv + cur.h) * kPage + kk) * W + half * WH + w] =
              lo | (hi << 16);
      }
      // radius of row `lane` (one part writes it)
      if (half == 0 && lane < kPage) {
        const int pos = base + lane;
        if (pos >= cur.start && pos < cur.end)
          radii[((int64_t)cur.blk * Hkv + cur.h) * kPage + lane] = (uint8_t)r8;
      }
      // the next tile's LDS writes wait for these reads
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    cur = nxt;
    nxt = nx2;
    nx2 = nn;
    bn2 = bnn;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      a[c] = an[c];
      an[c] = an2[c];
    }
  }
  if (qn != 0) flush();
}

} // namespace

hipError_t launch_encode(const uint16_t *k_pool, int64_t num_blocks,
                         const int32_t *block_table, int max_blocks, int batch,
                         const int32_t *enc_start, const int32_t *enc_end,
                         int max_encode_len, const uint16_t *proj, int Hkv,
                         int b, uint32_t *codes, uint8_t *radii,
                         hipStream_t stream) {
  if (max_encode_len <= 0 || batch <= 0) return hipSuccess;
  // a range of n positions meets at most ceil(n/16) + 1 pages
  const int pages_max = (max_encode_len + kPage - 1) / kPage + 1;
  const int64_t ntiles = (int64_t)batch * pages_max * Hkv;
  if (ntiles > 0x7FFFFFFF - 65536) return hipErrorInvalidValue;
  if ((int64_t)batch * max_blocks >= (int64_t)1 << 30) return hipErrorInvalidValue;
  // queued fixes name key rows and code words with 32-bit indices
  if ((uint64_t)num_blocks * kPage * Hkv * (b / 32) >= (uint64_t)1 << 32)
    return hipErrorInvalidValue;
  // persistent: two workgroups of four waves per CU, over all parts
  auto streams = [&](int parts) {
    return std::min<int64_t>((ntiles + 3) / 4,
                             std::max<int64_t>(1, 2LL * device_cu_count() / parts));
  };
#define DKV_ENCODE_CASE(BV, NBV, HV)                                           \
  if (b == BV) {                                                               \
    hipLaunchKernelGGL((encode_mfma_kernel<NBV, HV>), dim3((unsigned)(streams(HV) * HV)), \
                       dim3(kMmThreads), 0, stream, k_pool, num_blocks,        \
                       block_table, max_blocks, batch, enc_start, enc_end,     \
                       max_encode_len, pages_max, proj, Hkv, codes, radii);    \
    return hipGetLastError();                                                  \
  }
  DKV_ENCODE_CASE(64, 4, 1)
  DKV_ENCODE_CASE(128, 4, 2)
  DKV_ENCODE_CASE(256, 4, 4)
#undef DKV_ENCODE_CASE
  return hipErrorInvalidValue;
}

} // namespace dkv
