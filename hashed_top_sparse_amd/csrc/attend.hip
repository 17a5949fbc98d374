// attend.hip -- exact attention over the selected keys, split over the
// selection list, and the merge of the splits.
//
// [DySCO review, item 1]: attention is softmax(q k^T / sqrt(d)) v.
// [DeepSeek DSA]: the real attention only reads the selected history.
// Each split keeps an online-softmax state (m, l, acc[d]) per query head in
// fp32; the combine kernel merges the split states (attend_common.h).
//
// Work mapping of the split kernel: 4 waves, each taking its quarter of the
// split's rows in tiles of 16 (attend_common.h).  A wave requests all its
// tiles' key and value rows at once, then uses them in order (its row ids
// come with one load and are handed out by lane shuffles).  The selection
// list already holds physical row ids (page*16 + slot); all G query heads
// of the KV group share the rows.
//
// The list of a (sequence, KV head) is its sink rows, its window rows, then
// its top-k rows.  The sinks and the window need no selection: the split
// kernel's first nsw splits take their rows from the positions and the
// block table, and the other splits cover the list past them.  Or the
// query-prep launch attends over the window rows in workgroups of its own
// while the selection is still to come (its state is split 0); then
// nsw = 0 and the splits here cover the sinks and the top-k rows.
#include "attend_common.h"

namespace dkv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kWaveRows = kAttnRows / kWaves;
constexpr int kTiles = kWaveRows / kAttnTileRows;
static_assert(kTiles * kAttnTileRows * kWaves == kAttnRows, "whole tiles");
static_assert(kWaveRows <= 64, "one row id per lane");

// Split `split` of a unit: list rows [split*128, +128) of its sink and
// window rows when split < nsw, else entries [(split-nsw)*128, +128) of
// the rest of the list, up to its count: the rows past the sinks and the
// window (base = their number), preceded by the sinks when `sinks` is set
// (the window then attended elsewhere).  The state goes to split index
// split0 + split of the unit's nsplit.
template <int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 2, 8))) void attend_split_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_pool,
    const uint16_t *__restrict__ v_pool, const int32_t *__restrict__ rows,
    const int32_t *__restrict__ cnt, int cap, const int32_t *__restrict__ seq_lens,
    int n_max, const int32_t *__restrict__ block_table, int max_blocks,
    int64_t num_blocks, int w, int sigma, float *__restrict__ part, int Hq,
    int Hkv, int nsw, bool sinks, int split0, int nsplit) {
  const int split = blockIdx.x;
  const int unit = blockIdx.y;
  const int s = unit / Hkv, g = unit % Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const bool win = split < nsw; // workgroup-uniform
  const int N = seq_len_clamped(seq_lens, s, n_max);
  const SinkWindow sw(N, w, sigma);
  // entries [lo, r1) of this split; entry i of the rest is list row
  // i < ns' ? i : base + i - ns' (ns' = the sinks, or none)
  const int nsk = sinks ? sw.ns : 0;
  const int lo = (win ? split : split - nsw) * kAttnRows;
  const int hi = win ? sw.base : nsk + max(0, min(cnt[unit], cap) - sw.base);
  const int r1 = (lo + kAttnRows < hi) ? lo + kAttnRows : hi;

  // Every load below is issued by every lane, at a clamped in-bounds
  // address, and values that are not needed are dropped where they are
  // used: a load inside a lane-dependent branch makes the compiler wait for
  // it (and for every load issued before it) at the end of the branch.
  //
  // this wave's row ids, one per lane (handed out by lane shuffles): a
  // window row's from its block id, a listed row's from the list (filled
  // up to cap, -1 past the count)
  const int myr = lo + wave * kWaveRows + lane;
  const int wpos = sw.pos(myr);
  const int lrow = myr < nsk ? myr : sw.base + (myr - nsk);
  const int32_t *src = win ? block_table + (int64_t)s * max_blocks +
                                 clamp_int(wpos, 0, max(N - 1, 0)) / kPage
                           : rows + (int64_t)unit * cap + clamp_int(lrow, 0, cap - 1);
  const int raw = *src;
  const int id = win ? ((raw >= 0 && raw < num_blocks) ? raw * kPage + wpos % kPage : -1) : raw;
  const int myid = lane < kWaveRows && myr < r1 ? id : -1;

  __shared__ __attribute__((aligned(16))) float sp[kWaves][kAttnTileRows][kAttnPStride];
  __shared__ __attribute__((aligned(16))) float sc[kWaves][kAttnPStride];
  AttnWave<G> aw;
  aw.init(q + ((int64_t)s * Hq + (int64_t)g * G) * kHeadDim, lane, sp[wave], sc[wave]);
  // the wave's rows (wave-uniform): a tile without any adds nothing to the
  // state (its rows' weights are 0 and the rescale factor 1), so it is
  // neither loaded nor used
  const int wrows = r1 - (lo + wave * kWaveRows);
  static_assert(kTiles == 2, "tile cases below");
  if (wrows > kAttnTileRows) {
    // every tile's rows are requested at once, then used in order
    uint4 kt[kTiles][4], vt[kTiles][4];
    uint32_t ok[kTiles], vok[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
      aw.load_tile(myid, t * kAttnTileRows, k_pool, v_pool, Hkv, g, kt[t], vt[t], ok[t], vok[t]);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) aw.use_tile(kt[t], vt[t], ok[t], vok[t]);
  } else if (wrows > 0) {
    uint4 kt[4], vt[4];
    uint32_t ok, vok;
    aw.load_tile(myid, 0, k_pool, v_pool, Hkv, g, kt, vt, ok, vok);
    aw.use_tile(kt, vt, ok, vok);
  }
  __shared__ float sm[kWaves][G][kAttnPartStride];
  aw.store(sm[wave]);
  __syncthreads();
  attn_merge_waves<G, kWaves, kThreads>(
      sm, part + ((int64_t)unit * nsplit + split0 + split) * G * kAttnPartStride);
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
  const float *src0 = part + ((int64_t)unit * nsplit * G + h) * kAttnPartStride;
  const int64_t stride = (int64_t)G * kAttnPartStride;
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
      attn_merge_state(mm, ll, &aa, mc, lc, &ac, 1);
    }
    __syncthreads(); // sml is rewritten by the next chunk
  }
  out[(int64_t)sh * kHeadDim + dim] = (ll > 0.f) ? aa / ll : 0.f;
}

// Float maximum and sum over a wave, every lane active (DPP moves inside
// rows, then the row swaps; see internal.h).
__device__ __forceinline__ float wave_max_f32(float x) {
  uint32_t v = __float_as_uint(x);
#define DKV_FMAX(A, B) __float_as_uint(fmaxf(__uint_as_float(A), __uint_as_float(B)))
  DKV_DPP_ROW_ALL(v, DKV_FMAX, DKV_DPP_MOV_U32)
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = DKV_FMAX(r[0], r[1]);
  r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = DKV_FMAX(r[0], r[1]);
#undef DKV_FMAX
  return __uint_as_float(v);
}
__device__ __forceinline__ float wave_sum_f32(float x) {
  uint32_t v = __float_as_uint(x);
#define DKV_FADD(A, B) __float_as_uint(__uint_as_float(A) + __uint_as_float(B))
  DKV_DPP_ROW_ALL(v, DKV_FADD, DKV_DPP_MOV_U32)
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = DKV_FADD(r[0], r[1]);
  r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = DKV_FADD(r[0], r[1]);
#undef DKV_FADD
  return __uint_as_float(v);
}

// The merge for more than kCombineWide states (the 4 x 256K workload has
// 34): one workgroup of 128 threads (one per dim) per (sequence, query
// head).  Splits are taken 64 at a time with all their loads issued before
// any is used (one round trip for up to 64 states): every thread loads its dim of the splits' accumulators, and the
// first wave, one split a lane, their (m, l).  That wave takes the chunk's
// maximum m*, each split's factor 2^(m_p - m*) (once per split, into LDS)
// and the chunk's l = sum l_p 2^(m_p - m*).
constexpr int kCombineWide = 64;

__global__ __launch_bounds__(kHeadDim) void attend_combine_wide_kernel(
    const float *__restrict__ part, float *__restrict__ out, int Hq, int Hkv,
    int G, int nsplit) {
  const int sh = blockIdx.x;
  const int s = sh / Hq, hq = sh % Hq;
  const int g = hq / G, h = hq % G;
  const int unit = s * Hkv + g;
  const int dim = threadIdx.x;
  const float *src0 = part + ((int64_t)unit * nsplit * G + h) * kAttnPartStride;
  const int64_t stride = (int64_t)G * kAttnPartStride;
  __shared__ float sfac[kCombineWide];
  __shared__ float sml[2];
  float mm = -INFINITY, ll = 0.f, aa = 0.f;
  for (int p0 = 0; p0 < nsplit; p0 += kCombineWide) { // workgroup-uniform
    const int n = min(kCombineWide, nsplit - p0);
    // loads at clamped in-bounds addresses; values past n are dropped at use
    float ap[kCombineWide];
#pragma unroll
    for (int i = 0; i < kCombineWide; ++i)
      ap[i] = src0[(int64_t)(p0 + min(i, n - 1)) * stride + 2 + dim];
    if (dim < 64) { // the whole first wave
      const float *src = src0 + (int64_t)(p0 + min(dim, n - 1)) * stride;
      const float m_raw = src[0], l_raw = src[1];
      const float mp = dim < n ? m_raw : -INFINITY;
      const float mc = wave_max_f32(mp);
      const float f = (mp == -INFINITY) ? 0.f : exp2f(mp - mc);
      const float lc = wave_sum_f32(dim < n ? l_raw * f : 0.f);
      sfac[dim] = f;
      if (dim == 0) {
        sml[0] = mc;
        sml[1] = lc;
      }
    }
    __syncthreads();
    const float mc = sml[0];
    if (mc != -INFINITY) { // workgroup-uniform
      float ac = 0.f;
#pragma unroll
      for (int i = 0; i < kCombineWide; ++i) ac = fmaf(i < n ? ap[i] : 0.f, sfac[i], ac);
      attn_merge_state(mm, ll, &aa, mc, sml[1], &ac, 1);
    }
    __syncthreads(); // sfac and sml are rewritten by the next chunk
  }
  out[(int64_t)sh * kHeadDim + dim] = (ll > 0.f) ? aa / ll : 0.f;
}

} // namespace

hipError_t launch_attend(const DecodeDims &d, const uint16_t *q,
                         const uint16_t *k_pool, const uint16_t *v_pool,
                         const int32_t *rows, const int32_t *cnt,
                         const int32_t *seq_lens, const int32_t *block_table,
                         float *part, hipStream_t stream) {
  // with the window attended in the prep launch, its state is split 0 and
  // this kernel covers the sinks and the top-k rows
  const int nsw = d.window_in_prep ? 0 : d.nsplit_w;
  const int split0 = d.window_in_prep ? d.nsplit_w : 0;
  const int ns = d.nsplit - split0;
  if (ns == 0) return hipSuccess; // nothing can be listed past the window
  dim3 grid(ns, d.B * d.Hkv);
#define DKV_ATTEND_CASE(GG)                                                    \
  case GG:                                                                     \
    hipLaunchKernelGGL(attend_split_kernel<GG>, grid, dim3(kThreads), 0,       \
                       stream, q, k_pool, v_pool, rows, cnt, d.cap, seq_lens,  \
                       d.n_max, block_table, d.max_blocks, d.num_blocks, d.w,  \
                       d.sigma, part, d.Hq, d.Hkv, nsw, d.window_in_prep,      \
                       split0, d.nsplit);                                      \
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
  // up to 32 states: the per-thread merge (its loads match the state
  // count); more: the wide merge, one round trip for up to 64
  if (d.nsplit <= kCombineChunk)
    hipLaunchKernelGGL(attend_combine_kernel, dim3(d.B * d.Hq), dim3(kHeadDim),
                       0, stream, part, out, d.Hq, d.Hkv, d.G, d.nsplit);
  else
    hipLaunchKernelGGL(attend_combine_wide_kernel, dim3(d.B * d.Hq), dim3(kHeadDim),
                       0, stream, part, out, d.Hq, d.Hkv, d.G, d.nsplit);
  return hipGetLastError();
}

} // namespace dkv
