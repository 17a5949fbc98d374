// select_common.h -- exact k-th largest over a workgroup's elements, and the
// position-ordered list built from a selection bitmap.
//
// Selection order ([DASH-KV Top-K pruning]; ties to the lowest position):
// values are biased scores u = S + 2^31 (or, for tie-breaking, inverted
// positions), so the range of a set of values can span all 32 bits.  The
// k-th largest value T and the number of elements equal to T to take are
// found with histogram passes over 4096 bins: the first over
// (u - min) >> shift, with the shift chosen so the elements' range fits the
// bins, then one pass per further 12 bits (or fewer) inside the bin found so
// far, until the bins are single values: at most three passes for a 32-bit
// range.
#pragma once

#include "internal.h"

namespace dkv {

constexpr int kHistBits = 12;
constexpr int kHistBins = 1 << kHistBits;

constexpr int kCutList = 64; // threshold-bin entries one wave ranks

template <int NT>
struct SelectShared {
  uint32_t hist[kHistBins];
  uint32_t red[4][NT / 64];
  int bin;
  uint32_t above;
  uint2 cut_list[kCutList];
  uint32_t cut_n, cut_u, cut_pos;
};

// Scanning bins from the top, finds the bin where the running count reaches
// kneed: count(bins above) < kneed <= count(bins above) + bin.  Every
// thread must call it; ends with a barrier.
template <int NT>
__device__ __forceinline__ void find_threshold_bin(SelectShared<NT> &sh, uint32_t kneed) {
  constexpr int kPer = kHistBins / NT;
  const int top = kHistBins - 1 - kPer * (int)threadIdx.x;
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) local += sh.hist[top - i];
  uint32_t total;
  const uint32_t above = wg_exclusive_scan<NT>(local, &sh.red[3][0], &total);
  if (above < kneed && kneed <= above + local) {
    uint32_t run = above;
    for (int i = 0; i < kPer; ++i) {
      const uint32_t c = sh.hist[top - i];
      if (run + c >= kneed) {
        sh.bin = top - i;
        sh.above = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
}

// Value range of the elements visit(fn) hands out, and the histogram of
// (v - vmin) >> shift with the shift chosen so the range fits the bins.
// Every thread must call it; ends with a barrier.
template <int NT, class Visit>
__device__ __forceinline__ void wg_histogram(SelectShared<NT> &sh, Visit visit, uint32_t &vmin,
                             int &shift) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  visit([&](uint32_t v) {
    lo = min(lo, v);
    hi = max(hi, v);
  });
  wave_min_max(lo, hi);
  if (lane == 0) {
    sh.red[0][wave] = lo;
    sh.red[1][wave] = hi;
  }
  for (int i = threadIdx.x; i < kHistBins; i += NT) sh.hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    lo = min(lo, sh.red[0][i]);
    hi = max(hi, sh.red[1][i]);
  }
  const uint32_t range = hi - lo;
  const int bits = range == 0 ? 0 : 32 - __clz(range);
  shift = bits > kHistBits ? bits - kHistBits : 0;
  vmin = lo;
  const int sh_ = shift;
  visit([&](uint32_t v) { atomicAdd(&sh.hist[(v - lo) >> sh_], 1u); });
  __syncthreads();
}

// A lower bound of the kneed-th largest element (1 <= kneed <= element
// count): the lowest value of the histogram bin that holds it, so at least
// kneed elements are >= the result.  Every thread must call it.
template <int NT, class Visit>
__device__ __forceinline__ uint32_t wg_kth_largest_floor(SelectShared<NT> &sh, Visit visit,
                                         uint32_t kneed) {
  uint32_t vmin;
  int shift;
  wg_histogram<NT>(sh, visit, vmin, shift);
  find_threshold_bin<NT>(sh, kneed);
  const uint32_t T = vmin + ((uint32_t)sh.bin << shift);
  __syncthreads();
  return T;
}

// Exact kneed-th largest value (1 <= kneed <= element count) of the
// elements that visit(fn) hands to fn(uint32_t) -- each element exactly
// once across the workgroup.  Returns T, the number of elements equal to T
// (n_eq) and how many of those complete the top kneed (take_eq, >= 1).
// Every thread must call it (barriers inside).
template <int NT, class Visit>
__device__ __forceinline__ void wg_kth_largest(SelectShared<NT> &sh, Visit visit, uint32_t kneed,
                               uint32_t &T, uint32_t &take_eq, uint32_t &n_eq) {
  uint32_t vmin;
  int shift;
  wg_histogram<NT>(sh, visit, vmin, shift);
  find_threshold_bin<NT>(sh, kneed);
  // prefix: the bits of (T - vmin) above `shift` found so far
  uint32_t prefix = (uint32_t)sh.bin;
  uint32_t kleft = kneed - sh.above; // >= 1: elements still to take at or below the prefix
  n_eq = sh.hist[sh.bin];
  __syncthreads();
  while (shift > 0) { // workgroup-uniform
    // the next (at most) kHistBits bits below the prefix
    const int next = shift > kHistBits ? shift - kHistBits : 0;
    const int width = shift - next;
    const uint32_t mask = (1u << width) - 1u;
    for (int i = threadIdx.x; i < kHistBins; i += NT) sh.hist[i] = 0;
    __syncthreads();
    const int sh_ = shift;
    visit([&](uint32_t v) {
      const uint32_t d = v - vmin;
      if ((d >> sh_) == prefix) atomicAdd(&sh.hist[(d >> next) & mask], 1u);
    });
    __syncthreads();
    find_threshold_bin<NT>(sh, kleft);
    prefix = (prefix << width) | (uint32_t)sh.bin;
    kleft -= sh.above;
    n_eq = sh.hist[sh.bin];
    shift = next;
    __syncthreads();
  }
  // the bins of the last pass were single values
  T = vmin + prefix;
  take_eq = kleft;
}

// The top kneed (1 <= kneed <= element count) of (u, pos) pairs under the
// order (u descending, pos ascending), positions distinct: visit2(fn) hands
// every pair to fn(u, pos) once across the workgroup.  On success the cut
// (Tu, Tpos) is returned: a pair is in the top kneed iff u > Tu, or u == Tu
// and pos <= Tpos.  One histogram pass finds the bin of the kneed-th
// largest u; when that bin holds at most kCutList pairs, one wave ranks
// them exactly.  Returns false otherwise (the caller then searches with
// wg_kth_largest).  Every thread must call it.
template <int NT, class Visit2>
__device__ __forceinline__ bool wg_topk_cut_tail(SelectShared<NT> &sh, Visit2 visit2,
                                                 uint32_t kneed, uint32_t vmin, int shift,
                                                 uint32_t &Tu, uint32_t &Tpos);

template <int NT, class Visit2>
__device__ __forceinline__ bool wg_topk_cut(SelectShared<NT> &sh, Visit2 visit2, uint32_t kneed,
                            uint32_t &Tu, uint32_t &Tpos) {
  uint32_t vmin;
  int shift;
  wg_histogram<NT>(sh, [&](auto fn) {
    visit2([&](uint32_t u, int) { fn(u); });
  }, vmin, shift);
  return wg_topk_cut_tail<NT>(sh, visit2, kneed, vmin, shift, Tu, Tpos);
}

// wg_topk_cut when the caller already has the range: sh.red[0][w] and
// sh.red[1][w] hold wave w's minimum and maximum u, and sh.hist is zero,
// both written before a barrier that every thread has passed.
template <int NT, class Visit2>
__device__ __forceinline__ bool wg_topk_cut_ranged(SelectShared<NT> &sh, Visit2 visit2,
                                                   uint32_t kneed, uint32_t &Tu,
                                                   uint32_t &Tpos) {
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    lo = min(lo, sh.red[0][i]);
    hi = max(hi, sh.red[1][i]);
  }
  const uint32_t range = hi - lo;
  const int bits = range == 0 ? 0 : 32 - __clz(range);
  const int shift = bits > kHistBits ? bits - kHistBits : 0;
  visit2([&](uint32_t u, int) { atomicAdd(&sh.hist[(u - lo) >> shift], 1u); });
  __syncthreads();
  return wg_topk_cut_tail<NT>(sh, visit2, kneed, lo, shift, Tu, Tpos);
}

// The rest of wg_topk_cut once sh.hist holds the histogram of
// (u - vmin) >> shift (followed by a barrier).
template <int NT, class Visit2>
__device__ __forceinline__ bool wg_topk_cut_tail(SelectShared<NT> &sh, Visit2 visit2,
                                                 uint32_t kneed, uint32_t vmin, int shift,
                                                 uint32_t &Tu, uint32_t &Tpos) {
  find_threshold_bin<NT>(sh, kneed);
  const uint32_t b1 = (uint32_t)sh.bin;
  const uint32_t kneed2 = kneed - sh.above; // >= 1
  const uint32_t nb1 = sh.hist[b1];
  if (nb1 > (uint32_t)kCutList) return false; // workgroup-uniform
  if (threadIdx.x == 0) sh.cut_n = 0;
  __syncthreads();
  visit2([&](uint32_t u, int pos) {
    if (((u - vmin) >> shift) == b1)
      sh.cut_list[atomicAdd(&sh.cut_n, 1u)] = make_uint2(u, (uint32_t)pos);
  });
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const uint2 e = lane < (int)nb1 ? sh.cut_list[lane] : make_uint2(0u, 0xFFFFFFFFu);
    uint32_t rank = 0; // pairs ahead of e in the order
    // the list is read back with broadcast LDS reads, eight at a time
    for (int j0 = 0; j0 < (int)nb1; j0 += 8) {
      uint2 f[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) f[t] = sh.cut_list[j0 + t];
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (j0 + t < (int)nb1)
          rank += (f[t].x > e.x) || (f[t].x == e.x && f[t].y < e.y);
    }
    if (lane < (int)nb1 && rank == kneed2 - 1) {
      sh.cut_u = e.x;
      sh.cut_pos = e.y;
    }
  }
  __syncthreads();
  Tu = sh.cut_u;
  Tpos = sh.cut_pos;
  __syncthreads();
  return true;
}

// Writes the positions of the set bits of bitmap[0, nwords) (bit p = word
// p/32, bit p%32) in ascending order to pos_out[0..] / row_out[0..] (row =
// page*16 + slot through the block table, -1 for an invalid page), at most
// max_out of them; returns their number.  Every thread must call it.
template <int NT>
__device__ __forceinline__ uint32_t emit_bitmap(const uint32_t *bitmap, int nwords, const int32_t *bt,
                                int64_t num_blocks, int32_t *row_out,
                                int32_t *pos_out, uint32_t *tmp, uint32_t max_out) {
  const int per = (nwords + NT - 1) / NT;
  const int w0 = min(nwords, (int)threadIdx.x * per);
  const int w1 = min(nwords, w0 + per);
  uint32_t c = 0;
  for (int i = w0; i < w1; ++i) c += __popc(bitmap[i]);
  uint32_t total;
  uint32_t o = wg_exclusive_scan<NT>(c, tmp, &total);
  for (int i = w0; i < w1; ++i) {
    uint32_t m = bitmap[i];
    while (m && o < max_out) {
      const int bitp = __ffs(m) - 1;
      m &= m - 1;
      const int pos = i * 32 + bitp;
      const int blk = bt[pos / kPage];
      row_out[o] = (blk >= 0 && blk < num_blocks) ? blk * kPage + pos % kPage : -1;
      if (pos_out) pos_out[o] = pos;
      ++o;
    }
  }
  return min(total, max_out);
}

} // namespace dkv
