// merge.hip -- final selection of one decode step per (sequence, KV head).
//
// [DASH-KV Top-K pruning; DeepSeek DSA]: exact attention runs over the
// top-k keys only; [DeepSeek CSA]: plus the sliding window of the most
// recent tokens; [DySCO FAQ 3]: plus the first tokens (attention sinks).
//   sinks   [0, min(sigma, N))
//   window  [max(min(sigma, N), N - w), N)
//   top-k   the min(k, |C|) best of C = [sigma, N - w) by (S desc, pos asc)
// The score kernel left each chunk's exact top-k in position order; their
// union holds the global top-k.  Two 12-bit radix histogram passes over the
// union find the threshold score T and how many ties at T to keep, and a
// workgroup scan writes the survivors in position order.
//
// Output list per unit: sinks, window, then the top-k in ascending
// position, as physical row ids (page*16 + slot, for the attention gather)
// and, when asked, as logical positions; -1 past the count.
#include "internal.h"

namespace dkv {
namespace {

constexpr int kThreads = 1024;
constexpr int kHistBits = 12;
constexpr int kHistBins = 1 << kHistBits;
constexpr int kMaxChunks = 4096;

__device__ void find_threshold_bin(const uint32_t *hist, uint32_t kneed,
                                   uint32_t *tmp, int *out_bin,
                                   uint32_t *out_above) {
  constexpr int kPer = kHistBins / kThreads;
  const int top = kHistBins - 1 - kPer * threadIdx.x;
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) local += hist[top - i];
  uint32_t total;
  const uint32_t above = wg_exclusive_scan<kThreads>(local, tmp, &total);
  if (above < kneed && kneed <= above + local) {
    uint32_t run = above;
    for (int i = 0; i < kPer; ++i) {
      const uint32_t c = hist[top - i];
      if (run + c >= kneed) {
        *out_bin = top - i;
        *out_above = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ int row_of(const int32_t *bt, int pos,
                                      int64_t num_blocks) {
  const int blk = bt[pos / kPage];
  return (blk >= 0 && blk < num_blocks) ? blk * kPage + pos % kPage : -1;
}

__global__ __launch_bounds__(kThreads) void merge_kernel(
    const uint2 *__restrict__ cand, const int32_t *__restrict__ cand_cnt,
    int nchunks, const int32_t *__restrict__ seq_lens, int n_max,
    const int32_t *__restrict__ block_table, int max_blocks,
    int64_t num_blocks, int Hkv, int k, int w, int sigma, int cap,
    int32_t *__restrict__ rows, int32_t *__restrict__ cnt,
    int32_t *__restrict__ user_sel, int32_t *__restrict__ user_cnt) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t tmp[kThreads / 64];
  __shared__ uint32_t coff[kMaxChunks + 1]; // prefix offsets of chunk counts
  __shared__ int sh_bin;
  __shared__ uint32_t sh_above;

  const int unit = blockIdx.x;
  const int s = unit / Hkv;
  const int tid = threadIdx.x;
  const int N = seq_len_clamped(seq_lens, s, n_max);
  const int ns = sigma < N ? sigma : N;
  const int ws = (N - w > ns) ? N - w : ns;
  const int nwin = N - ws;
  const int nc = max(0, N - w - sigma);
  const int keff = min(k, nc);
  const int total = ns + nwin + keff;
  const int base = ns + nwin;
  const int32_t *bt = block_table + (int64_t)s * max_blocks;
  int32_t *R = rows + (int64_t)unit * cap;
  int32_t *U = user_sel ? user_sel + (int64_t)unit * cap : nullptr;

  for (int i = tid; i < base; i += kThreads) {
    const int pos = i < ns ? i : ws + (i - ns);
    R[i] = row_of(bt, pos, num_blocks);
    if (U) U[i] = pos;
  }
  for (int i = total + tid; i < cap; i += kThreads) {
    R[i] = -1;
    if (U) U[i] = -1;
  }

  if (keff > 0) {
    const int npages = (N + kPage - 1) / kPage;
    const int nch = min(nchunks, (npages + kChunkPages - 1) / kChunkPages);
    const int32_t *cc = cand_cnt + (int64_t)unit * nchunks;
    const uint2 *cu = cand + (int64_t)unit * nchunks * (int64_t)k;
    // chunk offsets in the flattened (chunk-major, position-ordered) list
    if (tid == 0) {
      uint32_t run = 0;
      for (int c = 0; c < nch; ++c) {
        coff[c] = run;
        run += (uint32_t)cc[c];
      }
      coff[nch] = run;
    }
    __syncthreads();
    const uint32_t nall = coff[nch];
    auto elem = [&](uint32_t e) -> uint2 {
      // chunk holding flattened index e (binary search over offsets)
      int lo = 0, hi = nch - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (coff[mid] <= e) lo = mid; else hi = mid - 1;
      }
      return cu[(int64_t)lo * k + (e - coff[lo])];
    };
    // position-ordered contiguous ranges per thread
    const uint32_t per = (nall + kThreads - 1) / kThreads;
    const uint32_t e0 = min(nall, (uint32_t)tid * per);
    const uint32_t e1 = min(nall, e0 + per);
    if ((uint32_t)keff == nall) {
      for (uint32_t e = e0; e < e1; ++e) {
        const int pos = (int)elem(e).y;
        R[base + e] = row_of(bt, pos, num_blocks);
        if (U) U[base + e] = pos;
      }
    } else {
      for (int i = tid; i < kHistBins; i += kThreads) hist[i] = 0;
      __syncthreads();
      for (int c = 0; c < nch; ++c)
        for (int i = tid; i < cc[c]; i += kThreads)
          atomicAdd(&hist[cu[(int64_t)c * k + i].x >> kHistBits], 1u);
      __syncthreads();
      find_threshold_bin(hist, (uint32_t)keff, tmp, &sh_bin, &sh_above);
      const uint32_t b1 = (uint32_t)sh_bin;
      uint32_t kneed = (uint32_t)keff - sh_above;
      for (int i = tid; i < kHistBins; i += kThreads) hist[i] = 0;
      __syncthreads();
      for (int c = 0; c < nch; ++c)
        for (int i = tid; i < cc[c]; i += kThreads) {
          const uint32_t u = cu[(int64_t)c * k + i].x;
          if ((u >> kHistBits) == b1) atomicAdd(&hist[u & (kHistBins - 1)], 1u);
        }
      __syncthreads();
      find_threshold_bin(hist, kneed, tmp, &sh_bin, &sh_above);
      const uint32_t T = (b1 << kHistBits) | (uint32_t)sh_bin;
      kneed -= sh_above;
      uint32_t gt = 0, eq = 0;
      for (uint32_t e = e0; e < e1; ++e) {
        const uint32_t u = elem(e).x;
        gt += u > T;
        eq += u == T;
      }
      uint32_t tot;
      uint32_t above = wg_exclusive_scan<kThreads>(gt, tmp, &tot);
      uint32_t rank = wg_exclusive_scan<kThreads>(eq, tmp, &tot);
      for (uint32_t e = e0; e < e1; ++e) {
        const uint2 v = elem(e);
        int slot = -1;
        if (v.x > T) {
          slot = (int)(above + (rank < kneed ? rank : kneed));
          ++above;
        } else if (v.x == T) {
          if (rank < kneed) slot = (int)(above + rank);
          ++rank;
        }
        if (slot >= 0) {
          const int pos = (int)v.y;
          R[base + slot] = row_of(bt, pos, num_blocks);
          if (U) U[base + slot] = pos;
        }
      }
    }
  }
  if (tid == 0) {
    cnt[unit] = total;
    if (user_cnt) user_cnt[unit] = total;
  }
}

} // namespace

hipError_t launch_merge(const DecodeDims &d, const uint2 *cand,
                        const int32_t *cand_cnt, const int32_t *seq_lens,
                        const int32_t *block_table, int32_t *rows,
                        int32_t *cnt, int32_t *user_sel, int32_t *user_cnt,
                        hipStream_t stream) {
  if (d.nchunks > kMaxChunks) return hipErrorInvalidValue;
  hipLaunchKernelGGL(merge_kernel, dim3(d.B * d.Hkv), dim3(kThreads), 0,
                     stream, cand, cand_cnt, d.nchunks, seq_lens, d.n_max,
                     block_table, d.max_blocks, d.num_blocks, d.Hkv, d.k, d.w,
                     d.sigma, d.cap, rows, cnt, user_sel, user_cnt);
  return hipGetLastError();
}

} // namespace dkv
