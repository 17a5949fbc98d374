// score_select.hip -- code-domain scores of every cached key and the
// per-(sequence, KV head) selection.
//
// Score ([SPHERICAL KV §2.1]: logits from the radius and the angle code, no
// dense key rebuilt; [DeepSeek DSA]: a light indexer scores all history):
//   s_h = sum_j q8_hj * (bit_j ? +1 : -1) for each query head of the group,
//   S   = r8 * max_h s_h                    (exact int32, |S| < 2^23).
// Selection ([DASH-KV Top-K pruning]; [DeepSeek CSA]: sliding window;
// [DySCO FAQ 3]: attention sinks):
//   sinks [0, min(sigma,N)), window [max(min(sigma,N), N-w), N) and the top
//   min(k, |C|) of C = [sigma, N-w) ordered by (S desc, position asc).
//   The order is made unique by the key (S + 2^23, position): an exact
//   radix select on the 24-bit score finds the threshold score T, every
//   candidate above T is taken, and the ties at T are taken in position
//   order.
#include "internal.h"

namespace dkv {
namespace {

constexpr int kScoreThreads = 256; // 16 pages x 16 slots
constexpr int kSelThreads = 1024;
constexpr uint32_t kScoreBias = 1u << 23;

__global__ __launch_bounds__(kScoreThreads) void score_kernel(
    const uint32_t *__restrict__ codes, const uint8_t *__restrict__ radii,
    int64_t num_blocks, const int32_t *__restrict__ block_table,
    int max_blocks, const int32_t *__restrict__ seq_lens, int n_max,
    const int8_t *__restrict__ q8, int32_t *__restrict__ scores,
    int score_stride, int Hq, int Hkv, int G, int b) {
  const int s = blockIdx.z, g = blockIdx.y;
  __shared__ int sq[8 * 256];
  const int8_t *qg = q8 + ((int64_t)s * Hq + (int64_t)g * G) * b;
  for (int i = threadIdx.x; i < G * b; i += kScoreThreads) sq[i] = qg[i];
  __syncthreads();
  const int N = seq_len_clamped(seq_lens, s, n_max);
  const int page = blockIdx.x * (kScoreThreads / kPage) + threadIdx.x / kPage;
  const int slot = threadIdx.x % kPage;
  const int pos = page * kPage + slot;
  if (pos >= N) return;
  const int blk = block_table[(int64_t)s * max_blocks + page];
  int32_t S = 0;
  if (blk >= 0 && blk < num_blocks) {
    const int W = b / 32;
    const uint32_t *cw = codes + ((int64_t)blk * Hkv + g) * W * kPage + slot;
    uint32_t words[8];
    for (int w = 0; w < W; ++w) words[w] = cw[w * kPage];
    const int r8 = radii[((int64_t)blk * Hkv + g) * kPage + slot];
    int best = 0;
    for (int h = 0; h < G; ++h) {
      int acc = 0;
      for (int j = 0; j < b; ++j) {
        const int qv = sq[h * b + j];
        acc += ((words[j >> 5] >> (j & 31)) & 1u) ? qv : -qv;
      }
      best = (h == 0 || acc > best) ? acc : best;
    }
    S = r8 * best;
  }
  scores[((int64_t)s * Hkv + g) * score_stride + pos] = S;
}

// One workgroup per (sequence, KV head).
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const int32_t *__restrict__ scores, int score_stride,
    const int32_t *__restrict__ seq_lens, int n_max, int Hkv, int k, int w,
    int sigma, int cap, int32_t *__restrict__ sel, int32_t *__restrict__ cnt,
    int32_t *__restrict__ user_sel, int32_t *__restrict__ user_cnt) {
  const int unit = blockIdx.x;
  const int s = unit / Hkv;
  const int tid = threadIdx.x;
  const int N = seq_len_clamped(seq_lens, s, n_max);
  const int ns = sigma < N ? sigma : N;
  const int ws = (N - w > ns) ? N - w : ns;
  const int nwin = N - ws;
  const int c0 = sigma;
  const int nc = (N - w - sigma) > 0 ? (N - w - sigma) : 0;
  const int keff = k < nc ? k : nc;
  const int total = ns + nwin + keff;
  int32_t *L = sel + (int64_t)unit * cap;
  const int32_t *S = scores + (int64_t)unit * score_stride + c0;

  for (int i = tid; i < ns + nwin; i += kSelThreads)
    L[i] = i < ns ? i : ws + (i - ns);
  for (int i = total + tid; i < cap; i += kSelThreads) L[i] = -1;
  const int base = ns + nwin;

  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_prefix, sh_kneed;
  __shared__ uint32_t tie_count[kSelThreads];
  __shared__ uint32_t gt_count[kSelThreads];

  if (keff > 0 && keff == nc) {
    for (int i = tid; i < nc; i += kSelThreads) L[base + i] = c0 + i;
  } else if (keff > 0) {
    uint32_t prefix = 0, mask = 0, kneed = (uint32_t)keff;
    for (int shift = 16; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < nc; i += kSelThreads) {
        const uint32_t u = (uint32_t)S[i] + kScoreBias;
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        uint32_t cum = 0;
        for (int dg = 255; dg >= 0; --dg) {
          const uint32_t c = hist[dg];
          if (cum + c >= kneed) {
            prefix |= (uint32_t)dg << shift;
            kneed -= cum;
            break;
          }
          cum += c;
        }
        sh_prefix = prefix;
        sh_kneed = kneed;
      }
      __syncthreads();
      prefix = sh_prefix;
      kneed = sh_kneed;
      mask |= 255u << shift;
      __syncthreads();
    }
    const uint32_t T = prefix;
    // Candidates above T and the first kneed ties at T are written in
    // position order (deterministic list): contiguous ranges per thread,
    // exclusive scans of the per-thread counts.
    const int chunk = (nc + kSelThreads - 1) / kSelThreads;
    const int i0 = tid * chunk;
    const int i1 = (i0 + chunk < nc) ? i0 + chunk : nc;
    uint32_t gt = 0, ties = 0;
    for (int i = i0; i < i1; ++i) {
      const uint32_t u = (uint32_t)S[i] + kScoreBias;
      gt += u > T;
      ties += u == T;
    }
    gt_count[tid] = gt;
    tie_count[tid] = ties;
    __syncthreads();
    if (tid == 0) {
      uint32_t run_gt = 0, run_tie = 0;
      for (int t = 0; t < kSelThreads; ++t) {
        const uint32_t a = gt_count[t], c = tie_count[t];
        gt_count[t] = run_gt;
        tie_count[t] = run_tie;
        run_gt += a;
        run_tie += c;
      }
    }
    __syncthreads();
    uint32_t rank = tie_count[tid];
    uint32_t above = gt_count[tid];
    // merged order: a tie of rank r (< kneed) precedes every candidate above
    // T that comes after it, so the output position is (#above before it) +
    // (#taken ties before it).
    for (int i = i0; i < i1; ++i) {
      const uint32_t u = (uint32_t)S[i] + kScoreBias;
      if (u > T) {
        const uint32_t taken = rank < kneed ? rank : kneed;
        L[base + above + taken] = c0 + i;
        ++above;
      } else if (u == T) {
        if (rank < kneed) L[base + above + rank] = c0 + i;
        ++rank;
      }
    }
  }
  if (tid == 0) cnt[unit] = total;
  if (user_sel != nullptr || user_cnt != nullptr) {
    __syncthreads();
    if (user_sel != nullptr)
      for (int i = tid; i < cap; i += kSelThreads)
        user_sel[(int64_t)unit * cap + i] = L[i];
    if (user_cnt != nullptr && tid == 0) user_cnt[unit] = total;
  }
}

} // namespace

hipError_t launch_score(const DecodeDims &d, const uint32_t *codes,
                        const uint8_t *radii, const int32_t *block_table,
                        const int32_t *seq_lens, const int8_t *q8,
                        int32_t *scores, hipStream_t stream) {
  const int pages = (d.n_max + kPage - 1) / kPage;
  const int per_wg = kScoreThreads / kPage;
  if (pages == 0) return hipSuccess;
  dim3 grid((pages + per_wg - 1) / per_wg, d.Hkv, d.B);
  hipLaunchKernelGGL(score_kernel, grid, dim3(kScoreThreads), 0, stream,
                     codes, radii, d.num_blocks, block_table, d.max_blocks,
                     seq_lens, d.n_max, q8, scores, d.max_seq_len, d.Hq, d.Hkv,
                     d.G, d.b);
  return hipGetLastError();
}

hipError_t launch_select(const DecodeDims &d, const int32_t *scores,
                         const int32_t *seq_lens, int32_t *sel, int32_t *cnt,
                         int32_t *user_sel, int32_t *user_cnt,
                         hipStream_t stream) {
  hipLaunchKernelGGL(select_kernel, dim3(d.B * d.Hkv), dim3(kSelThreads), 0,
                     stream, scores, d.max_seq_len, seq_lens, d.n_max, d.Hkv,
                     d.k, d.w, d.sigma, d.cap, sel, cnt, user_sel, user_cnt);
  return hipGetLastError();
}

} // namespace dkv
