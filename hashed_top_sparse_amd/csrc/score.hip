// score.hip -- code-domain score of every cached key, with an exact
// chunk-local top-k so that only candidates leave the chip.
//
// [SPHERICAL KV, §2.1]: logits come straight from the stored radius and the
// packed angle code; no dense key is rebuilt.  [DeepSeek, "starting from
// DSA"]: a light indexer scores every cached key against the query.
//   s_h = sum_j q8_hj * (bit_j ? +1 : -1)  for the G heads of a KV group,
//   S   = r8 * max_h s_h                    (exact integer, |S| < 2^23).
//
// Work: one workgroup per (sequence, KV head, chunk of 512 pages = 8192
// keys).  Each wave streams 64-page groups: one coalesced 256 B (b = 128)
// code load per page (lane L reads dword L of the page's code block, which
// is word L/16 of the key in slot L%16), the page's 16 radius bytes, and one
// 16x16x128 fp8 x fp4 matrix-core op per 128 code bits:
//   - the code word is expanded to fp4 with 5 bit operations: nibble values
//     0.5/1/2/0.5 for bits j = 4e+m, m = 0..3 (masks 0x1.., 0x2.., 0x4..,
//     and (w >> 3) & 0x1..);
//   - the query operand (qprep.hip) holds 2*hi/f_m and 2*lo/f_m per head,
//     so the result rows give 2*D_hi and 2*D_lo - Q exactly (the
//     accumulator starts at -Q in the low rows);
//   - s_h = 16*row(2h) + row(2h+1); max over the group's heads with one or
//     two lane swaps; S = r8 * max in fp32 (exact below 2^24).
// Biased scores u = S + 2^23 of the chunk stay in LDS.
//
// Chunk top-k ([DASH-KV Top-K pruning]): the global top-k of a (sequence,
// KV head) is contained in the union of the chunks' top-k, so each chunk
// keeps only min(k, #candidates) candidates of [sinks, N - window), chosen
// exactly by (u desc, position asc): two 12-bit radix histogram passes in
// LDS find the threshold score T and the number of ties at T to keep; a
// workgroup scan then writes the survivors in position order.
//
// Workgroup order is XCD-aware: the Hkv workgroups of one (sequence, chunk)
// get ids congruent mod 8 (same XCD, so the page's shared radius line and
// block-table entries are served by one L2) and consecutive in dispatch.
#include "internal.h"

namespace dkv {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr uint32_t kBias = 1u << 23;
constexpr int kHistBits = 12;
constexpr int kHistBins = 1 << kHistBits;
constexpr int kUnroll = 8; // pages in flight per wave

__device__ __forceinline__ v8i expand_code_word(uint32_t w) {
  v8i r;
  r[0] = (int)(w & 0x11111111u);
  r[1] = (int)(w & 0x22222222u);
  r[2] = (int)(w & 0x44444444u);
  r[3] = (int)((w >> 3) & 0x11111111u);
  r[4] = r[5] = r[6] = r[7] = 0;
  return r;
}

// Finds, scanning bins from the top, the bin where the running count
// reaches kneed: count(bins above) < kneed <= count(bins above) + bin.
// Results land in *out_bin / *out_above (LDS); ends with a barrier.
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

template <int KS, int G>
__global__ __launch_bounds__(kThreads) void score_chunk_kernel(
    const uint32_t *__restrict__ codes, const uint8_t *__restrict__ radii,
    int64_t num_blocks, const int32_t *__restrict__ block_table,
    int max_blocks, const int32_t *__restrict__ seq_lens, int n_max,
    const uint32_t *__restrict__ qop, const float *__restrict__ qneg, int B,
    int Hkv, int W, int nchunks, int k, int w, int sigma,
    uint2 *__restrict__ cand, int32_t *__restrict__ cand_cnt,
    int32_t *__restrict__ scores_out, int score_stride) {
  __shared__ uint32_t su[kChunkKeys];
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t tmp[kWaves];
  __shared__ int sh_bin;
  __shared__ uint32_t sh_above;

  // XCD-aware decode of the workgroup id.
  const int wid = blockIdx.x;
  const int xcd = wid & 7, j = wid >> 3;
  const int sc = (j / Hkv) * 8 + xcd;
  const int g = j % Hkv;
  if (sc >= B * nchunks) return;
  const int s = sc / nchunks, c = sc % nchunks;
  const int unit = s * Hkv + g;
  const int N = seq_len_clamped(seq_lens, s, n_max);
  const int npages = (N + kPage - 1) / kPage;
  const int p_begin = c * kChunkPages;
  if (p_begin >= npages) return; // this chunk does not exist for s
  const int p_end = min(npages, p_begin + kChunkPages);
  const int key0 = p_begin * kPage;
  const int key_end = min(N, p_end * kPage);
  const int lo = max(sigma, key0), hi = min(N - w, key_end);
  const int ncand = max(0, hi - lo);
  const bool want_scores = scores_out != nullptr;
  int32_t *cnt_out = cand_cnt + (int64_t)unit * nchunks + c;
  if (ncand == 0 && !want_scores) {
    if (threadIdx.x == 0) *cnt_out = 0;
    return;
  }

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int Hq = Hkv * G;
  v8i aop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint4 *src = reinterpret_cast<const uint4 *>(
        qop + (((int64_t)unit * KS + ks) * 64 + lane) * 8);
    const uint4 x0 = src[0], x1 = src[1];
    aop[ks][0] = (int)x0.x; aop[ks][1] = (int)x0.y;
    aop[ks][2] = (int)x0.z; aop[ks][3] = (int)x0.w;
    aop[ks][4] = (int)x1.x; aop[ks][5] = (int)x1.y;
    aop[ks][6] = (int)x1.z; aop[ks][7] = (int)x1.w;
  }
  v4f cinit = {0.f, 0.f, 0.f, 0.f};
  {
    const int h0 = 2 * (lane >> 4), h1 = h0 + 1;
    const float *qn = qneg + (int64_t)s * Hq + (int64_t)g * G;
    if (h0 < G) cinit[1] = qn[h0];
    if (h1 < G) cinit[3] = qn[h1];
  }

  const int32_t *bt = block_table + (int64_t)s * max_blocks;
  const int code_dwords = W * kPage; // per (page, head)
  for (int pg0 = p_begin + wave * 64; pg0 < p_end; pg0 += kWaves * 64) {
    const int npg = min(64, p_end - pg0);
    const int my_blk = lane < npg ? bt[pg0 + lane] : -1;
    for (int jb = 0; jb < npg; jb += kUnroll) {
      uint32_t cw[kUnroll][KS];
      uint32_t r8[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int jj = jb + u;
        const int blk = __builtin_amdgcn_readlane(my_blk, jj < 64 ? jj : 63);
        const bool ok = jj < npg && blk >= 0 && blk < num_blocks;
        const int64_t base = ((int64_t)(ok ? blk : 0) * Hkv + g);
        const uint32_t *cp = codes + base * code_dwords;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int dw = 64 * ks + lane;
          cw[u][ks] = (ok && dw < code_dwords) ? cp[dw] : 0u;
        }
        r8[u] = (ok && lane < kPage) ? (uint32_t)radii[base * kPage + lane] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int jj = jb + u;
        if (jj >= npg) break;
        v4f acc = cinit;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              aop[ks], expand_code_word(cw[u][ks]), acc, 0, 4, 0, 127, 0, 127);
        const float s0 = 16.f * acc[0] + acc[1];
        float m = s0;
        if (G >= 2) m = fmaxf(s0, 16.f * acc[2] + acc[3]);
        if (G >= 4) m = fmaxf(m, __shfl_xor(m, 16));
        if (G >= 8) m = fmaxf(m, __shfl_xor(m, 32));
        const float S = (float)r8[u] * m;
        if (lane < kPage) {
          const int idx = (pg0 + jj - p_begin) * kPage + lane;
          const int Si = (int)S;
          su[idx] = (uint32_t)(Si + (int)kBias);
          if (want_scores && key0 + idx < N)
            scores_out[(int64_t)unit * score_stride + key0 + idx] = Si;
        }
      }
    }
  }
  __syncthreads();

  // ---- exact top-k of the chunk's candidates [lo, hi)
  const int klo = lo - key0, khi = hi - key0;
  const int kc = min(k, ncand);
  uint2 *out = cand + ((int64_t)unit * nchunks + c) * (int64_t)k;
  if (kc == ncand) {
    for (int i = threadIdx.x; i < ncand; i += kThreads)
      out[i] = make_uint2(su[klo + i], (uint32_t)(key0 + klo + i));
  } else if (kc > 0) {
    for (int i = threadIdx.x; i < kHistBins; i += kThreads) hist[i] = 0;
    __syncthreads();
    for (int i = klo + threadIdx.x; i < khi; i += kThreads)
      atomicAdd(&hist[su[i] >> kHistBits], 1u);
    __syncthreads();
    find_threshold_bin(hist, (uint32_t)kc, tmp, &sh_bin, &sh_above);
    const uint32_t b1 = (uint32_t)sh_bin;
    uint32_t kneed = (uint32_t)kc - sh_above;
    for (int i = threadIdx.x; i < kHistBins; i += kThreads) hist[i] = 0;
    __syncthreads();
    for (int i = klo + threadIdx.x; i < khi; i += kThreads) {
      const uint32_t u = su[i];
      if ((u >> kHistBits) == b1) atomicAdd(&hist[u & (kHistBins - 1)], 1u);
    }
    __syncthreads();
    find_threshold_bin(hist, kneed, tmp, &sh_bin, &sh_above);
    const uint32_t T = (b1 << kHistBits) | (uint32_t)sh_bin;
    kneed -= sh_above;
    // position-ordered compaction over contiguous per-thread ranges
    const int per = (ncand + kThreads - 1) / kThreads;
    const int i0 = min(khi, klo + (int)threadIdx.x * per);
    const int i1 = min(khi, i0 + per);
    uint32_t gt = 0, eq = 0;
    for (int i = i0; i < i1; ++i) {
      const uint32_t u = su[i];
      gt += u > T;
      eq += u == T;
    }
    uint32_t tot;
    uint32_t above = wg_exclusive_scan<kThreads>(gt, tmp, &tot);
    uint32_t rank = wg_exclusive_scan<kThreads>(eq, tmp, &tot);
    for (int i = i0; i < i1; ++i) {
      const uint32_t u = su[i];
      if (u > T) {
        const uint32_t taken = rank < kneed ? rank : kneed;
        out[above + taken] = make_uint2(u, (uint32_t)(key0 + i));
        ++above;
      } else if (u == T) {
        if (rank < kneed) out[above + rank] = make_uint2(u, (uint32_t)(key0 + i));
        ++rank;
      }
    }
  }
  if (threadIdx.x == 0) *cnt_out = kc;
}

} // namespace

hipError_t launch_score(const DecodeDims &d, const uint32_t *codes,
                        const uint8_t *radii, const int32_t *block_table,
                        const int32_t *seq_lens, const uint32_t *qop,
                        const float *qneg, uint2 *cand, int32_t *cand_cnt,
                        int32_t *scores_out, hipStream_t stream) {
  if (d.nchunks == 0) return hipSuccess;
  const int64_t sc = (int64_t)d.B * d.nchunks;
  const int64_t groups = (sc + 7) / 8;
  const int64_t nwg = groups * 8 * d.Hkv;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  dim3 grid((unsigned)nwg);
#define DKV_SCORE_CASE(KSV, GV)                                                \
  if (d.KS == KSV && d.G == GV) {                                              \
    hipLaunchKernelGGL((score_chunk_kernel<KSV, GV>), grid, dim3(kThreads), 0, \
                       stream, codes, radii, d.num_blocks, block_table,        \
                       d.max_blocks, seq_lens, d.n_max, qop, qneg, d.B, d.Hkv, \
                       d.W, d.nchunks, d.k, d.w, d.sigma, cand, cand_cnt,      \
                       scores_out, d.max_seq_len);                             \
    return hipGetLastError();                                                  \
  }
  DKV_SCORE_CASE(1, 1)
  DKV_SCORE_CASE(1, 2)
  DKV_SCORE_CASE(1, 4)
  DKV_SCORE_CASE(1, 8)
  DKV_SCORE_CASE(2, 1)
  DKV_SCORE_CASE(2, 2)
  DKV_SCORE_CASE(2, 4)
  DKV_SCORE_CASE(2, 8)
#undef DKV_SCORE_CASE
  return hipErrorInvalidValue;
}

} // namespace dkv
