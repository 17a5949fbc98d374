// score.hip -- code-domain score of every cached key in one streaming pass;
// keys reaching the (sequence, KV head)'s candidate threshold L leave the
// chip as (biased score, position) candidates.
//
// [SPHERICAL KV, §2.1]: the logit comes straight from the stored radius and
// the packed angle code, no dense key rebuilt; [DeepSeek, "starting from
// DSA"]: a light indexer scores every cached key.  The per-page scoring is
// in score_common.h (one fp8 x fp4 matrix-core op per 128 code bits).
//
// Work: one wave per (sequence, 64-page group, KV head); the 8 waves of a
// workgroup are consecutive KV heads of the same pages (for Hkv = 8: all of
// them), so a page's radius line and block-table entries are shared in one
// CU.  Each wave streams its 64 pages straight-line with two 8-page batches
// of buffer loads in flight, scores them four pages at a time (the four
// pages' results are gathered into one register, page j in lanes
// 16j..16j+15, so the epilogue and the radius load run once for 64 keys),
// keeps the 1024 biased scores in its own LDS
// slice, then appends the candidates (positions in [sinks, N - window) with
// u >= L) to the (sequence, KV head)'s list with one atomic add: ballots
// give each lane its place, in position order within the wave.  The list
// holds at most `cap` entries; the counter still counts every candidate, so
// an overflow is visible to the merge, which then rescans exactly.
#include "score_common.h"

namespace dkv {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kGroupPages = 64;
constexpr int kBatch = 8; // pages per load batch (two batches in flight)

template <int KS>
struct PageBatch {
  uint32_t cw[2][4][KS]; // two quads of pages
  uint32_t r8[2];        // radius of key (lane & 15) of page (lane >> 4)
};

template <int KS, int G>
__global__ __launch_bounds__(kThreads) void filter_kernel(
    const uint32_t *__restrict__ codes, const uint8_t *__restrict__ radii,
    int64_t num_blocks, uint32_t code_bytes, uint32_t radius_bytes,
    const int32_t *__restrict__ block_table, int max_blocks,
    const int32_t *__restrict__ seq_lens, int n_max,
    const uint32_t *__restrict__ qop, const float *__restrict__ qneg,
    const uint32_t *__restrict__ lthr, int B, int Hkv, int W, int ngroups,
    int w, int sigma, uint32_t *__restrict__ counter,
    uint32_t *__restrict__ cand_u, int32_t *__restrict__ cand_pos, int cap,
    int32_t *__restrict__ scores_out, int score_stride) {
  __shared__ uint32_t su[kWaves][kGroupPages * kPage];
  const int lane = threadIdx.x & 63;
  // wave-uniform (keeps the page offsets below in scalar registers)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t task = (int64_t)blockIdx.x * kWaves + wave;
  const int g = (int)(task % Hkv);
  const int64_t sg = task / Hkv;
  const int grp = (int)(sg % ngroups);
  const int s = (int)(sg / ngroups);
  if (s >= B) return;
  const int N = seq_len_clamped(seq_lens, s, n_max);
  const int npages = (N + kPage - 1) / kPage;
  const int pg0 = grp * kGroupPages;
  if (pg0 >= npages) return;
  const int npg = min(kGroupPages, npages - pg0);
  const int key0 = pg0 * kPage;
  const int lo = max(sigma, key0), hi = min(N - w, key0 + npg * kPage);
  if (hi <= lo && scores_out == nullptr) return; // no candidates in this group
  const int unit = s * Hkv + g;
  const int Hq = Hkv * G;

  const QueryOperand<KS> op = load_query_operand<KS, G>(qop, qneg, unit, s, g, Hq, lane);
  const uint32_t L = lthr[unit];
  const PoolView view = make_pool_view(codes, radii, code_bytes, radius_bytes, W,
                                       Hkv, g, lane);
  // Lane j holds page pg0 + j's byte offsets: its code block, and its radius
  // line (past the end of the radius buffer for an invalid page or one past
  // the sequence, so its radius loads as 0 and its score is 0).  Invalid
  // pages read the code block of physical page 0; it is multiplied by 0.
  uint32_t my_code_off = 0, my_rad_off = 0x80000000u;
  {
    const int blk = lane < npg ? block_table[(int64_t)s * max_blocks + pg0 + lane] : -1;
    if (blk >= 0 && blk < num_blocks) {
      const uint32_t ph = (uint32_t)blk * (uint32_t)Hkv + (uint32_t)g;
      my_code_off = ph * view.page_code_bytes;
      my_rad_off = ph * (uint32_t)kPage;
    }
  }
  // ds_bpermute byte address of lane (quad page of this lane) + 4 * quad
  const int rad_src = (lane >> 4) * 4;
  uint32_t *mys = su[wave];

  auto load_batch = [&](int jb, PageBatch<KS> &pb) {
#pragma unroll
    for (int q4 = 0; q4 < 2; ++q4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t soff = __builtin_amdgcn_readlane(my_code_off, jb + 4 * q4 + j);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          pb.cw[q4][j][ks] = __builtin_amdgcn_raw_buffer_load_b32(
              view.code, view.code_voff + 256 * ks, soff, 0);
      }
      // one radius byte per lane: key (lane & 15) of page (lane >> 4)
      const uint32_t roff = (uint32_t)__builtin_amdgcn_ds_bpermute(
          rad_src + 4 * (jb + 4 * q4), (int)my_rad_off);
      pb.r8[q4] = __builtin_amdgcn_raw_buffer_load_b8(
          view.radius, (int)(roff + (uint32_t)view.radius_voff), 0, 0);
    }
  };
  auto score_batch = [&](int jb, const PageBatch<KS> &pb) {
#pragma unroll
    for (int q4 = 0; q4 < 2; ++q4) {
      const int m = score_quad_max<KS, G>(op, pb.cw[q4]);
      mys[(jb + 4 * q4) * kPage + lane] =
          (uint32_t)(__mul24((int)pb.r8[q4], m) + (int)kScoreBias);
    }
  };
  // Straight-line over the group's 64 pages (pages past npg score 0 and are
  // ignored), so the wait counters stay exact and one batch's loads are in
  // flight while the other batch is scored.
  {
    PageBatch<KS> pa, pb;
    load_batch(0, pa);
#pragma unroll
    for (int jb = 0; jb < kGroupPages; jb += 2 * kBatch) {
      load_batch(jb + kBatch, pb);
      score_batch(jb, pa);
      if (jb + 2 * kBatch < kGroupPages) load_batch(jb + 2 * kBatch, pa);
      score_batch(jb + kBatch, pb);
    }
  }
  // the wave's own LDS writes must be visible to all its lanes
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (scores_out != nullptr) {
    int32_t *so = scores_out + (int64_t)unit * score_stride;
    for (int e = lane; e < npg * kPage && key0 + e < N; e += 64)
      so[key0 + e] = (int32_t)(mys[e] - kScoreBias);
  }
  if (hi <= lo) return;

  // candidates of this group: positions in [lo, hi) with u >= L
  constexpr int kRows = kGroupPages * kPage / 64;
  uint32_t total = 0;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int pos = key0 + r * 64 + lane;
    const bool cand = pos >= lo && pos < hi && mys[r * 64 + lane] >= L;
    total += __popcll(__ballot(cand));
  }
  if (total == 0) return;
  uint32_t base = 0;
  if (lane == 0) base = atomicAdd(&counter[unit], total);
  base = __builtin_amdgcn_readfirstlane(base);
  uint32_t *ou = cand_u + (int64_t)unit * cap;
  int32_t *op_ = cand_pos + (int64_t)unit * cap;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int pos = key0 + r * 64 + lane;
    const uint32_t u = mys[r * 64 + lane];
    const bool cand = pos >= lo && pos < hi && u >= L;
    const uint64_t m = __ballot(cand);
    const uint32_t slot = base + lanes_below(m);
    if (cand && slot < (uint32_t)cap) {
      ou[slot] = u;
      op_[slot] = pos;
    }
    base += __popcll(m);
  }
}

} // namespace

hipError_t launch_score(const DecodeDims &d, const uint32_t *codes,
                        const uint8_t *radii, const int32_t *block_table,
                        const int32_t *seq_lens, const uint32_t *qop,
                        const float *qneg, const uint32_t *lthr,
                        uint32_t *counter, uint32_t *cand_u, int32_t *cand_pos,
                        int32_t *scores_out, hipStream_t stream) {
  const int pages = (d.n_max + kPage - 1) / kPage;
  const int ngroups = (pages + kGroupPages - 1) / kGroupPages;
  if (ngroups == 0) return hipSuccess;
  const uint32_t code_bytes = (uint32_t)((uint64_t)d.num_blocks * d.Hkv * d.W * kPage * 4);
  const uint32_t radius_bytes = (uint32_t)((uint64_t)d.num_blocks * d.Hkv * kPage);
  const int64_t tasks = (int64_t)d.B * ngroups * d.Hkv;
  const int64_t nwg = (tasks + kWaves - 1) / kWaves;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
#define DKV_SCORE_CASE(KSV, GV)                                                \
  if (d.KS == KSV && d.G == GV) {                                              \
    hipLaunchKernelGGL((filter_kernel<KSV, GV>), dim3((unsigned)nwg),          \
                       dim3(kThreads), 0, stream, codes, radii, d.num_blocks,  \
                       code_bytes, radius_bytes, block_table, d.max_blocks,    \
                       seq_lens, d.n_max, qop, qneg, lthr, d.B, d.Hkv, d.W,    \
                       ngroups, d.w, d.sigma, counter, cand_u, cand_pos,       \
                       d.cand_cap, scores_out, d.max_seq_len);                 \
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
