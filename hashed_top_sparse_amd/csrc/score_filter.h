// score_filter.h -- code-domain score of every cached key in one streaming
// pass; keys reaching the (sequence, KV head)'s candidate threshold L leave
// the chip as (biased score, position) candidates -- or, for page-granular
// selection, pages as (best biased score of their candidate keys, page).
// The kernel template and its launcher are instantiated in the score_*.hip
// files, one per (radius weight, selection granularity), so they compile
// side by side.
//
// [SPHERICAL KV, §2.1]: the logit comes straight from the stored radius and
// the packed angle code, no dense key rebuilt; [DeepSeek, "starting from
// DSA"]: a light indexer scores every cached key.  The per-page scoring is
// in score_common.h (one fp8 x fp4 matrix-core op per 128 code bits).
//
// Work: persistent waves (4 per workgroup), each streaming a static stride
// of 64-page tasks (sequence, page group, KV head).  The (sequence, page
// group) pairs that hold keys come from a list the prep kernel writes, so
// ragged batches spread evenly; task ids run KV head fastest over that
// list, so the heads of one page block are read together.  Codes are key-major, so one 16-byte load per lane
// brings a page quad: lanes 16j..16j+15 read page j's 16 keys (each lane a
// whole 128-bit key; 64-bit keys use 8-byte loads, 256-bit keys two loads).
// Four gfx950 row swaps (v_permlane32_swap, v_permlane16_swap) transpose
// that into the matrix-core operand of each page (lane L: word L/16 of key
// L%16).  Each lane also loads one radius byte per quad.  A wave keeps
// kDepth quads of loads in flight in registers (the compiler's own wait
// counts order them), continuing into the next task; the block ids of the
// task after next are loaded one task ahead.  Candidates (positions in
// [sinks, N - window) with u >= L) are compacted per quad by ballots, in
// position order, into the task's own region of the candidate buffer (room
// for every key of the group, so no atomics and no overflow), and the
// task's count is written beside it.
#pragma once

#include <algorithm>
#include <type_traits>

#include "score_common.h"

namespace dkv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTaskQuads = kGroupPages / 4; // page quads per task
// quads of loads in flight per wave: 8 KB per wave for 128- and 256-bit
// codes (a 256-bit quad is 2 KB), 4 KB for 64-bit codes (at most half a
// task ahead)
template <int W>
constexpr int kDepthFor = W > 4 ? 4 : 8;
// quad of a task at which the task after next and the next task's operand
// are loaded: kDepth quads before the next task's first prefetch
template <int W>
constexpr int kLookaheadFor = kTaskQuads - 2 * kDepthFor<W>;
// Workgroups per CU: one wave per SIMD each, three waves per SIMD in all
// (up to 168 registers a lane).  Three waves with 8 KB in flight each beat
// four with 4 KB (the register budget of four per SIMD): 62.4 vs 63.7 us on
// 16 x 128K keys, although the task count then divides less evenly.
constexpr int kWgPerCu = 3;
// per-wave candidate list: kCandList entries, then one spare entry per lane
// (8 KB of LDS in all)
constexpr int kCandList = kGroupKeys - 64;
constexpr int kTaskTable = 16;        // tasks recorded before a forced write

// Compile-time loop: f(std::integral_constant<int, I>) for I in [I0, N).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// One task of the stream (all fields wave-uniform); unit < 0: none.
struct Task {
  int s, g, grp, unit, N, key0, npg, lo, hi;
};

// Loaded code words of one page quad: lane 16j+c holds the KS*4 words of
// key c of page j (words 4ks..4ks+3 in d[ks]).
template <int KS>
struct QuadLoad {
  uint32_t d[KS][4];
};

// An empty use of a register value: the compiler waits for its load here
// (32-bit operands only, which the host pass of the compiler also accepts).
__device__ __forceinline__ void mark_loaded(uint32_t x) { asm volatile("" ::"v"(x)); }

// W: code words per key (2, 4 or 8); KS: 128-bit matrix-core K-steps;
// DBG: also write every score to scores_out (inspection builds only); LIN:
// linear radius weight (looked up in a per-workgroup LDS table); PAGES:
// candidates are pages (the best score of their keys in [lo, hi)).
template <int W, int G, bool DBG, bool LIN, bool PAGES, int KS = (W > 4 ? W / 4 : 1)>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8))) void filter_kernel(
    const uint32_t *__restrict__ codes, const uint8_t *__restrict__ radii,
    int64_t num_blocks, uint32_t code_bytes, uint32_t radius_bytes,
    const int32_t *__restrict__ block_table, int max_blocks,
    const uint32_t *__restrict__ tasks, int n_max,
    const uint32_t *__restrict__ qop, const float *__restrict__ qneg,
    const uint32_t *__restrict__ lthr, int B, int Hkv, int max_entries,
    int w, int sigma, uint2 *__restrict__ cand,
    uint32_t *__restrict__ tcount, int cand_groups,
    int32_t *__restrict__ scores_out, int score_stride, int round_wgs) {
  constexpr int kDepth = kDepthFor<W>;
  constexpr int kLookahead = kLookaheadFor<W>;
  static_assert(kTaskQuads % kDepth == 0 && kTaskQuads >= 2 * kDepth, "prefetch rounds");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // linear radius weights of the 256 codes (before any wave can leave)
  __shared__ uint16_t wlut[LIN ? 256 : 1];
  if constexpr (LIN) {
    for (int i = threadIdx.x; i < 256; i += kThreads)
      wlut[i] = (uint16_t)radius_weight_linear((uint32_t)i);
    __syncthreads();
  }
  const int Hq = Hkv * G;
  const __amdgpu_buffer_rsrc_t code_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t *>(codes), 0, code_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rad_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(radii), 0, radius_bytes, kBufferWord3);
  // Sequence lengths and thresholds are read with vector loads: a scalar
  // load in the stream would make every wait on the LDS counter a full wait
  // (scalar loads complete out of order), including the candidate writes.
  const __amdgpu_buffer_rsrc_t task_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t *>(tasks), 0, 16u + 16u * (uint32_t)max_entries, kBufferWord3);
  const __amdgpu_buffer_rsrc_t thr_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t *>(lthr), 0, (uint32_t)(B * Hkv) * 4u, kBufferWord3);
  const uint32_t page_bytes = (uint32_t)(kPage * W * 4);
  // physical page id past the pools: its code and radius loads read 0
  const uint32_t ph_none = (uint32_t)(num_blocks * Hkv);
  const uint32_t key_byte = (uint32_t)((lane & 15) * W * 4);
  const int row = lane >> 4;
  // per-wave tables of the current and the next task's page ids (lane j
  // writes page j), read back per page quad by row: one LDS read per quad
  __shared__ uint32_t ptab[kWaves][2][kGroupPages];
  uint32_t *tabC = ptab[wave][0], *tab1 = ptab[wave][1];
  // the current task's radius lines (16 bytes per page, page order), and
  // its candidates staged before they are written out
  __shared__ __attribute__((aligned(16))) uint8_t rtab[kWaves][kGroupKeys];
  // The wave's candidates, (u, index in the task), kept in LDS until the
  // wave has streamed all its tasks, then written out with the counts: a
  // global store inside the stream would hold up the completion of every
  // load issued after it (one in-order counter covers loads and stores).
  // Per task: (region, first position, entries in the list, count).  A
  // task that finds the list full writes the rest of its candidates to its
  // region at once (rare).
  __shared__ uint2 cstage[kWaves][kCandList + 64];
  __shared__ uint32_t ttab[kWaves][kTaskTable][4];
  uint8_t *radC = rtab[wave];
  uint2 *cst = cstage[wave];
  uint32_t (*tt)[4] = ttab[wave];
  uint32_t used = 0;  // list entries in use
  int ntab = 0;       // tasks recorded
  // Writes every recorded task's listed candidates and its count.  Lanes
  // past a task's list length repeat its last entry (same bytes, same slot).
  auto flush_all = [&]() {
    uint32_t start = 0;
    for (int k = 0; k < ntab; ++k) {
      const uint32_t t_idx = tt[k][0], key0 = tt[k][1], nbuf = tt[k][2], ncount = tt[k][3];
      uint2 *reg = cand + (int64_t)t_idx * kGroupKeys;
      for (uint32_t e0 = 0; e0 < nbuf; e0 += 64) {
        const uint32_t e = min(e0 + (uint32_t)lane, nbuf - 1);
        const uint2 v = cst[start + e];
        // key lists hold raw scores: biased here, once per candidate
        reg[e] = make_uint2(PAGES ? v.x : v.x + kScoreBias, key0 + v.y);
      }
      if (lane == 0) tcount[t_idx] = ncount;
      start += nbuf;
    }
    used = 0;
    ntab = 0;
  };

  // The task list: tasks[0] entries, entry e (16 bytes at byte 16 + 16 e)
  // one page group that holds keys, (sequence, group, length); task id
  // t = e * Hkv + KV head.  Every entry is real work, so the static stride
  // below gives each wave the same number of tasks (up to one) whatever the
  // sequence lengths.
  const int ntasks = min(__builtin_amdgcn_readfirstlane(
                             __builtin_amdgcn_raw_buffer_load_b32(task_rsrc, 0, 0, 0)),
                         (uint32_t)max_entries) * Hkv;
  // The wave's task entries, 64 at a time in registers: lane j holds the
  // entry of the wave's task kbase + j (task id first + (kbase + j) *
  // stride).  They are loaded before the stream starts, so decoding a task
  // inside the stream waits for no load (a load used at once would also
  // wait for every load issued before it: the stream's prefetch).
  //
  // The wave's tasks are first, first + stride, ... below tend.  With one
  // round of workgroups per CU (round_wgs each), the waves of a SIMD issue
  // oldest first: the first workgroup placed on a CU streams fastest and
  // the last slowest (on 16 x 128K keys with equal shares, 44, 47 and 56 us
  // to the end on average, the last alone at the end).  So the rounds
  // share the task list 13 : 10 : 8 per wave, oldest first: round 0 takes
  // the first n0 * Wr tasks, round 1 the next n1 * Wr, round 2 the rest,
  // each with the stride Wr (its waves), so the four waves of a workgroup
  // still read four KV heads of the same page block side by side.
  static_assert(kWgPerCu == 3, "three dispatch rounds");
  int first = blockIdx.x * kWaves + wave, stride = gridDim.x * kWaves, tend = ntasks;
  if (round_wgs > 0) {
    const int Wr = round_wgs * kWaves;
    const int64_t den = (int64_t)31 * Wr;
    const int n0 = (int)(((int64_t)ntasks * 13 + den / 2) / den);
    const int n1 = (int)(((int64_t)ntasks * 10 + den / 2) / den);
    if (n0 >= 1) { // (few tasks: one stride over all waves)
      const int c0 = min(ntasks, n0 * Wr);
      const int c1 = min(ntasks - c0, n1 * Wr);
      const int r = min((int)blockIdx.x / round_wgs, 2);
      first = (r == 0 ? 0 : (r == 1 ? c0 : c0 + c1)) +
              ((int)blockIdx.x - r * round_wgs) * kWaves + wave;
      tend = r == 0 ? c0 : (r == 1 ? c0 + c1 : ntasks);
      stride = Wr;
    }
  }
  int kbase = 0;
  uint32_t te0 = 0, te1 = 0, te2 = 0;
  auto load_entries = [&](int kb) {
    const int t = first + (kb + lane) * stride;
    const int e = min(t, max(ntasks - 1, 0)) / Hkv; // clamped to a listed entry
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(task_rsrc, 16 + 16 * e, 0, 0);
    te0 = v[0];
    te1 = v[1];
    te2 = v[2];
    // used here, so no later read waits for this load
    mark_loaded(te0);
    mark_loaded(te1);
    mark_loaded(te2);
    kbase = kb;
  };
  load_entries(0);
  // task id (first + k * stride) -> task, or none if it holds no keys
  auto decode = [&](int t, Task &T) -> bool {
    T.g = t % Hkv;
    const int kk = (t - first) / stride;
    if (kk - kbase >= 64) load_entries(kk & ~63); // (more than 64 tasks a wave)
    const int l = kk - kbase;
    T.s = (int)__builtin_amdgcn_readlane(te0, l);
    T.grp = (int)__builtin_amdgcn_readlane(te1, l);
    T.N = clamp_int((int)__builtin_amdgcn_readlane(te2, l), 0, n_max);
    T.key0 = T.grp * kGroupKeys;
    if (T.key0 >= T.N || T.s >= B) return false;
    T.unit = T.s * Hkv + T.g;
    T.npg = min(kGroupPages, (T.N - T.key0 + kPage - 1) / kPage);
    T.lo = max(sigma, T.key0);
    T.hi = max(T.lo, min(T.N - w, T.key0 + T.npg * kPage)); // empty: hi == lo
    return true;
  };
  // the first non-empty task at or after t in this wave's stride
  auto find = [&](int t, Task &T) {
    for (; t < tend; t += stride)
      if (decode(t, T)) return t;
    T.unit = -1;
    return tend;
  };
  // Lane j: physical page id (page block index) of the task's page j, or
  // ph_none past the task or for an invalid block id.
  auto load_pages = [&](const Task &T) -> int {
    int blk = -1;
    if (T.unit >= 0 && lane < T.npg)
      blk = block_table[(int64_t)T.s * max_blocks + T.key0 / kPage + lane];
    return blk;
  };
  auto page_ids = [&](const Task &T, int blk) -> uint32_t {
    return (blk >= 0 && blk < num_blocks) ? (uint32_t)blk * (uint32_t)Hkv + (uint32_t)T.g
                                          : ph_none;
  };
  auto load_op = [&](const Task &T, QueryOperandRaw<KS> &op, uint32_t &L) {
    const int unit = T.unit >= 0 ? T.unit : 0;
    load_query_operand_raw<KS, G>(qop, qneg, unit, unit / Hkv, unit % Hkv, Hq, lane, op);
    L = __builtin_amdgcn_raw_buffer_load_b32(thr_rsrc, unit * 4, 0, 0); // uniform
  };
  // Loads a page quad; `mine` is the page id of this lane's page (page
  // lane>>4 of the quad).
  auto load_quad = [&](uint32_t mine, QuadLoad<KS> &ql) {
    const int voff = (int)(mine * page_bytes + key_byte);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (W == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(code_rsrc, voff, 0, 0);
        ql.d[ks][0] = v[0];
        ql.d[ks][1] = v[1];
        ql.d[ks][2] = 0u;
        ql.d[ks][3] = 0u;
      } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(code_rsrc, voff + 16 * ks, 0, 0);
        ql.d[ks][0] = v[0];
        ql.d[ks][1] = v[1];
        ql.d[ks][2] = v[2];
        ql.d[ks][3] = v[3];
      }
    }
  };

  // ---- prologue: the first task, its successor, their page ids, operand
  Task C, T1;
  const int tC = find(first, C);
  if (C.unit < 0) return;
  int t1 = find(tC + stride, T1);
  tabC[lane] = page_ids(C, load_pages(C));
  tab1[lane] = page_ids(T1, load_pages(T1));
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  QueryOperand<KS> opC;
  uint32_t LC;
  int LCs; // LC as a signed score: S >= LCs iff S + 2^31 >= LC
  {
    QueryOperandRaw<KS> raw;
    load_op(C, raw, LC);
    opC = finish_query_operand<KS, G>(raw, lane);
  }
  // The loop below carries opC; uses here make the compiler wait for its
  // loads now, before the stream starts, instead of (merging this path into
  // the loop head) in every task.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int i = 0; i < 8; ++i) mark_loaded((uint32_t)opC.a[ks][i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) mark_loaded(__float_as_uint(opC.cinit[i]));
  LCs = (int)(LC ^ kScoreBias);
  // radius lines: lane j loads page j's 16 bytes (a task ahead of use)
  auto load_radius = [&](uint32_t ph) -> uint4 {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rad_rsrc, (int)(ph * (uint32_t)kPage), 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  auto store_radius = [&](const uint4 &v) {
    *reinterpret_cast<uint4 *>(radC + 16 * lane) = v;
  };
  store_radius(load_radius(tabC[lane]));
  uint4 radN = load_radius(tab1[lane]);
  QuadLoad<KS> buf[kDepth];
  static_for<0, kDepth>([&](auto qc) {
    constexpr int q = decltype(qc)::value;
    load_quad(tabC[4 * q + row], buf[q]);
  });
  // LDS values of the current quad (see run_task)
  uint32_t r8c = radC[lane];
  uint32_t refc = tabC[4 * kDepth + row];

  // One task: score C's 16 quads while prefetching, then rotate the stream.
  // The first call is peeled off the loop so that the loop head is only
  // entered in the state a task leaves (the compiler's wait counts at the
  // loop head then match the steady state).
  auto run_task = [&]() -> bool {
    Task T2 = {0, 0, 0, -1, 0, 0, 0, 0, 0};
    int t2 = tend;
    int blk2 = -1; // raw block ids, turned into page ids one task later
    QueryOperandRaw<KS> op1;
    uint32_t L1 = 0;
    const int64_t t_idx = (int64_t)C.unit * cand_groups + C.grp;
    // first position (page, for PAGES) of the task: list entries hold
    // their index relative to it
    const uint32_t cbase = PAGES ? (uint32_t)(C.key0 / kPage) : (uint32_t)C.key0;
    // pos - lo of this lane's key in quad q is lrel + 64 q (one add a quad)
    const uint32_t lrel = (uint32_t)(lane + C.key0 - C.lo);
    const uint32_t nrange = (uint32_t)(C.hi - C.lo);
    uint2 *reg = cand + t_idx * kGroupKeys;
    uint32_t nc = 0; // the task's candidates so far
    // Scores quad q of C from its loaded words x (transposed here) and the
    // radius weights, and returns its candidates: the entry (cu, cidx) of
    // this lane, whether it is one (isc), and the wave's mask of them.
    struct QuadCand {
      uint32_t cu, cidx;
      bool isc;
      uint64_t m;
    };
    auto quad_cands = [&](int q, uint32_t (&x)[KS][4], int wgt) -> QuadCand {
      uint32_t cw[4][KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        transpose_rows(x[ks]);
#pragma unroll
        for (int j = 0; j < 4; ++j) cw[j][ks] = x[ks][j];
      }
      // (256-bit codes: the pages one after another, which needs fewer
      // registers)
      const int mx = KS > 1 ? score_quad_max_seq<KS, G>(opC, cw) : score_quad_max<KS, G>(opC, cw);
      const int Sv = __mul24(wgt, mx);
      const uint32_t u = biased_score(Sv);
      const int pos = C.key0 + 64 * q + lane;
      if constexpr (DBG) {
        if (pos < C.N)
          scores_out[(int64_t)C.unit * score_stride + pos] = (int32_t)(u - kScoreBias);
      }
      // A candidate: position in [lo, hi) and u >= L, each test one compare
      // (the range one on pos - lo, unsigned, as lrel + 64 q).
      const bool inr = lrel + (uint32_t)(64 * q) < nrange;
      QuadCand c;
      // PAGES: the first lane of each 16-lane row stands for its page, with
      // the best u of the page's keys in [lo, hi) (0: none there).  Keys:
      // the raw score, compared signed with the threshold and biased when
      // the list is written out.
      c.cu = PAGES ? row_max16(inr ? u : 0u) : (uint32_t)Sv;
      const bool pass = PAGES ? c.cu >= LC : Sv >= LCs;
      c.cidx = PAGES ? (uint32_t)(4 * q + (lane >> 4)) : (uint32_t)(64 * q + lane);
      c.isc = PAGES ? ((lane & 15) == 0 && c.cu != 0u && pass) : (inr && pass);
      c.m = PAGES ? __ballot(c.cu != 0u) & __ballot(pass) & kRowHeads
                  : __ballot(inr) & __ballot(pass);
      return c;
    };
    static_for<0, kTaskQuads>([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      constexpr int slot = q % kDepth;
      if constexpr (q == kLookahead) {
        // the task after next (its page ids, used one task from now) and
        // the next task's operand (used from the next task's first quad)
        if (T1.unit >= 0) t2 = find(t1 + stride, T2);
        blk2 = load_pages(T2);
        load_op(T1, op1, L1);
      }
      // ---- score quad q of C
      uint32_t x[KS][4];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[ks][i] = buf[slot].d[ks][i];
      // radius byte of key lane&15 of page 4q + lane>>4, and the page id
      // of the refill below, both read from LDS one quad ahead
      const uint32_t r8 = r8c;
      // its weight (LIN: an LDS read issued before the next quad's reads)
      const int wgt = LIN ? (int)wlut[r8] : (int)r8;
      // ---- refill the slot: the quad kDepth further on (C's, or T1's
      // first ones)
      load_quad(refc, buf[slot]);
      // ---- the next quad's LDS reads, before this quad's candidate write
      // (LDS operations complete in order)
      if constexpr (q + 1 < kTaskQuads) {
        r8c = radC[64 * (q + 1) + lane];
        refc = (q + 1 + kDepth < kTaskQuads) ? tabC[4 * (q + 1 + kDepth) + row]
                                            : tab1[4 * (q + 1 + kDepth - kTaskQuads) + row];
      }
      const QuadCand c = quad_cands(q, x, wgt);
      const uint32_t lslot = __builtin_amdgcn_mbcnt_hi(
          (uint32_t)(c.m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)c.m, used + nc));
      // Every lane writes (a branch around the write would leave the
      // compiler unsure whether it was issued, and every later LDS wait
      // would then wait for it): lanes without a listed candidate write
      // their spare entry.  An address-space-qualified pointer keeps this an
      // LDS store (a flat store would count against the vector-memory wait
      // counter).  A candidate past the list's end is left out here and
      // written by the rescoring below, so the quads of a task form one
      // branch-free block that the compiler can interleave.
      const uint32_t wslot =
          (c.isc && lslot < (uint32_t)kCandList) ? lslot : (uint32_t)(kCandList + lane);
      ((__attribute__((address_space(3))) uint64_t *)cst)[wslot] =
          ((uint64_t)c.cidx << 32) | c.cu;
      nc += (uint32_t)__popcll(c.m);
    });
    // A task with more candidates than the list had room for (rare): its
    // quads are scored again, from the same page ids, radius lines and
    // operand, and the candidates past the room go straight to the task's
    // region, at their rank in position order.
    const uint32_t room = (uint32_t)kCandList - used;
    if (nc > room) {
      uint32_t nc2 = 0;
      for (int q = 0; q < kTaskQuads; ++q) {
        QuadLoad<KS> ql;
        load_quad(tabC[4 * q + row], ql);
        const uint32_t r8 = radC[64 * q + lane];
        const int wgt = LIN ? (int)wlut[r8] : (int)r8;
        uint32_t x[KS][4];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[ks][i] = ql.d[ks][i];
        const QuadCand c = quad_cands(q, x, wgt);
        const uint32_t rank = __builtin_amdgcn_mbcnt_hi(
            (uint32_t)(c.m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)c.m, nc2));
        if (c.isc && rank >= room)
          reg[rank] = make_uint2(PAGES ? c.cu : c.cu + kScoreBias, cbase + c.cidx);
        nc2 += (uint32_t)__popcll(c.m);
      }
    }
    // record the task: its first min(nc, room) candidates are in the list
    {
      const uint32_t nbuf = min(nc, (uint32_t)kCandList - used);
      if (lane == 0) {
        tt[ntab][0] = (uint32_t)t_idx;
        tt[ntab][1] = cbase;
        tt[ntab][2] = nbuf;
        tt[ntab][3] = nc;
      }
      used += nbuf;
      ++ntab;
      if (ntab == kTaskTable) flush_all(); // many tasks per wave (rare)
    }

    // rotate the stream
    if (T1.unit < 0) return false;
    C = T1;
    opC = finish_query_operand<KS, G>(op1, lane);
    LC = L1;
    LCs = (int)(LC ^ kScoreBias);
    T1 = T2;
    t1 = t2;
    {
      uint32_t *t = tabC;
      tabC = tab1;
      tab1 = t;
    }
    // the old current table is no longer read: T2's page ids go there
    tab1[lane] = page_ids(T2, blk2);
    // the new current task's radius lines (loaded a task ago) into LDS, and
    // the new next task's lines requested
    store_radius(radN);
    radN = load_radius(tab1[lane]);
    r8c = radC[lane];
    refc = tabC[4 * kDepth + row];
    return true;
  };
  if (run_task())
    while (run_task()) {
    }
  flush_all();
}

template <bool LIN, bool PAGES>
hipError_t launch_filter_impl(const DecodeDims &d, const uint32_t *codes,
                         const uint8_t *radii, const int32_t *block_table,
                         const uint32_t *tasks, const uint32_t *qop,
                         const float *qneg, const uint32_t *lthr, uint2 *cand,
                         uint32_t *tcount, int32_t *scores_out,
                         hipStream_t stream) {
  const int pages = (d.n_max + kPage - 1) / kPage;
  const int64_t ngroups = (pages + kGroupPages - 1) / kGroupPages;
  if (ngroups == 0) return hipSuccess;
  // at most one task list entry per (sequence, page group)
  const int64_t max_entries = (int64_t)d.B * ngroups;
  const int64_t ntasks = max_entries * d.Hkv;
  if (ntasks > 0x7FFFFFFF - 65536 || max_entries >= ((int64_t)1 << 27))
    return hipErrorInvalidValue;
  const uint32_t code_bytes = (uint32_t)((uint64_t)d.num_blocks * d.Hkv * d.W * kPage * 4);
  const uint32_t radius_bytes = (uint32_t)((uint64_t)d.num_blocks * d.Hkv * kPage);
#define DKV_SCORE_LAUNCH(WV, GV, DV)                                           \
  {                                                                            \
    const int ncu = device_cu_count();                                         \
    const int64_t nwg = std::min<int64_t>((ntasks + kWaves - 1) / kWaves,       \
                                          (int64_t)kWgPerCu * ncu);            \
    hipLaunchKernelGGL((filter_kernel<WV, GV, DV, LIN, PAGES>),                \
                       dim3((unsigned)nwg), dim3(kThreads), 0, stream, codes,  \
                       radii, d.num_blocks, code_bytes, radius_bytes,          \
                       block_table, d.max_blocks, tasks, d.n_max, qop,         \
                       qneg, lthr, d.B, d.Hkv, (int)max_entries, d.w,          \
                       d.sigma, cand, tcount, d.cand_groups, scores_out,       \
                       d.max_seq_len,                                          \
                       nwg == (int64_t)kWgPerCu * ncu ? ncu : 0);              \
    return hipGetLastError();                                                  \
  }
#define DKV_SCORE_CASE(WV, GV)                                                 \
  if (d.W == WV && d.G == GV) {                                                \
    if (scores_out != nullptr) DKV_SCORE_LAUNCH(WV, GV, true)                  \
    DKV_SCORE_LAUNCH(WV, GV, false)                                            \
  }
  DKV_SCORE_CASE(2, 1)
  DKV_SCORE_CASE(2, 2)
  DKV_SCORE_CASE(2, 4)
  DKV_SCORE_CASE(2, 8)
  DKV_SCORE_CASE(4, 1)
  DKV_SCORE_CASE(4, 2)
  DKV_SCORE_CASE(4, 4)
  DKV_SCORE_CASE(4, 8)
  DKV_SCORE_CASE(8, 1)
  DKV_SCORE_CASE(8, 2)
  DKV_SCORE_CASE(8, 4)
  DKV_SCORE_CASE(8, 8)
#undef DKV_SCORE_CASE
#undef DKV_SCORE_LAUNCH
  return hipErrorInvalidValue;
}

} // namespace
} // namespace dkv
