// score.hip -- code-domain score of every cached key in one streaming pass;
// keys reaching the (sequence, KV head)'s candidate threshold L leave the
// chip as (biased score, position) candidates.
//
// [SPHERICAL KV, §2.1]: the logit comes straight from the stored radius and
// the packed angle code, no dense key rebuilt; [DeepSeek, "starting from
// DSA"]: a light indexer scores every cached key.  The per-page scoring is
// in score_common.h (one fp8 x fp4 matrix-core op per 128 code bits).
//
// Work: persistent waves (4 per workgroup, up to 4 workgroups per CU),
// each streaming a static stride of 64-page tasks (sequence, page group, KV
// head); task ids run KV head fastest, then sequence, then page group, so
// the heads of one page block are read together.  A wave's code pages go to
// an 8 KB ring in LDS by direct buffer-to-LDS loads of 1 KB (one page quad
// for 128-bit codes: lanes 16j..16j+15 fetch page j's 256 bytes, each lane
// at its own page address), issued a ring ahead; each task's 64 radius
// lines arrive the same way in one 1 KB load, double-buffered.  Each page
// quad is scored from the ring (four matrix-core ops, results gathered into
// one register: page j in lanes 16j..16j+15), and its ring slot is refilled
// at once with the quad one ring further on (the next task's quads once the
// current task's are all issued).  The 1024 biased scores of a task stay in
// 16 registers; its candidates (positions in [sinks, N - window) with
// u >= L) go, compacted by ballots in position order, to the task's own
// region of the candidate buffer (room for every key of the group, so no
// atomics and no overflow), and the task's count beside it.  A task always
// issues the same number of stores, all lanes active (kTaskStores: one per
// score row, the lanes without a candidate writing to the region's last
// slot, which is read only when every key is a candidate, plus the count),
// so both the ring waits and the compiler's own wait counts include them.
#include <algorithm>
#include <type_traits>

#include "score_common.h"

namespace dkv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTaskQuads = kGroupPages / 4;  // page quads per task
constexpr int kRingBytes = 8192;             // code ring per wave
constexpr int kRadBytes = 1024;              // radius lines of one task
constexpr uint32_t kRadiusOob = 0x80000000u; // past any radius buffer
constexpr int kTaskStores = kTaskQuads + 1;  // stores issued per task

// Buffer-to-LDS loads are invisible to the compiler's wait-count
// tracking: a read of a ring slot must first wait until at most `n` vector
// memory operations are outstanding, n being a lower bound on the number
// issued after the slot's own loads (loads complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm_at_most() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [I0, N).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// One LDS round trip per page quad, as a single asm block that also waits
// for its results (the compiler cannot order reads of the ring against the
// buffer-to-LDS loads; the explicit vmcnt wait before it does):
//   - the page byte offsets of the KS refill loads (ds_bpermute of the
//     refilled task's per-page offsets; `lp4` = 4 * page of this lane within
//     a load, OFFB = 4 * first page of the refill);
//   - this lane's code word of each page and K-step of ring slot SLOT (page
//     p, K-step ks at word 64*(KS*p + ks) + lane; `base` = ring byte address
//     + 4*lane);
//   - its radius byte (key lane&15 of page 4*Q + lane>>4; `rbase` = radius
//     buffer byte address + lane).
template <int KS, int SLOT, int Q, int OFFB>
__device__ __forceinline__ void read_quad(uint32_t base, uint32_t rbase,
                                          uint32_t lp4, uint32_t page_off,
                                          uint32_t (&cw)[4][KS], uint32_t &r8,
                                          uint32_t (&vo)[KS]) {
  constexpr int o = 4 * KS * SLOT; // in 256-byte units
  if constexpr (KS == 1) {
    uint64_t a, b;
    asm volatile(
        "ds_bpermute_b32 %3, %6, %7 offset:%8\n\t"
        "ds_read2st64_b32 %0, %4 offset0:%9 offset1:%10\n\t"
        "ds_read2st64_b32 %1, %4 offset0:%11 offset1:%12\n\t"
        "ds_read_u8 %2, %5 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a), "=&v"(b), "=&v"(r8), "=&v"(vo[0])
        : "v"(base), "v"(rbase), "v"(lp4), "v"(page_off), "n"(OFFB), "n"(o),
          "n"(o + 1), "n"(o + 2), "n"(o + 3), "n"(64 * Q)
        : "memory");
    cw[0][0] = (uint32_t)a;
    cw[1][0] = (uint32_t)(a >> 32);
    cw[2][0] = (uint32_t)b;
    cw[3][0] = (uint32_t)(b >> 32);
  } else {
    static_assert(KS == 2, "K-steps");
    uint64_t a, b, c, d;
    asm volatile(
        "ds_bpermute_b32 %5, %9, %10 offset:%11\n\t"
        "ds_bpermute_b32 %6, %9, %10 offset:%12\n\t"
        "ds_read2st64_b32 %0, %7 offset0:%13 offset1:%14\n\t"
        "ds_read2st64_b32 %1, %7 offset0:%15 offset1:%16\n\t"
        "ds_read2st64_b32 %2, %7 offset0:%17 offset1:%18\n\t"
        "ds_read2st64_b32 %3, %7 offset0:%19 offset1:%20\n\t"
        "ds_read_u8 %4, %8 offset:%21\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d), "=&v"(r8), "=&v"(vo[0]),
          "=&v"(vo[1])
        : "v"(base), "v"(rbase), "v"(lp4), "v"(page_off), "n"(OFFB),
          "n"(OFFB + 8), "n"(o), "n"(o + 1), "n"(o + 2), "n"(o + 3), "n"(o + 4),
          "n"(o + 5), "n"(o + 6), "n"(o + 7), "n"(64 * Q)
        : "memory");
    cw[0][0] = (uint32_t)a; cw[0][1] = (uint32_t)(a >> 32);
    cw[1][0] = (uint32_t)b; cw[1][1] = (uint32_t)(b >> 32);
    cw[2][0] = (uint32_t)c; cw[2][1] = (uint32_t)(c >> 32);
    cw[3][0] = (uint32_t)d; cw[3][1] = (uint32_t)(d >> 32);
  }
}

// An empty use of a register value: the compiler waits for its load here
// (32-bit operands only, which the host pass of the compiler also accepts).
__device__ __forceinline__ void mark_loaded(uint32_t x) { asm volatile("" ::"v"(x)); }

// One 1 KB buffer-to-LDS load: lane L's 16 bytes at voff land at lds + 16*L.
__device__ __forceinline__ void load_kb_to_lds(__amdgpu_buffer_rsrc_t rsrc,
                                               uint32_t *lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void *)lds, 16, (int)voff, 0, 0, 0);
}

// One task of the stream (all fields wave-uniform); unit < 0: none.
struct Task {
  int s, g, grp, unit, N, key0, npg, lo, hi;
};

template <int KS, int G>
__global__ __launch_bounds__(kThreads) void filter_kernel(
    const uint32_t *__restrict__ codes, const uint8_t *__restrict__ radii,
    int64_t num_blocks, uint32_t code_bytes, uint32_t radius_bytes,
    const int32_t *__restrict__ block_table, int max_blocks,
    const int32_t *__restrict__ seq_lens, int n_max,
    const uint32_t *__restrict__ qop, const float *__restrict__ qneg,
    const uint32_t *__restrict__ lthr, int B, int Hkv, int W, int ngroups,
    int ntasks, int w, int sigma, uint2 *__restrict__ cand,
    uint32_t *__restrict__ tcount, int cand_groups,
    int32_t *__restrict__ scores_out, int score_stride) {
  constexpr int kQuadBytes = 1024 * KS;
  constexpr int kRingQuads = kRingBytes / kQuadBytes;
  // vector memory operations issued after a ring quad's loads, at least:
  // the other ring quads' loads, and the previous task's stores when the
  // quad was loaded during the previous task
  constexpr int kAfterSame = (kRingQuads - 1) * KS;
  constexpr int kAfterCross = kAfterSame + kTaskStores;
  static_assert(kAfterCross < 64, "vmcnt is 6 bits");
  static_assert(kRingQuads <= kTaskQuads && kTaskQuads % kRingQuads == 0, "ring");
  __shared__ __attribute__((aligned(16))) uint32_t ring[kWaves][kRingBytes / 4];
  __shared__ __attribute__((aligned(16))) uint32_t rring[kWaves][2][kRadBytes / 4];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int stride = gridDim.x * kWaves;
  const int Hq = Hkv * G;
  uint32_t *myring = ring[wave];
  const uint32_t ring_base =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)myring + 4u * lane;
  // radius halves: the current task's and the next task's
  uint32_t *rad_cur = rring[wave][0], *rad_next = rring[wave][1];
  const PoolView view = make_pool_view(codes, radii, code_bytes, radius_bytes, W,
                                       Hkv, 0, lane);
  const int code_dwords = W * kPage;
  // this lane's page within a 1 KB load and its 16-byte chunk of that page
  // (for 64-bit codes the upper half of each 256-byte slot repeats the page)
  const uint32_t lp4 = (uint32_t)(lane / (16 * KS)) * 4u;
  const uint32_t chunk = 16u * (uint32_t)(lane & (code_dwords / 4 - 1));

  // task id -> task, or none if its page group is past the sequence
  auto decode = [&](int t, Task &T) -> bool {
    T.g = t % Hkv;
    const int r = t / Hkv;
    T.s = r % B;
    T.grp = r / B;
    T.N = seq_len_clamped(seq_lens, T.s, n_max);
    T.key0 = T.grp * kGroupPages * kPage;
    if (T.key0 >= T.N) return false;
    T.unit = T.s * Hkv + T.g;
    T.npg = min(kGroupPages, (T.N - T.key0 + kPage - 1) / kPage);
    T.lo = max(sigma, T.key0);
    T.hi = min(T.N - w, T.key0 + T.npg * kPage);
    return true;
  };
  // the first non-empty task at or after t in this wave's stride
  auto find = [&](int t, Task &T) -> int {
    for (; t < ntasks; t += stride)
      if (decode(t, T)) return t;
    T.unit = -1;
    return ntasks;
  };
  // Lane j: the task's block id of page j (-1 past the task), loaded one
  // task before its offsets are needed so the load is long done by then.
  auto load_blk = [&](const Task &T) -> int {
    int blk = -1;
    if (T.unit >= 0 && lane < T.npg)
      blk = block_table[(int64_t)T.s * max_blocks + T.key0 / kPage + lane];
    return blk;
  };
  // Lane j: byte offsets of page j (code block, radius line); invalid
  // pages read physical page 0's code and a radius of 0.
  auto page_offsets = [&](const Task &T, int blk, uint32_t &code_off,
                          uint32_t &rad_off) {
    const bool ok = blk >= 0 && blk < num_blocks;
    const uint32_t ph = (uint32_t)blk * (uint32_t)Hkv + (uint32_t)T.g;
    code_off = ok ? ph * view.page_code_bytes : 0u;
    rad_off = ok ? ph * (uint32_t)kPage : kRadiusOob;
  };
  auto load_op = [&](const Task &T, QueryOperand<KS> &op, uint32_t &L) {
    const int unit = T.unit >= 0 ? T.unit : 0;
    op = load_query_operand<KS, G>(qop, qneg, unit, unit / Hkv, unit % Hkv, Hq, lane);
    L = lthr[unit];
  };

  Task C, N1;
  int tC = find(blockIdx.x * kWaves + wave, C);
  if (C.unit < 0) return;
  int tN = find(tC + stride, N1);
  uint32_t cC, rC, cN, rN;
  {
    const int blkC = load_blk(C), blkN = load_blk(N1);
    page_offsets(C, blkC, cC, rC);
    page_offsets(N1, blkN, cN, rN);
  }
  QueryOperand<KS> opC;
  uint32_t LC;
  load_op(C, opC, LC);
  // everything above has landed before the stream starts, so no wait in
  // the loop below is ever for a load of this prologue; the empty asm uses
  // tell the compiler so too (it does not read the wait above), otherwise
  // it would wait for them again, behind the whole ring, in every task
  wait_vm_at_most<0>();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int i = 0; i < 8; ++i) mark_loaded((uint32_t)opC.a[ks][i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) mark_loaded(__float_as_uint(opC.cinit[i]));
  mark_loaded(cC);
  mark_loaded(rC);
  mark_loaded(cN);
  mark_loaded(rN);
  load_kb_to_lds(view.radius, rad_cur, rC);
  static_for<0, kRingQuads>([&](auto qc) {
    constexpr int q = decltype(qc)::value;
#pragma unroll
    for (int m = 0; m < KS; ++m) {
      const uint32_t page = 4 * q + m * (4 / KS) + (lane / (16 * KS));
      const uint32_t vo = (uint32_t)__builtin_amdgcn_ds_bpermute((int)page * 4, (int)cC);
      load_kb_to_lds(view.code, myring + (q * kQuadBytes + 1024 * m) / 4, vo + chunk);
    }
  });
  // the stores a finished task would have issued, so that the first task's
  // ring waits count the same operations as every later one (written to the
  // last slot of C's region, which is never read unless C's own candidate
  // writes, issued later by this wave, fill it); written as asm so that
  // exactly kTaskStores store instructions are issued
  {
    const uint64_t dummy = reinterpret_cast<uint64_t>(
        cand + ((int64_t)C.unit * cand_groups + C.grp) * kGroupKeys + (kGroupKeys - 1));
    const uint64_t zero = 0;
#pragma unroll
    for (int r = 0; r < kTaskStores; ++r)
      asm volatile("global_store_dwordx2 %0, %1, off" ::"v"(dummy), "v"(zero)
                   : "memory");
  }

  while (true) {
    // look ahead: the task after next (its block ids) and the next task's
    // query operand
    Task N2 = {0, 0, 0, -1, 0, 0, 0, 0, 0};
    const int tN2 = N1.unit >= 0 ? find(tN + stride, N2) : ntasks;
    if (N1.unit < 0) N2.unit = -1;
    const int blkN2 = load_blk(N2);
    QueryOperand<KS> opN;
    uint32_t LN;
    load_op(N1, opN, LN);
    const uint32_t rad_base =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)rad_cur +
        (uint32_t)lane;

    uint32_t u[kTaskQuads];
    static_for<0, kTaskQuads>([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      constexpr int slot = q % kRingQuads;
      constexpr int tq = q + kRingQuads; // stream position one ring ahead
      constexpr bool next = tq >= kTaskQuads;
      constexpr int rq = next ? tq - kTaskQuads : tq; // refilled task's quad
      // the next task's radius lines go out before its first code
      if constexpr (next && rq == 0) load_kb_to_lds(view.radius, rad_next, rN);
      wait_vm_at_most<(q >= kRingQuads) ? kAfterSame : kAfterCross>();
      uint32_t cw[4][KS], r8, vo[KS];
      read_quad<KS, slot, q, 16 * rq>(ring_base, rad_base, lp4, next ? cN : cC,
                                      cw, r8, vo);
#pragma unroll
      for (int m = 0; m < KS; ++m)
        load_kb_to_lds(view.code, myring + (slot * kQuadBytes + 1024 * m) / 4,
                       vo[m] + chunk);
      const int mx = score_quad_max<KS, G>(opC, cw);
      u[q] = (uint32_t)(__mul24((int)r8, mx) + (int)kScoreBias);
    });

    if (scores_out != nullptr) {
      int32_t *so = scores_out + (int64_t)C.unit * score_stride;
#pragma unroll
      for (int q = 0; q < kTaskQuads; ++q) {
        const int pos = C.key0 + 64 * q + lane;
        if (pos < C.N) so[pos] = (int32_t)(u[q] - kScoreBias);
      }
    }
    // this task's candidates, in position order, to its own region
    {
      const int64_t t_idx = (int64_t)C.unit * cand_groups + C.grp;
      uint2 *reg = cand + t_idx * kGroupKeys;
      uint32_t nc = 0;
#pragma unroll
      for (int r = 0; r < kTaskQuads; ++r) {
        const int pos = C.key0 + r * 64 + lane;
        const bool c = pos >= C.lo && pos < C.hi && u[r] >= LC;
        const uint64_t m = __ballot(c);
        const uint32_t slot = c ? nc + lanes_below(m) : kGroupKeys - 1;
        reg[slot] = make_uint2(u[r], (uint32_t)pos);
        nc += __popcll(m);
      }
      tcount[t_idx] = nc;
    }

    // rotate the stream
    if (N1.unit < 0) break;
    C = N1;
    tC = tN;
    cC = cN;
    rC = rN;
    opC = opN;
    LC = LN;
    N1 = N2;
    tN = tN2;
    page_offsets(N2, blkN2, cN, rN);
    uint32_t *t = rad_cur;
    rad_cur = rad_next;
    rad_next = t;
  }
  // no buffer-to-LDS load may still be in flight when the wave ends
  wait_vm_at_most<0>();
}

} // namespace

hipError_t launch_score(const DecodeDims &d, const uint32_t *codes,
                        const uint8_t *radii, const int32_t *block_table,
                        const int32_t *seq_lens, const uint32_t *qop,
                        const float *qneg, const uint32_t *lthr, uint2 *cand,
                        uint32_t *tcount, int32_t *scores_out,
                        hipStream_t stream) {
  const int pages = (d.n_max + kPage - 1) / kPage;
  const int64_t ngroups = (pages + kGroupPages - 1) / kGroupPages;
  if (ngroups == 0) return hipSuccess;
  const int64_t ntasks = (int64_t)d.B * ngroups * d.Hkv;
  if (ntasks > 0x7FFFFFFF - 65536) return hipErrorInvalidValue;
  const uint32_t code_bytes = (uint32_t)((uint64_t)d.num_blocks * d.Hkv * d.W * kPage * 4);
  const uint32_t radius_bytes = (uint32_t)((uint64_t)d.num_blocks * d.Hkv * kPage);
  // persistent grid: as many workgroups as fit in a CU's LDS
  constexpr int kLdsPerWg = kWaves * (kRingBytes + 2 * kRadBytes);
  const int wg_per_cu = std::max(1, std::min(8, kLdsPerCu / kLdsPerWg));
  const int64_t nwg = std::min<int64_t>((ntasks + kWaves - 1) / kWaves,
                                        (int64_t)wg_per_cu * device_cu_count());
#define DKV_SCORE_CASE(KSV, GV)                                                \
  if (d.KS == KSV && d.G == GV) {                                              \
    hipLaunchKernelGGL((filter_kernel<KSV, GV>), dim3((unsigned)nwg),          \
                       dim3(kThreads), 0, stream, codes, radii, d.num_blocks,  \
                       code_bytes, radius_bytes, block_table, d.max_blocks,    \
                       seq_lens, d.n_max, qop, qneg, lthr, d.B, d.Hkv, d.W,    \
                       (int)ngroups, (int)ntasks, d.w, d.sigma, cand, tcount,  \
                       d.cand_groups, scores_out, d.max_seq_len);              \
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
