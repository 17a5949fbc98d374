// score.hip -- code-domain score of every cached key in one streaming pass;
// keys reaching the (sequence, KV head)'s candidate threshold L leave the
// chip as (biased score, position) candidates.
//
// [SPHERICAL KV, §2.1]: the logit comes straight from the stored radius and
// the packed angle code, no dense key rebuilt; [DeepSeek, "starting from
// DSA"]: a light indexer scores every cached key.  The per-page scoring is
// in score_common.h (one fp8 x fp4 matrix-core op per 128 code bits).
//
// Work: persistent waves (4 per workgroup, 2 workgroups per CU), each
// streaming a static stride of 64-page tasks (sequence, page group, KV
// head); task ids run KV head fastest, then sequence, then page group, so
// the waves working at any one time spread over every (sequence, KV head)
// counter, and the heads of one page block are read together.  The code
// pages of a wave, and their radius lines, go to a 17 KB ring in LDS by
// direct buffer-to-LDS loads issued a full ring ahead (about 60 loads,
// 15 KB, in flight per wave).  Each page quad is scored from the
// ring (four matrix-core ops, results gathered into one register: page j
// in lanes 16j..16j+15) and the ring slot is refilled at once with the
// page one ring further on (the next task's pages once the current task's
// are all issued).  The 1024 biased scores of a task stay in 16 registers;
// its candidates (positions in [sinks, N - window) with u >= L) are
// counted by ballots and reserved with one atomic add on the (sequence,
// KV head) counter, and written out one task later, so the atomic's round
// trip overlaps the next task's stream.  The list holds at most `cap`
// entries; the counter still counts every candidate, so an overflow is
// visible to the merge, which then rescans exactly.
#include <algorithm>
#include <type_traits>

#include "score_common.h"

namespace dkv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kGroupPages = 64;              // pages per task
constexpr int kTaskQuads = kGroupPages / 4;  // page quads per task
constexpr int kRingDwords = 4096;            // 16 KB code ring per wave
constexpr int kRadRingDwords = 256;          // radius lines of up to 16 quads
constexpr uint32_t kRadiusOob = 0x80000000u; // past any radius buffer

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

// Reads ring quad slot SLOT: this lane's code word of each page and K-step
// (page p, K-step ks at word 64*(KS*p + ks) + lane; `base` = ring byte
// address + 4*lane) and its radius byte (key lane&15 of page lane>>4;
// `rbase` = radius ring byte address + lane).  Written as one asm block
// that also waits for the reads: the compiler cannot order these reads
// against the buffer-to-LDS loads, the explicit wait above does.
template <int KS, int SLOT>
__device__ __forceinline__ void read_quad(uint32_t base, uint32_t rbase,
                                          uint32_t (&cw)[4][KS], uint32_t &r8) {
  constexpr int o = 4 * KS * SLOT; // in 256-byte units
  if constexpr (KS == 1) {
    uint64_t a, b;
    asm volatile(
        "ds_read2st64_b32 %0, %3 offset0:%5 offset1:%6\n\t"
        "ds_read2st64_b32 %1, %3 offset0:%7 offset1:%8\n\t"
        "ds_read_u8 %2, %4 offset:%9\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a), "=&v"(b), "=&v"(r8)
        : "v"(base), "v"(rbase), "n"(o), "n"(o + 1), "n"(o + 2), "n"(o + 3),
          "n"(64 * SLOT)
        : "memory");
    cw[0][0] = (uint32_t)a;
    cw[1][0] = (uint32_t)(a >> 32);
    cw[2][0] = (uint32_t)b;
    cw[3][0] = (uint32_t)(b >> 32);
  } else {
    static_assert(KS == 2, "K-steps");
    uint64_t a, b, c, d;
    asm volatile(
        "ds_read2st64_b32 %0, %5 offset0:%7 offset1:%8\n\t"
        "ds_read2st64_b32 %1, %5 offset0:%9 offset1:%10\n\t"
        "ds_read2st64_b32 %2, %5 offset0:%11 offset1:%12\n\t"
        "ds_read2st64_b32 %3, %5 offset0:%13 offset1:%14\n\t"
        "ds_read_u8 %4, %6 offset:%15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d), "=&v"(r8)
        : "v"(base), "v"(rbase), "n"(o), "n"(o + 1), "n"(o + 2), "n"(o + 3),
          "n"(o + 4), "n"(o + 5), "n"(o + 6), "n"(o + 7), "n"(64 * SLOT)
        : "memory");
    cw[0][0] = (uint32_t)a; cw[0][1] = (uint32_t)(a >> 32);
    cw[1][0] = (uint32_t)b; cw[1][1] = (uint32_t)(b >> 32);
    cw[2][0] = (uint32_t)c; cw[2][1] = (uint32_t)(c >> 32);
    cw[3][0] = (uint32_t)d; cw[3][1] = (uint32_t)(d >> 32);
  }
}

// One task of the stream (all fields wave-uniform); unit < 0: none.
struct Task {
  int s, g, unit, N, key0, npg, lo, hi;
};

template <int KS, int G>
__global__ __launch_bounds__(kThreads) void filter_kernel(
    const uint32_t *__restrict__ codes, const uint8_t *__restrict__ radii,
    int64_t num_blocks, uint32_t code_bytes, uint32_t radius_bytes,
    const int32_t *__restrict__ block_table, int max_blocks,
    const int32_t *__restrict__ seq_lens, int n_max,
    const uint32_t *__restrict__ qop, const float *__restrict__ qneg,
    const uint32_t *__restrict__ lthr, int B, int Hkv, int W, int ngroups,
    int ntasks, int w, int sigma, uint32_t *__restrict__ counter,
    uint32_t *__restrict__ cand_u, int32_t *__restrict__ cand_pos, int cap,
    int32_t *__restrict__ scores_out, int score_stride) {
  constexpr int kPageDwords = 64 * KS;
  constexpr int kRingPages = kRingDwords / kPageDwords;
  constexpr int kRingQuads = kRingPages / 4;
  // loads issued after a quad's own: the other ring quads' code and radius
  constexpr int kAfter =
      (kRingQuads - 1) * (4 * KS + 1) < 63 ? (kRingQuads - 1) * (4 * KS + 1) : 63;
  static_assert(kRingQuads <= kTaskQuads && kTaskQuads % kRingQuads == 0, "ring");
  __shared__ __attribute__((aligned(16))) uint32_t ring[kWaves][kRingDwords];
  __shared__ __attribute__((aligned(16))) uint32_t rring[kWaves][kRadRingDwords];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int stride = gridDim.x * kWaves;
  const int Hq = Hkv * G;
  uint32_t *myring = ring[wave];
  uint32_t *myrad = rring[wave];
  // LDS byte addresses of this lane's word in ring slot 0 and its radius byte
  const uint32_t ring_base =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)myring + 4u * lane;
  const uint32_t rad_base =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)myrad + (uint32_t)lane;
  const PoolView view = make_pool_view(codes, radii, code_bytes, radius_bytes, W,
                                       Hkv, 0, lane);

  // task id -> task, or none if its page group is past the sequence
  auto decode = [&](int t, Task &T) -> bool {
    T.g = t % Hkv;
    const int r = t / Hkv;
    T.s = r % B;
    const int grp = r / B;
    T.N = seq_len_clamped(seq_lens, T.s, n_max);
    T.key0 = grp * kGroupPages * kPage;
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
  // Loads quad q of a task into ring quad slot `slot`: per page and K-step
  // one buffer-to-LDS load (lane L's dword lands at slot word L), and one
  // for the quad's four radius lines (lanes 0..15, four bytes each).
  auto issue_quad = [&](uint32_t code_off, uint32_t rad_off, int q, int slot) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t soff = __builtin_amdgcn_readlane(code_off, 4 * q + j);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            view.code,
            (__attribute__((address_space(3))) void *)(myring +
                                                       (4 * slot + j) * kPageDwords +
                                                       64 * ks),
            4, view.code_voff + 256 * ks, soff, 0, 0);
    }
    const uint32_t roff = (uint32_t)__builtin_amdgcn_ds_bpermute(
                              (4 * q + (lane >> 2)) * 4, (int)rad_off) +
                          4u * (uint32_t)(lane & 3);
    if (lane < 16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          view.radius,
          (__attribute__((address_space(3))) void *)(myrad + 16 * slot), 4,
          (int)roff, 0, 0, 0);
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
  // the loop below is ever for a load of this prologue
  wait_vm_at_most<0>();
#pragma unroll
  for (int q = 0; q < kRingQuads; ++q) issue_quad(cC, rC, q, q);
  // an address the compiler cannot prove uniform keeps the atomic add below
  // a single lane-0 operation whose result is read one task later
  uint32_t opaque_zero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(opaque_zero));

  // the previous task, whose candidates are still to be written
  Task P;
  P.unit = -1;
  uint32_t pu[kTaskQuads], p_base = 0, p_total = 0, p_L = 0;

  auto write_previous = [&]() {
    if (P.unit < 0 || p_total == 0) return;
    uint32_t base = __builtin_amdgcn_readfirstlane(p_base);
    uint32_t *ou = cand_u + (int64_t)P.unit * cap;
    int32_t *op_ = cand_pos + (int64_t)P.unit * cap;
#pragma unroll
    for (int r = 0; r < kTaskQuads; ++r) {
      const int pos = P.key0 + r * 64 + lane;
      const bool cand = pos >= P.lo && pos < P.hi && pu[r] >= p_L;
      const uint64_t m = __ballot(cand);
      const uint32_t slot = base + lanes_below(m);
      if (cand && slot < (uint32_t)cap) {
        ou[slot] = pu[r];
        op_[slot] = pos;
      }
      base += __popcll(m);
    }
  };

  while (true) {
    // look ahead: the task after next (its page offsets) and the next
    // task's query operand
    Task N2 = {0, 0, -1, 0, 0, 0, 0, 0};
    const int tN2 = N1.unit >= 0 ? find(tN + stride, N2) : ntasks;
    if (N1.unit < 0) N2.unit = -1;
    const int blkN2 = load_blk(N2);
    QueryOperand<KS> opN;
    uint32_t LN;
    load_op(N1, opN, LN);

    uint32_t u[kTaskQuads];
    static_for<0, kTaskQuads>([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      constexpr int slot = q % kRingQuads;
      wait_vm_at_most<kAfter>();
      uint32_t cw[4][KS], r8;
      read_quad<KS, slot>(ring_base, rad_base, cw, r8);
      constexpr int tq = q + kRingQuads; // stream position one ring ahead
      if constexpr (tq < kTaskQuads)
        issue_quad(cC, rC, tq, slot);
      else
        issue_quad(cN, rN, tq - kTaskQuads, slot);
      const int m = score_quad_max<KS, G>(opC, cw);
      u[q] = (uint32_t)(__mul24((int)r8, m) + (int)kScoreBias);
    });

    if (scores_out != nullptr) {
      int32_t *so = scores_out + (int64_t)C.unit * score_stride;
#pragma unroll
      for (int q = 0; q < kTaskQuads; ++q) {
        const int pos = C.key0 + 64 * q + lane;
        if (pos < C.N) so[pos] = (int32_t)(u[q] - kScoreBias);
      }
    }
    write_previous();
    // count this task's candidates and reserve their slots; the atomic's
    // result is read one task later
    uint32_t total = 0;
#pragma unroll
    for (int r = 0; r < kTaskQuads; ++r) {
      const int pos = C.key0 + r * 64 + lane;
      total += __popcll(__ballot(pos >= C.lo && pos < C.hi && u[r] >= LC));
    }
    if (total != 0 && lane == 0)
      p_base = atomicAdd(counter + C.unit + opaque_zero, total);
    P = C;
    p_total = total;
    p_L = LC;
#pragma unroll
    for (int r = 0; r < kTaskQuads; ++r) pu[r] = u[r];

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
  }
  write_previous();
  // no buffer-to-LDS load may still be in flight when the wave ends
  wait_vm_at_most<0>();
}

} // namespace

hipError_t launch_score(const DecodeDims &d, const uint32_t *codes,
                        const uint8_t *radii, const int32_t *block_table,
                        const int32_t *seq_lens, const uint32_t *qop,
                        const float *qneg, const uint32_t *lthr,
                        uint32_t *counter, uint32_t *cand_u, int32_t *cand_pos,
                        int32_t *scores_out, hipStream_t stream) {
  const int pages = (d.n_max + kPage - 1) / kPage;
  const int64_t ngroups = (pages + kGroupPages - 1) / kGroupPages;
  if (ngroups == 0) return hipSuccess;
  const int64_t ntasks = (int64_t)d.B * ngroups * d.Hkv;
  if (ntasks > 0x7FFFFFFF - 65536) return hipErrorInvalidValue;
  const uint32_t code_bytes = (uint32_t)((uint64_t)d.num_blocks * d.Hkv * d.W * kPage * 4);
  const uint32_t radius_bytes = (uint32_t)((uint64_t)d.num_blocks * d.Hkv * kPage);
  // persistent grid: two workgroups per CU, fewer for small calls
  const int64_t nwg = std::min<int64_t>((ntasks + kWaves - 1) / kWaves,
                                        2 * (int64_t)device_cu_count());
#define DKV_SCORE_CASE(KSV, GV)                                                \
  if (d.KS == KSV && d.G == GV) {                                              \
    hipLaunchKernelGGL((filter_kernel<KSV, GV>), dim3((unsigned)nwg),          \
                       dim3(kThreads), 0, stream, codes, radii, d.num_blocks,  \
                       code_bytes, radius_bytes, block_table, d.max_blocks,    \
                       seq_lens, d.n_max, qop, qneg, lthr, d.B, d.Hkv, d.W,    \
                       (int)ngroups, (int)ntasks, d.w, d.sigma, counter,       \
                       cand_u, cand_pos, d.cand_cap, scores_out,               \
                       d.max_seq_len);                                         \
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
