// internal.h -- shapes, workspace plan and kernel launchers shared by the
// libdkv translation units (host side) plus small device helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dkv.h"

namespace dkv {

constexpr int kPage = 16;       // tokens per page
constexpr int kHeadDim = 128;   // d
constexpr int kAttnRows = 128;  // selected rows per attention split
constexpr int kGroupPages = 64; // pages per candidate group (one scoring task)
constexpr int kGroupKeys = kGroupPages * kPage;
constexpr int kLdsPerCu = 160 * 1024; // gfx950 LDS per compute unit

// Validated shape of one decode call.
struct DecodeDims {
  int B, Hq, Hkv, G, b, W;   // W = b/32 code words per key
  int KS;                    // 128-bit MFMA K-steps per key: max(1, b/128)
  int k, w, sigma, cap;      // cap = k + w + sigma (selection list length)
  bool lin;                  // linear radius weight (DKV_RADIUS_LINEAR)
  bool pages;                // page-granular selection (select_pages)
  int lsh_T, lsh_m;          // LSH tables and bits per table (T = 0: none)
  int max_seq_len;           // caller's bound (workspace stride)
  int n_max;                 // min(max_seq_len, 16*max_blocks)
  int max_blocks;
  int64_t num_blocks;
  int cand_groups;           // candidate groups per (sequence, KV head):
                             // ceil(max_seq_len / kGroupKeys)
  int bm_words;              // selection bitmap words per (sequence, KV head)
  int nsplit;                // attention split states per (sequence, KV head):
  int nsplit_w;              // the first nsplit_w over its sink and window
                             // rows, the rest over its top-k rows
  bool window_in_prep;       // the window rows are attended by extra
                             // workgroups of the prep launch (one state,
                             // split 0), the sinks with the top-k rows
  int nsplit_max;            // the most splits either way (workspace size)
};

// Byte offsets of the decode workspace regions (each 256-byte aligned).
struct WorkspacePlan {
  size_t q8, qop, qneg, lthr, cand, tcount, bitmap, rows, cnt, part, qbits, tasks, total;
};

// Byte layout of the LSH index of one (sequence, KV head) unit: a 64-byte
// header (int32 indexed length), then per table the bucket offsets
// [2^m + 1] and the positions [max_seq_len] (int32), the unit padded to 256
// bytes.
struct LshLayout {
  size_t off0, pos0;   // byte offsets of table 0's offsets and positions
  size_t off_stride;   // bytes between tables' offset arrays
  size_t pos_stride;   // bytes between tables' position arrays
  size_t unit_bytes;
};
LshLayout lsh_layout(int T, int m, int max_seq_len);

WorkspacePlan plan_workspace(const DecodeDims &d);

// Compute units of the current device (cached per device id).
int device_cu_count();

// Kernel launchers (one per translation unit that owns the kernel).
hipError_t launch_encode(const uint16_t *k_pool, int64_t num_blocks,
                         const int32_t *block_table, int max_blocks, int batch,
                         const int32_t *enc_start, const int32_t *enc_end,
                         int max_encode_len, const uint16_t *proj, int Hkv,
                         int b, uint32_t *codes, uint8_t *radii,
                         hipStream_t stream);

// Query codes q8 [B][Hq][b], the score matrix-core operand qop
// [B*Hkv][KS][64 lanes][8 dwords], qneg [B][Hq] = -sum_j q8, and per
// (sequence, KV head) the candidate threshold lthr (from a page sample).
// With qbits (LSH decode) it also writes each query head's sign code
// [B][Hq][b/32] and no threshold sample is taken (lthr = 0).  tasks: the
// score filter's task list (see launch_score).
// With d.window_in_prep the same launch also attends over every unit's
// window rows (v_pool, part: as launch_attend), in workgroups of its own.
hipError_t launch_prep(const DecodeDims &d, const uint16_t *q,
                       const uint16_t *proj, const uint32_t *codes,
                       const uint8_t *radii, const uint16_t *k_pool,
                       const uint16_t *v_pool, uint32_t *codes_w, uint8_t *radii_w,
                       const int32_t *block_table,
                       const int32_t *seq_lens, int8_t *q8, uint32_t *qop,
                       float *qneg, uint32_t *lthr, uint32_t *qbits,
                       uint32_t *tasks, float *part, hipStream_t stream);

// LSH (lsh.hip): the bucket index of positions [0, seq_lens[s]); the probe
// that marks each unit's candidates in its bitmap [B*Hkv][bm_words]; and
// the scoring of the pages that hold candidates, which leaves them in the
// candidate regions as the streaming filter would (u, position), with
// their counts.
hipError_t launch_lsh_build(const DecodeDims &d, const uint32_t *codes,
                            const int32_t *block_table, const int32_t *seq_lens,
                            char *index, hipStream_t stream);
hipError_t launch_lsh_probe(const DecodeDims &d, const uint32_t *codes,
                            const int32_t *block_table, const int32_t *seq_lens,
                            const char *index, const uint32_t *qbits,
                            uint32_t *bitmap, hipStream_t stream);
hipError_t launch_lsh_score(const DecodeDims &d, const uint32_t *codes,
                            const uint8_t *radii, const int32_t *block_table,
                            const int32_t *seq_lens, const uint32_t *qop,
                            const float *qneg, const uint32_t *bitmap, uint2 *cand,
                            uint32_t *tcount, hipStream_t stream);

// Scores every cached key once; the candidates (u >= lthr) of each
// (sequence, KV head, group of kGroupKeys positions) go to that group's
// region of cand [B*Hkv][cand_groups][kGroupKeys] as (u, position) in
// position order, with their number in tcount [B*Hkv][cand_groups].  Groups
// at or past a sequence's length are not written.
// With page-granular selection the candidates are pages instead: (best u
// of the page's keys in [sinks, N - window), page index), one per page that
// meets that range.
// tasks: the list prep writes (a count word, then per page group of a
// sequence that holds keys, (sequence, group, length) as 16 bytes).
hipError_t launch_score(const DecodeDims &d, const uint32_t *codes,
                        const uint8_t *radii, const int32_t *block_table,
                        const uint32_t *tasks, const uint32_t *qop,
                        const float *qneg, const uint32_t *lthr, uint2 *cand,
                        uint32_t *tcount, int32_t *scores_out,
                        hipStream_t stream);

// The filter of each (selection granularity, radius weight), one per
// translation unit (score_keys_log.hip, score_keys_linear.hip,
// score_pages_log.hip, score_pages_linear.hip) so they compile in parallel;
// launch_score picks one.  Same arguments as launch_score.
#define DKV_FILTER_DECL(NAME)                                                  \
  hipError_t NAME(const DecodeDims &d, const uint32_t *codes,                  \
                  const uint8_t *radii, const int32_t *block_table,            \
                  const uint32_t *tasks, const uint32_t *qop,                  \
                  const float *qneg, const uint32_t *lthr, uint2 *cand,        \
                  uint32_t *tcount, int32_t *scores_out, hipStream_t stream)
DKV_FILTER_DECL(launch_filter_keys_log);
DKV_FILTER_DECL(launch_filter_keys_linear);
DKV_FILTER_DECL(launch_filter_pages_log);
DKV_FILTER_DECL(launch_filter_pages_linear);

// Final selection (sinks, window, exact top-k in position order): rows
// (physical row ids blk*16+slot, -1 past the count), cnt, and the optional
// user lists.
hipError_t launch_merge(const DecodeDims &d, const uint2 *cand,
                        const uint32_t *tcount,
                        const int32_t *seq_lens, const int32_t *block_table,
                        uint32_t *bitmap, int32_t *rows, int32_t *cnt,
                        int32_t *user_sel, int32_t *user_cnt,
                        const uint32_t *codes, const uint8_t *radii,
                        const uint32_t *qop, const float *qneg,
                        hipStream_t stream);

// Attention splits over the selection list rows (physical row ids, cnt
// per unit) into part [B*Hkv][nsplit][G][2 + d]; the sink and window rows
// are found from the positions and the block table, or the window rows
// were attended in the prep launch (d.window_in_prep).
hipError_t launch_attend(const DecodeDims &d, const uint16_t *q,
                         const uint16_t *k_pool, const uint16_t *v_pool,
                         const int32_t *rows, const int32_t *cnt,
                         const int32_t *seq_lens, const int32_t *block_table,
                         float *part, hipStream_t stream);

hipError_t launch_combine(const DecodeDims &d, const float *part, float *out,
                          hipStream_t stream);

// ---------------------------------------------------------------- device
__device__ __forceinline__ float bf16_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ int clamp_int(int x, int lo, int hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// Cached length of sequence s, clamped to what the grids and pools allow.
__device__ __forceinline__ int seq_len_clamped(const int32_t *seq_lens, int s,
                                               int n_max) {
  return clamp_int(seq_lens[s], 0, n_max);
}

// Wave-wide reductions and scans with every lane active, without LDS
// round trips: DPP moves inside each 16-lane row (quad perms [1,0,3,2] and
// [2,3,0,1], the half-row and row mirrors, whose sources are always in the
// row), then the gfx950 swaps across rows 16 and 32 lanes apart.  Every
// lane gets the result.
#define DKV_DPP_ROW_ALL(X, OP, MOV)                                            \
  X = OP(X, MOV(X, 0xB1));                                                     \
  X = OP(X, MOV(X, 0x4E));                                                     \
  X = OP(X, MOV(X, 0x141));                                                    \
  X = OP(X, MOV(X, 0x140));
#define DKV_DPP_MOV_U32(X, C)                                                  \
  ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)(X), C, 0xF, 0xF, false))
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
#define DKV_ADD(A, B) ((A) + (B))
  DKV_DPP_ROW_ALL(x, DKV_ADD, DKV_DPP_MOV_U32)
#undef DKV_ADD
  auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = a[0] + a[1];
  a = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return a[0] + a[1];
}
__device__ __forceinline__ void wave_min_max(uint32_t &lo, uint32_t &hi) {
#define DKV_MIN(A, B) min((A), (B))
#define DKV_MAX(A, B) max((A), (B))
  DKV_DPP_ROW_ALL(lo, DKV_MIN, DKV_DPP_MOV_U32)
  DKV_DPP_ROW_ALL(hi, DKV_MAX, DKV_DPP_MOV_U32)
  auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  lo = DKV_MIN(a[0], a[1]);
  a = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  hi = DKV_MAX(a[0], a[1]);
  a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  lo = DKV_MIN(a[0], a[1]);
  a = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  hi = DKV_MAX(a[0], a[1]);
#undef DKV_MIN
#undef DKV_MAX
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#define DKV_MAX(A, B) max((A), (B))
  DKV_DPP_ROW_ALL(x, DKV_MAX, DKV_DPP_MOV_U32)
  auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = DKV_MAX(a[0], a[1]);
  a = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return DKV_MAX(a[0], a[1]);
#undef DKV_MAX
}
// Maximum of non-negative doubles, whose bit patterns order as unsigned
// 64-bit integers: the largest high word, then the largest low word among
// the lanes that hold it.
__device__ __forceinline__ double wave_max_nonneg_f64(double x) {
  const uint64_t v = (uint64_t)__double_as_longlong(x);
  const uint32_t hi = wave_max_u32((uint32_t)(v >> 32));
  const uint32_t lo = wave_max_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0u);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive prefix sum over a wave in lane order: row_shr steps 1, 2, 4, 8
// inside each 16-lane row (a lane whose source would lie outside its row
// adds 0), then the totals of the rows below.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);
  const uint32_t r0 = __builtin_amdgcn_readlane(x, 15);
  const uint32_t r1 = __builtin_amdgcn_readlane(x, 31);
  const uint32_t r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Exclusive prefix sum over a workgroup of NT threads (NT/64 waves), in
// thread order.  tmp needs NT/64 words of LDS.  Every thread must call it.
template <int NT>
__device__ __forceinline__ uint32_t wg_exclusive_scan(uint32_t v, uint32_t *tmp,
                                                      uint32_t *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t t = tmp[i];
    base += (i < wave) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

} // namespace dkv
