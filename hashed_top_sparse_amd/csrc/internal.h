// internal.h -- shapes, workspace plan and kernel launchers shared by the
// libdkv translation units (host side) plus small device helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dkv.h"

namespace dkv {

constexpr int kPage = 16;     // tokens per page
constexpr int kHeadDim = 128; // d
constexpr int kAttnRows = 256; // selected rows per attention split

// Validated shape of one decode call.
struct DecodeDims {
  int B, Hq, Hkv, G, b, W;   // W = b/32 code words per key
  int k, w, sigma, cap;      // cap = k + w + sigma (selection list length)
  int max_seq_len;           // caller's bound (workspace stride)
  int n_max;                 // min(max_seq_len, 16*max_blocks)
  int max_blocks;
  int64_t num_blocks;
  int nsplit;                // attention splits per (sequence, KV head)
};

// Byte offsets of the decode workspace regions (each 256-byte aligned).
struct WorkspacePlan {
  size_t q8, scores, sel, cnt, part, total;
};

WorkspacePlan plan_workspace(const DecodeDims &d);

// Kernel launchers (one per translation unit that owns the kernel).
hipError_t launch_encode(const uint16_t *k_pool, int64_t num_blocks,
                         const int32_t *block_table, int max_blocks, int batch,
                         const int32_t *enc_start, const int32_t *enc_end,
                         int max_encode_len, const uint16_t *proj, int Hkv,
                         int b, uint32_t *codes, uint8_t *radii,
                         hipStream_t stream);

hipError_t launch_qprep(const DecodeDims &d, const uint16_t *q,
                        const uint16_t *proj, int8_t *q8, hipStream_t stream);

hipError_t launch_score(const DecodeDims &d, const uint32_t *codes,
                        const uint8_t *radii, const int32_t *block_table,
                        const int32_t *seq_lens, const int8_t *q8,
                        int32_t *scores, hipStream_t stream);

hipError_t launch_select(const DecodeDims &d, const int32_t *scores,
                         const int32_t *seq_lens, int32_t *sel, int32_t *cnt,
                         int32_t *user_sel, int32_t *user_cnt,
                         hipStream_t stream);

hipError_t launch_attend(const DecodeDims &d, const uint16_t *q,
                         const uint16_t *k_pool, const uint16_t *v_pool,
                         const int32_t *block_table, const int32_t *sel,
                         const int32_t *cnt, float *part, float *out,
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

} // namespace dkv
