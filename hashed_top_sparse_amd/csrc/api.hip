// api.hip -- the C ABI of libdkv: argument validation, workspace plan and
// the launch sequence of one decode step.  Every entry point validates on
// the host and returns a status before any launch; nothing is allocated.
#include <string.h>

#include <algorithm>
#include <atomic>

#include "internal.h"

namespace dkv {
namespace {

constexpr int kDecodeStages = 5;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Kernels read pool rows, code words, radius lines and the projection with
// 16-byte loads.
bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

bool valid_config(const dkv_config *cfg, dkv_status *why) {
  if (cfg == nullptr) {
    *why = DKV_ERR_INVALID_ARG;
    return false;
  }
  if (cfg->num_q_heads <= 0 || cfg->num_kv_heads <= 0 || cfg->top_k < 0 ||
      cfg->window < 0 || cfg->sinks < 0 ||
      cfg->num_q_heads % cfg->num_kv_heads != 0) {
    *why = DKV_ERR_INVALID_ARG;
    return false;
  }
  const int G = cfg->num_q_heads / cfg->num_kv_heads;
  const int64_t sel = (int64_t)cfg->top_k + cfg->window + cfg->sinks;
  if (cfg->head_dim != kHeadDim || cfg->page_size != kPage ||
      !(cfg->code_bits == 64 || cfg->code_bits == 128 ||
        cfg->code_bits == 256) ||
      !(G == 1 || G == 2 || G == 4 || G == 8) || sel > DKV_MAX_SELECT ||
      cfg->num_kv_heads > 4096 ||
      !(cfg->radius_weight == DKV_RADIUS_LOG ||
        cfg->radius_weight == DKV_RADIUS_LINEAR) ||
      !(cfg->select_pages == 0 || cfg->select_pages == 1) || cfg->lsh_tables < 0 ||
      (cfg->lsh_tables > 0 &&
       (cfg->lsh_bits < 1 || cfg->lsh_bits > 12 || cfg->select_pages != 0 ||
        (int64_t)cfg->lsh_tables * cfg->lsh_bits > cfg->code_bits))) {
    *why = DKV_ERR_UNSUPPORTED;
    return false;
  }
  return true;
}

bool make_dims(const dkv_config *cfg, int32_t batch, int32_t max_seq_len,
               int32_t max_blocks, int64_t num_blocks, DecodeDims *d,
               dkv_status *why) {
  if (!valid_config(cfg, why)) return false;
  if (batch <= 0 || batch > 65535 || max_seq_len < 0 || max_blocks < 0 ||
      num_blocks < 0) {
    *why = DKV_ERR_INVALID_ARG;
    return false;
  }
  if (max_seq_len > DKV_MAX_SEQ_LEN) {
    *why = DKV_ERR_UNSUPPORTED;
    return false;
  }
  d->B = batch;
  d->Hq = cfg->num_q_heads;
  d->Hkv = cfg->num_kv_heads;
  d->G = d->Hq / d->Hkv;
  d->b = cfg->code_bits;
  d->W = d->b / 32;
  d->KS = d->b > 128 ? d->b / 128 : 1;
  d->k = cfg->top_k;
  d->w = cfg->window;
  d->sigma = cfg->sinks;
  d->lin = cfg->radius_weight == DKV_RADIUS_LINEAR;
  d->pages = cfg->select_pages == 1;
  d->lsh_T = cfg->lsh_tables;
  d->lsh_m = cfg->lsh_tables > 0 ? cfg->lsh_bits : 0;
  d->cap = d->k + d->w + d->sigma;
  d->max_seq_len = max_seq_len;
  const int64_t by_blocks = (int64_t)kPage * max_blocks;
  d->n_max = (int)(by_blocks < max_seq_len ? by_blocks : max_seq_len);
  d->max_blocks = max_blocks;
  d->num_blocks = num_blocks;
  // The list holds at most sigma sink rows, w window rows, then at most k
  // top-k rows.  The prep launch attends over the window rows in one extra
  // workgroup per unit when those fit beside its own workgroups in one
  // round (they need a compute unit each); the split kernel then takes the
  // sinks with the top-k rows.  Otherwise it takes the sinks and window in
  // splits of their own.
  const int nsw = (d->sigma + d->w + kAttnRows - 1) / kAttnRows;
  d->window_in_prep = d->w > 0 && 2 * (int64_t)batch * d->Hkv <= device_cu_count();
  d->nsplit_w = d->window_in_prep ? 1 : nsw;
  d->nsplit = d->window_in_prep ? 1 + (d->sigma + d->k + kAttnRows - 1) / kAttnRows
                                : nsw + (d->k + kAttnRows - 1) / kAttnRows;
  d->nsplit_max = nsw + (d->sigma + d->k + kAttnRows - 1) / kAttnRows;
  d->cand_groups = (max_seq_len + kGroupKeys - 1) / kGroupKeys;
  d->bm_words = (max_seq_len + 31) / 32;
  // candidate regions are numbered with 32-bit ids
  if ((int64_t)d->B * d->Hkv * d->cand_groups >= (int64_t)1 << 31) {
    *why = DKV_ERR_UNSUPPORTED;
    return false;
  }
  // buffer views of the code and radius pools use 32-bit byte offsets; a
  // load of an invalid page starts at the pool's end, and stays below 2^32
  if ((uint64_t)num_blocks * d->Hkv * d->W * kPage * 4 > 0xFFFFF000ull) {
    *why = DKV_ERR_UNSUPPORTED;
    return false;
  }
  if ((int64_t)d->B * d->Hkv > 65535 * 64) {
    *why = DKV_ERR_UNSUPPORTED;
    return false;
  }
  return true;
}

dkv_status decode_impl(const dkv_config *cfg, const void *q,
                       const void *k_pool, const void *v_pool,
                       const uint32_t *codes, const uint8_t *radii,
                       int64_t num_blocks, const int32_t *block_table,
                       int32_t max_blocks_per_seq, const int32_t *seq_lens,
                       int32_t batch, int32_t max_seq_len, const void *proj,
                       float *out, int32_t *sel_idx, int32_t *sel_cnt,
                       void *workspace, size_t workspace_bytes, int8_t *q8_out,
                       int32_t *scores_out, dkv_event_t *events, bool append,
                       const void *lsh_index, size_t lsh_index_bytes,
                       hipStream_t stream) {
  DecodeDims d;
  dkv_status why = DKV_OK;
  if (!make_dims(cfg, batch, max_seq_len, max_blocks_per_seq, num_blocks, &d,
                 &why))
    return why;
  if (q == nullptr || k_pool == nullptr || v_pool == nullptr ||
      codes == nullptr || radii == nullptr || block_table == nullptr ||
      seq_lens == nullptr || proj == nullptr || out == nullptr ||
      max_blocks_per_seq <= 0 || num_blocks <= 0)
    return DKV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned16(codes) || !aligned16(radii) || !aligned16(proj))
    return DKV_ERR_INVALID_ARG;
  // an LSH config decodes through its index, and only then
  if ((d.lsh_T > 0) != (lsh_index != nullptr)) return DKV_ERR_INVALID_ARG;
  if (d.lsh_T > 0) {
    if (max_seq_len > DKV_LSH_MAX_SEQ_LEN) return DKV_ERR_UNSUPPORTED;
    const size_t need = (size_t)d.B * d.Hkv *
                        lsh_layout(d.lsh_T, d.lsh_m, d.max_seq_len).unit_bytes;
    if (lsh_index_bytes < need || ((uintptr_t)lsh_index & 255) != 0)
      return DKV_ERR_WORKSPACE;
  }
  const WorkspacePlan plan = plan_workspace(d);
  if (workspace == nullptr || workspace_bytes < plan.total ||
      ((uintptr_t)workspace & 255) != 0)
    return DKV_ERR_WORKSPACE;

  char *ws = static_cast<char *>(workspace);
  int8_t *q8 = q8_out ? q8_out : reinterpret_cast<int8_t *>(ws + plan.q8);
  uint32_t *qop = reinterpret_cast<uint32_t *>(ws + plan.qop);
  float *qneg = reinterpret_cast<float *>(ws + plan.qneg);
  uint32_t *lthr = reinterpret_cast<uint32_t *>(ws + plan.lthr);
  uint2 *cand = reinterpret_cast<uint2 *>(ws + plan.cand);
  uint32_t *tcount = reinterpret_cast<uint32_t *>(ws + plan.tcount);
  uint32_t *bitmap = reinterpret_cast<uint32_t *>(ws + plan.bitmap);
  int32_t *rows = reinterpret_cast<int32_t *>(ws + plan.rows);
  int32_t *cnt = reinterpret_cast<int32_t *>(ws + plan.cnt);
  float *part = reinterpret_cast<float *>(ws + plan.part);
  uint32_t *qbits = d.lsh_T > 0 ? reinterpret_cast<uint32_t *>(ws + plan.qbits) : nullptr;
  uint32_t *tasks = reinterpret_cast<uint32_t *>(ws + plan.tasks);
  const uint16_t *q16 = static_cast<const uint16_t *>(q);
  const uint16_t *k16 = static_cast<const uint16_t *>(k_pool);
  const uint16_t *v16 = static_cast<const uint16_t *>(v_pool);
  const uint16_t *p16 = static_cast<const uint16_t *>(proj);

  // Stage boundaries: an event is recorded before each stage and after the
  // last one when the caller asked for them.
  int stage = 0;
  auto mark = [&]() -> bool {
    if (events == nullptr) return true;
    return hipEventRecord(reinterpret_cast<hipEvent_t>(events[stage++]),
                          stream) == hipSuccess;
  };
  // append: the prep kernel also encodes each sequence's newest key
  uint32_t *codes_w = append ? const_cast<uint32_t *>(codes) : nullptr;
  uint8_t *radii_w = append ? const_cast<uint8_t *>(radii) : nullptr;
  if (!mark() || launch_prep(d, q16, p16, codes, radii, k16, v16, codes_w, radii_w,
                             block_table, seq_lens, q8, qop, qneg, lthr, qbits,
                             tasks, part, stream) != hipSuccess)
    return DKV_ERR_LAUNCH;
  if (d.lsh_T > 0) {
    // bucket probe, then scoring of the pages that hold candidates
    if (!mark() ||
        launch_lsh_probe(d, codes, block_table, seq_lens,
                         static_cast<const char *>(lsh_index), qbits, bitmap,
                         stream) != hipSuccess ||
        launch_lsh_score(d, codes, radii, block_table, seq_lens, qop, qneg, bitmap,
                         cand, tcount, stream) != hipSuccess)
      return DKV_ERR_LAUNCH;
  } else if (!mark() || launch_score(d, codes, radii, block_table, tasks, qop,
                                     qneg, lthr, cand, tcount, scores_out,
                                     stream) != hipSuccess) {
    return DKV_ERR_LAUNCH;
  }
  if (!mark() || launch_merge(d, cand, tcount, seq_lens,
                              block_table, bitmap, rows, cnt, sel_idx, sel_cnt,
                              codes, radii, qop, qneg, stream) != hipSuccess)
    return DKV_ERR_LAUNCH;
  if (!mark() || launch_attend(d, q16, k16, v16, rows, cnt, seq_lens, block_table,
                              part, stream) !=
                     hipSuccess)
    return DKV_ERR_LAUNCH;
  if (!mark() || launch_combine(d, part, out, stream) != hipSuccess)
    return DKV_ERR_LAUNCH;
  if (!mark()) return DKV_ERR_LAUNCH;
  return DKV_OK;
}

} // namespace

int device_cu_count() {
  // Per device id; relaxed atomics, so threads that race on a first call
  // each store the same value and no thread reads a torn one.
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess ||
      n <= 0)
    n = 256;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

WorkspacePlan plan_workspace(const DecodeDims &d) {
  WorkspacePlan p;
  const size_t units = (size_t)d.B * d.Hkv;
  size_t off = 0;
  p.q8 = off;
  off += align256((size_t)d.B * d.Hq * d.b);
  p.qop = off;
  off += align256(units * d.KS * 64 * 8 * 4);
  p.qneg = off;
  off += align256((size_t)d.B * d.Hq * 4);
  p.lthr = off;
  off += align256(units * 4);
  p.cand = off;
  off += align256(units * (size_t)d.cand_groups * kGroupKeys * 8);
  p.tcount = off;
  off += align256(units * (size_t)d.cand_groups * 4);
  p.bitmap = off;
  off += align256(units * (size_t)d.bm_words * 4);
  p.rows = off;
  off += align256(units * (size_t)d.cap * 4);
  p.cnt = off;
  off += align256(units * 4);
  p.part = off;
  off += align256(units * d.nsplit_max * d.G * (kHeadDim + 2) * 4);
  p.qbits = off;
  off += align256((size_t)d.B * d.Hq * d.W * 4);
  p.tasks = off; // count word (padded to 16 bytes), then 16 bytes per group
  off += align256(16 + (size_t)d.B * d.cand_groups * 16);
  p.total = off;
  return p;
}

} // namespace dkv

// The workspace of dkv_decode_append_noalloc: one copy per GPU, held until
// the process ends.  In host code this name is only a stand-in: kernels get
// the device address that hipGetSymbolAddress returns for the current
// device (noalloc_scratch below), never the name itself.
static __device__ __align__(256) unsigned char scratch[DKV_NOALLOC_SCRATCH_BYTES];

namespace dkv {
namespace {

constexpr int kMaxDevices = 64;

// Device address of the current device's copy of `scratch`, looked up on
// the first call on that device (with it current) and kept; nullptr when
// the lookup fails.  Threads racing on a first call store the same address.
void *noalloc_scratch() {
  static std::atomic<void *> addr[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void *p = addr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
    return nullptr;
  addr[dev].store(p, std::memory_order_release);
  return p;
}

} // namespace
} // namespace dkv

using namespace dkv;

extern "C" {

__attribute__((visibility("default"))) dkv_status
dkv_encode(const dkv_config *cfg, const void *k_pool, int64_t num_blocks,
           const int32_t *block_table, int32_t max_blocks_per_seq,
           int32_t batch, const int32_t *enc_start, const int32_t *enc_end,
           int32_t max_encode_len, const void *proj, uint32_t *codes,
           uint8_t *radii, dkv_stream_t stream) {
  dkv_status why = DKV_OK;
  if (!valid_config(cfg, &why)) return why;
  if (k_pool == nullptr || block_table == nullptr || enc_start == nullptr ||
      enc_end == nullptr || proj == nullptr || codes == nullptr ||
      radii == nullptr || num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      batch <= 0 || batch > 65535 || max_encode_len < 0)
    return DKV_ERR_INVALID_ARG;
  if (!aligned16(k_pool) || !aligned16(codes) || !aligned16(radii) ||
      !aligned16(proj))
    return DKV_ERR_INVALID_ARG;
  if (max_encode_len > DKV_MAX_SEQ_LEN ||
      max_blocks_per_seq > DKV_MAX_SEQ_LEN / kPage ||
      (int64_t)batch * max_blocks_per_seq >= (int64_t)1 << 30)
    return DKV_ERR_UNSUPPORTED;
  hipError_t e = launch_encode(
      static_cast<const uint16_t *>(k_pool), num_blocks, block_table,
      max_blocks_per_seq, batch, enc_start, enc_end, max_encode_len,
      static_cast<const uint16_t *>(proj), cfg->num_kv_heads, cfg->code_bits,
      codes, radii, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DKV_OK : DKV_ERR_LAUNCH;
}

__attribute__((visibility("default"))) size_t
dkv_decode_workspace_size(const dkv_config *cfg, int32_t batch,
                          int32_t max_seq_len) {
  DecodeDims d;
  dkv_status why;
  const int32_t max_blocks = (max_seq_len + kPage - 1) / kPage;
  if (!make_dims(cfg, batch, max_seq_len, max_blocks, 1, &d, &why)) return 0;
  return plan_workspace(d).total;
}

__attribute__((visibility("default"))) dkv_status
dkv_decode(const dkv_config *cfg, const void *q, const void *k_pool,
           const void *v_pool, const uint32_t *codes, const uint8_t *radii,
           int64_t num_blocks, const int32_t *block_table,
           int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t batch,
           int32_t max_seq_len, const void *proj, float *out, int32_t *sel_idx,
           int32_t *sel_cnt, void *workspace, size_t workspace_bytes,
           dkv_stream_t stream) {
  return decode_impl(cfg, q, k_pool, v_pool, codes, radii, num_blocks,
                     block_table, max_blocks_per_seq, seq_lens, batch,
                     max_seq_len, proj, out, sel_idx, sel_cnt, workspace,
                     workspace_bytes, nullptr, nullptr, nullptr, false, nullptr, 0,
                     reinterpret_cast<hipStream_t>(stream));
}

__attribute__((visibility("default"))) dkv_status dkv_decode_debug(
    const dkv_config *cfg, const void *q, const void *k_pool,
    const void *v_pool, const uint32_t *codes, const uint8_t *radii,
    int64_t num_blocks, const int32_t *block_table, int32_t max_blocks_per_seq,
    const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
    const void *proj, float *out, int32_t *sel_idx, int32_t *sel_cnt,
    void *workspace, size_t workspace_bytes, int8_t *q8_out,
    int32_t *scores_out, dkv_stream_t stream) {
  return decode_impl(cfg, q, k_pool, v_pool, codes, radii, num_blocks,
                     block_table, max_blocks_per_seq, seq_lens, batch,
                     max_seq_len, proj, out, sel_idx, sel_cnt, workspace,
                     workspace_bytes, q8_out, scores_out, nullptr, false, nullptr, 0,
                     reinterpret_cast<hipStream_t>(stream));
}

__attribute__((visibility("default"))) dkv_status dkv_decode_profiled(
    const dkv_config *cfg, const void *q, const void *k_pool,
    const void *v_pool, const uint32_t *codes, const uint8_t *radii,
    int64_t num_blocks, const int32_t *block_table, int32_t max_blocks_per_seq,
    const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
    const void *proj, float *out, int32_t *sel_idx, int32_t *sel_cnt,
    void *workspace, size_t workspace_bytes, dkv_event_t *stage_events,
    dkv_stream_t stream) {
  if (stage_events == nullptr) return DKV_ERR_INVALID_ARG;
  for (int i = 0; i <= kDecodeStages; ++i)
    if (stage_events[i] == nullptr) return DKV_ERR_INVALID_ARG;
  return decode_impl(cfg, q, k_pool, v_pool, codes, radii, num_blocks,
                     block_table, max_blocks_per_seq, seq_lens, batch,
                     max_seq_len, proj, out, sel_idx, sel_cnt, workspace,
                     workspace_bytes, nullptr, nullptr, stage_events, false, nullptr, 0,
                     reinterpret_cast<hipStream_t>(stream));
}

__attribute__((visibility("default"))) dkv_status dkv_decode_append(
    const dkv_config *cfg, const void *q, const void *k_pool,
    const void *v_pool, uint32_t *codes, uint8_t *radii, int64_t num_blocks,
    const int32_t *block_table, int32_t max_blocks_per_seq,
    const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
    const void *proj, float *out, int32_t *sel_idx, int32_t *sel_cnt,
    void *workspace, size_t workspace_bytes, dkv_event_t *stage_events,
    dkv_stream_t stream) {
  if (stage_events != nullptr)
    for (int i = 0; i <= kDecodeStages; ++i)
      if (stage_events[i] == nullptr) return DKV_ERR_INVALID_ARG;
  return decode_impl(cfg, q, k_pool, v_pool, codes, radii, num_blocks,
                     block_table, max_blocks_per_seq, seq_lens, batch,
                     max_seq_len, proj, out, sel_idx, sel_cnt, workspace,
                     workspace_bytes, nullptr, nullptr, stage_events, true, nullptr, 0,
                     reinterpret_cast<hipStream_t>(stream));
}

__attribute__((visibility("default"))) dkv_status dkv_decode_append_noalloc(
    const dkv_config *cfg, const void *q, const void *k_pool, const void *v_pool,
    uint32_t *codes, uint8_t *radii, int64_t num_blocks, const int32_t *block_table,
    int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t batch,
    int32_t max_seq_len, const void *proj, float *out, int32_t *sel_idx,
    int32_t *sel_cnt, dkv_stream_t stream) {
  DecodeDims d;
  dkv_status why = DKV_OK;
  if (!make_dims(cfg, batch, max_seq_len, max_blocks_per_seq, num_blocks, &d, &why))
    return why;
  if (d.lsh_T > 0) return DKV_ERR_INVALID_ARG; // LSH decodes through dkv_decode_lsh
  // the size check comes before the device lookup
  if (plan_workspace(d).total > DKV_NOALLOC_SCRATCH_BYTES) return DKV_ERR_WORKSPACE;
  if (q == nullptr || k_pool == nullptr || v_pool == nullptr || codes == nullptr ||
      radii == nullptr || block_table == nullptr || seq_lens == nullptr ||
      proj == nullptr || out == nullptr)
    return DKV_ERR_INVALID_ARG;
  void *ws = noalloc_scratch();
  if (ws == nullptr) return DKV_ERR_LAUNCH;
  return decode_impl(cfg, q, k_pool, v_pool, codes, radii, num_blocks, block_table,
                     max_blocks_per_seq, seq_lens, batch, max_seq_len, proj, out,
                     sel_idx, sel_cnt, ws, DKV_NOALLOC_SCRATCH_BYTES, nullptr, nullptr,
                     nullptr, true, nullptr, 0, reinterpret_cast<hipStream_t>(stream));
}

__attribute__((visibility("default"))) size_t
dkv_lsh_index_size(const dkv_config *cfg, int32_t batch, int32_t max_seq_len) {
  DecodeDims d;
  dkv_status why;
  const int32_t max_blocks = (max_seq_len + kPage - 1) / kPage;
  if (!make_dims(cfg, batch, max_seq_len, max_blocks, 1, &d, &why) || d.lsh_T == 0 ||
      max_seq_len > DKV_LSH_MAX_SEQ_LEN)
    return 0;
  return (size_t)d.B * d.Hkv * lsh_layout(d.lsh_T, d.lsh_m, max_seq_len).unit_bytes;
}

__attribute__((visibility("default"))) dkv_status
dkv_lsh_build(const dkv_config *cfg, const uint32_t *codes, int64_t num_blocks,
              const int32_t *block_table, int32_t max_blocks_per_seq, int32_t batch,
              const int32_t *seq_lens, int32_t max_seq_len, void *index,
              size_t index_bytes, dkv_stream_t stream) {
  DecodeDims d;
  dkv_status why = DKV_OK;
  if (!make_dims(cfg, batch, max_seq_len, max_blocks_per_seq, num_blocks, &d, &why))
    return why;
  if (codes == nullptr || block_table == nullptr || seq_lens == nullptr ||
      max_blocks_per_seq <= 0 || num_blocks <= 0 || d.lsh_T == 0 || !aligned16(codes))
    return DKV_ERR_INVALID_ARG;
  if (max_seq_len > DKV_LSH_MAX_SEQ_LEN) return DKV_ERR_UNSUPPORTED;
  const size_t need = (size_t)d.B * d.Hkv *
                      lsh_layout(d.lsh_T, d.lsh_m, d.max_seq_len).unit_bytes;
  if (index == nullptr || index_bytes < need || ((uintptr_t)index & 255) != 0)
    return DKV_ERR_WORKSPACE;
  return launch_lsh_build(d, codes, block_table, seq_lens, static_cast<char *>(index),
                          reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? DKV_OK
             : DKV_ERR_LAUNCH;
}

__attribute__((visibility("default"))) dkv_status dkv_decode_lsh(
    const dkv_config *cfg, const void *q, const void *k_pool, const void *v_pool,
    const uint32_t *codes, const uint8_t *radii, int64_t num_blocks,
    const int32_t *block_table, int32_t max_blocks_per_seq, const int32_t *seq_lens,
    int32_t batch, int32_t max_seq_len, const void *proj, const void *index,
    size_t index_bytes, float *out, int32_t *sel_idx, int32_t *sel_cnt,
    void *workspace, size_t workspace_bytes, dkv_event_t *stage_events,
    dkv_stream_t stream) {
  if (index == nullptr) return DKV_ERR_INVALID_ARG;
  if (stage_events != nullptr)
    for (int i = 0; i <= kDecodeStages; ++i)
      if (stage_events[i] == nullptr) return DKV_ERR_INVALID_ARG;
  return decode_impl(cfg, q, k_pool, v_pool, codes, radii, num_blocks, block_table,
                     max_blocks_per_seq, seq_lens, batch, max_seq_len, proj, out,
                     sel_idx, sel_cnt, workspace, workspace_bytes, nullptr, nullptr,
                     stage_events, false, index, index_bytes,
                     reinterpret_cast<hipStream_t>(stream));
}

__attribute__((visibility("default"))) int32_t dkv_decode_num_stages(void) {
  return kDecodeStages;
}

__attribute__((visibility("default"))) const char *
dkv_decode_stage_name(int32_t stage) {
  static const char *const names[kDecodeStages] = {
      "prep", "score", "merge", "attend", "combine"};
  if (stage < 0 || stage >= kDecodeStages) return "";
  return names[stage];
}

__attribute__((visibility("default"))) const char *
dkv_status_string(dkv_status status) {
  switch (status) {
  case DKV_OK:
    return "DKV_OK";
  case DKV_ERR_INVALID_ARG:
    return "DKV_ERR_INVALID_ARG: null pointer or invalid size/shape";
  case DKV_ERR_UNSUPPORTED:
    return "DKV_ERR_UNSUPPORTED: head_dim, code_bits, page_size, group size "
           "or a size limit is not supported";
  case DKV_ERR_WORKSPACE:
    return "DKV_ERR_WORKSPACE: workspace missing, misaligned or too small "
           "(dkv_decode_append_noalloc: the step needs more than "
           "DKV_NOALLOC_SCRATCH_BYTES of workspace)";
  case DKV_ERR_LAUNCH:
    return "DKV_ERR_LAUNCH: a kernel launch failed";
  }
  return "unknown dkv_status";
}

__attribute__((visibility("default"))) int32_t dkv_abi_version(void) {
  return DKV_ABI_VERSION;
}

} // extern "C"
