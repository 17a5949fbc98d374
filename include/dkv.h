/*
 * dkv.h -- C ABI of libdkv: score-then-select sparse decode attention over a
 * paged, GQA-shaped KV cache on AMD Instinct MI355X (gfx950).
 *
 * The method (sources are web pages, cited by title and section):
 *  - "SPHERICAL KV: Angle-Domain Attention and Rate-Distortion Retention for
 *    Efficient Long-Context Inference", technical summary §2.1 (keys stored
 *    as a quantised radius plus a packed angle code; logits computed from
 *    the codes without rebuilding dense keys) and §2.3 (paged, ragged KV
 *    substrate; dense keys are mapped to codes when written).
 *  - "DASH-KV: asymmetric hashing accelerates long-context LLM inference",
 *    sections on asymmetric deep hashing (queries and keys get different
 *    encoders; key codes are cached and reused) and on the quadratic-to-
 *    linear argument (a light pre-filter keeps only the Top-K keys for
 *    exact attention).
 *  - "DeepSeek: why 1M context cannot be bought with memory -- from DSA to
 *    CSA/HCA", section "starting from DSA" (a light indexer scores all
 *    history, then real attention runs on the top-k only) and the CSA
 *    section (a sliding window keeps the most recent tokens).
 *  - DySCO review page, item 1 of the mathematical model (attention is
 *    softmax(QK^T/sqrt(d))) and FAQ 3 (a few initial tokens act as
 *    attention sinks).
 *
 * The concrete code (the pages leave the encoders open):
 *   key code    b sign bits of p = k.P (P: seeded Gaussian d x b, bf16);
 *               bit j = [p_j > 0], p_j accumulated in double precision in
 *               index order; bits packed LSB-first into uint32 words.
 *   key radius  r8 = largest m in 1..255 with |k|^2 >= 2^((m-64)/8), else 0
 *               (|k|^2 summed in double precision in index order).
 *   query code  q8 = round_half_even(p*127/M), p = q.P in double precision,
 *               M = max |p| over the KV group's G query heads and b columns.
 *   score       S = w(r8) * max_{h in group} sum_j q8_hj * (bit_j ? +1 : -1)
 *               with the radius weight w chosen per config: the code itself
 *               (w = r8), or linear in the radius the code stands for
 *               (w = round_half_even(2^(r8/16)), 1..62757; [SKV §2.1]: the
 *               approximate logit scales the code similarity by the
 *               decoded radius).  |S| < 2^31 in both.
 *   selection   per (sequence, KV head): sinks [0, sigma), window
 *               [N-w, N), plus the top k of [sigma, N-w) by (S descending,
 *               position ascending); or, with select_pages, the keys in
 *               [sigma, N-w) of the top k/16 16-token pages by (page score
 *               descending, page index ascending), a page's score being
 *               the largest S of its keys in that range ([DeepSeek CSA]:
 *               several tokens condensed into one entry before the top-k;
 *               [SKV §2.2]: pages read as one stream instead of scattered
 *               rows).
 *   attention   exact softmax(q.k/sqrt(d)) . V over the selection, fp32
 *               accumulation, for each query head of the group.
 *
 * Memory layouts (all device memory, row-major, little-endian):
 *   bf16 tensors are passed as 16-bit bit patterns.
 *   k_pool, v_pool  [num_blocks][16][Hkv][d]   bf16  (16-token pages)
 *   codes           [num_blocks][Hkv][16][b/32] uint32 (key-major: the b/32
 *                   words of the key in slot t of the page are contiguous,
 *                   word w at index ((blk*Hkv + h)*16 + t)*(b/32) + w)
 *   radii           [num_blocks][Hkv][16]      uint8
 *   block_table     [batch][max_blocks_per_seq] int32 physical page ids
 *                   (the same id indexes k_pool, v_pool, codes and radii)
 *   proj            [d][b]                     bf16
 *   q               [batch][Hq][d]             bf16  (head h is in KV group
 *                                                      h / G)
 *   out             [batch][Hq][d]             fp32
 *   q, k_pool, v_pool, codes, radii and proj must be 16-byte aligned (a
 *   misaligned pointer returns DKV_ERR_INVALID_ARG); allocations from the
 *   HIP or torch allocators always are.
 *
 * Ownership and execution: the caller owns every buffer; the library
 * allocates no device or host memory and keeps no mutable global state
 * (apart from a per-device cache of the compute-unit count, and the static
 * scratch array of dkv_decode_append_noalloc with its per-device address),
 * so calls on different streams may run concurrently when their output and
 * workspace buffers differ.  Every call only validates its arguments on the
 * host and enqueues kernels on `stream` (a hipStream_t; NULL means the null
 * stream); it returns before the GPU work finishes.  Device-side values
 * (seq_lens, enc_start/enc_end, block ids) cannot be checked on the host:
 * kernels clamp lengths to [0, min(max_seq_len, 16*max_blocks_per_seq)] and
 * skip page ids outside [0, num_blocks); results for such inputs are
 * unspecified but no memory outside the buffers is touched.
 *
 * Errors: a non-OK status is returned before any launch when an argument is
 * invalid; DKV_ERR_LAUNCH reports a failed kernel launch.  Faults inside
 * kernels surface at the caller's next synchronisation.
 */
#ifndef DKV_H_
#define DKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same types as hipStream_t and hipEvent_t. */
typedef struct ihipStream_t *dkv_stream_t;
typedef struct ihipEvent_t *dkv_event_t;

typedef enum {
  DKV_OK = 0,
  DKV_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad shape     */
  DKV_ERR_UNSUPPORTED = 2, /* d != 128, b not in {64,128,256}, page != 16,
                              group size not in {1,2,4,8}, size limits    */
  DKV_ERR_WORKSPACE = 3,   /* workspace missing or too small             */
  DKV_ERR_LAUNCH = 4       /* hipLaunchKernel / hipGetLastError failure  */
} dkv_status;

typedef struct {
  int32_t head_dim;     /* d; must be 128                                 */
  int32_t num_q_heads;  /* Hq                                             */
  int32_t num_kv_heads; /* Hkv; Hq % Hkv == 0 and G = Hq/Hkv in {1,2,4,8} */
  int32_t code_bits;    /* b; 64, 128 or 256                              */
  int32_t page_size;    /* tokens per page; must be 16                    */
  int32_t top_k;        /* k >= 0                                         */
  int32_t window;       /* w >= 0: most recent tokens always kept         */
  int32_t sinks;        /* sigma >= 0: first tokens always kept           */
  int32_t radius_weight; /* score weight of a key's radius code r8:
                            DKV_RADIUS_LOG (0): w = r8;
                            DKV_RADIUS_LINEAR (1): w = rne(2^(r8/16));
                            other values: DKV_ERR_UNSUPPORTED            */
  int32_t select_pages;  /* 0: top_k keys; 1: the top top_k/16 pages, each
                            scored by its best key in [sigma, N-w), and
                            their keys in that range (see dkv_decode);
                            other values: DKV_ERR_UNSUPPORTED            */
  int32_t lsh_tables;    /* T >= 0 LSH tables (0: none; > 0: decode with
                            dkv_decode_lsh, see there); T*lsh_bits <= b,
                            and select_pages must be 0                   */
  int32_t lsh_bits;      /* m: bits per LSH table, 1..12 when T > 0     */
} dkv_config;

#define DKV_RADIUS_LOG 0
#define DKV_RADIUS_LINEAR 1

/* Limits checked by every entry point (DKV_ERR_UNSUPPORTED beyond them). */
#define DKV_MAX_SEQ_LEN (1 << 24)
#define DKV_MAX_SELECT (1 << 20) /* top_k + window + sinks */
#define DKV_LSH_MAX_SEQ_LEN (1 << 19) /* dkv_decode_lsh */

/*
 * dkv_encode -- build key codes and radii when keys are written to the
 * cache ([SKV §2.3]: dense keys are turned into codes at write time;
 * [DASH]: key codes are computed once and reused by every later query).
 *
 * For every sequence s and every token position t in
 * [enc_start[s], enc_end[s]) and every KV head h, reads the key row
 * k_pool[block_table[s][t/16]][t%16][h][:] and writes its code words and
 * radius into the page's slot in `codes` / `radii`.  Other slots are not
 * touched.
 *   k_pool       device, bf16 [num_blocks][16][Hkv][d]
 *   num_blocks   number of pages in every pool (> 0)
 *   block_table  device, int32 [batch][max_blocks_per_seq]
 *   enc_start, enc_end  device, int32 [batch]; positions are clamped to
 *                [0, 16*max_blocks_per_seq]; empty ranges do nothing
 *   max_encode_len  host bound on enc_end[s]-enc_start[s] for every s (sizes
 *                the grid; tokens beyond it are not encoded)
 *   proj         device, bf16 [d][b]
 *   codes        device, uint32 [num_blocks][Hkv][16][b/32] (output)
 *   radii        device, uint8  [num_blocks][Hkv][16]       (output)
 * Bits are bit-exact with the definition above: the projection is summed in
 * double precision in index order (a product of two bf16 values is exact in
 * double), and the radius code comes from an exact double-precision
 * threshold table.  (The library computes the projections on the matrix
 * cores in fp32, keeps each sign whose margin exceeds a bound on the fp32
 * error, and recomputes the others with the double-precision chain; the
 * result is the same.)  batch * max_blocks_per_seq must stay below 2^30
 * and max_blocks_per_seq at or below DKV_MAX_SEQ_LEN/16 (positions are
 * below DKV_MAX_SEQ_LEN); DKV_ERR_UNSUPPORTED otherwise.
 */
dkv_status dkv_encode(const dkv_config *cfg, const void *k_pool,
                      int64_t num_blocks, const int32_t *block_table,
                      int32_t max_blocks_per_seq, int32_t batch,
                      const int32_t *enc_start, const int32_t *enc_end,
                      int32_t max_encode_len, const void *proj,
                      uint32_t *codes, uint8_t *radii, dkv_stream_t stream);

/*
 * dkv_decode_workspace_size -- bytes of device workspace dkv_decode needs
 * for `batch` sequences of at most `max_seq_len` tokens (0 on invalid
 * arguments).  The workspace needs no initialisation and may be reused by
 * later calls on the same stream.
 */
size_t dkv_decode_workspace_size(const dkv_config *cfg, int32_t batch,
                                 int32_t max_seq_len);

/*
 * dkv_decode -- one decode step: query codes, code-domain scores of every
 * cached key, selection (sinks + window + top-k), exact attention over the
 * selection ([DSA]: indexer then attention over the top-k; [SKV §2.1]:
 * logits straight from the codes; [DYS]: softmax(QK^T/sqrt(d))).
 *
 *   q            device, bf16 [batch][Hq][d] (the step's queries)
 *   k_pool, v_pool  device, bf16 [num_blocks][16][Hkv][d]
 *   codes, radii device, as written by dkv_encode for every cached token
 *   num_blocks   pages in every pool
 *   block_table  device, int32 [batch][max_blocks_per_seq]
 *   seq_lens     device, int32 [batch]: tokens cached per sequence,
 *                the current token included (it falls in the window)
 *   max_seq_len  host bound on seq_lens (sizes grids and the workspace)
 *   proj         device, bf16 [d][b] (the projection the codes were built
 *                with)
 *   out          device, fp32 [batch][Hq][d] (output; 0 for an empty
 *                sequence)
 *   sel_idx      optional (may be NULL) device, int32
 *                [batch][Hkv][top_k+window+sinks]: selected logical
 *                positions, order within a list unspecified, -1 past the
 *                count
 *   sel_cnt      optional (may be NULL) device, int32 [batch][Hkv]:
 *                min(N, sinks+window+top_k)
 *   workspace    device, at least dkv_decode_workspace_size(cfg, batch,
 *                max_seq_len) bytes, 256-byte aligned
 * The selection is bit-exact with the definition above (ties in S go to
 * the lowest position); `out` is within |err| <= 2e-3 + 1e-2*|exact|.
 */
dkv_status dkv_decode(const dkv_config *cfg, const void *q,
                      const void *k_pool, const void *v_pool,
                      const uint32_t *codes, const uint8_t *radii,
                      int64_t num_blocks, const int32_t *block_table,
                      int32_t max_blocks_per_seq, const int32_t *seq_lens,
                      int32_t batch, int32_t max_seq_len, const void *proj,
                      float *out, int32_t *sel_idx, int32_t *sel_cnt,
                      void *workspace, size_t workspace_bytes,
                      dkv_stream_t stream);

/*
 * dkv_decode_debug -- dkv_decode plus two inspection outputs, for parity
 * tests (it moves more bytes than dkv_decode; do not time it):
 *   q8_out      optional device, int8 [batch][Hq][b]: the query codes
 *   scores_out  optional device, int32 [batch][Hkv][max_seq_len]: S of every
 *               cached key (entries at positions >= N are not written)
 */
dkv_status dkv_decode_debug(const dkv_config *cfg, const void *q,
                            const void *k_pool, const void *v_pool,
                            const uint32_t *codes, const uint8_t *radii,
                            int64_t num_blocks, const int32_t *block_table,
                            int32_t max_blocks_per_seq,
                            const int32_t *seq_lens, int32_t batch,
                            int32_t max_seq_len, const void *proj, float *out,
                            int32_t *sel_idx, int32_t *sel_cnt, void *workspace,
                            size_t workspace_bytes, int8_t *q8_out,
                            int32_t *scores_out, dkv_stream_t stream);

/*
 * dkv_decode_profiled -- dkv_decode that also records stage_events[i] on
 * `stream` right before decode stage i and stage_events[n] after the last
 * stage, n = dkv_decode_num_stages() (at most DKV_MAX_DECODE_STAGES).  The
 * caller creates the n+1 events (hipEventCreate) and reads the stage times
 * with hipEventElapsedTime after synchronising.  For instrumentation: the
 * event records add a little launch overhead.
 */
#define DKV_MAX_DECODE_STAGES 8
dkv_status dkv_decode_profiled(const dkv_config *cfg, const void *q,
                               const void *k_pool, const void *v_pool,
                               const uint32_t *codes, const uint8_t *radii,
                               int64_t num_blocks, const int32_t *block_table,
                               int32_t max_blocks_per_seq,
                               const int32_t *seq_lens, int32_t batch,
                               int32_t max_seq_len, const void *proj,
                               float *out, int32_t *sel_idx, int32_t *sel_cnt,
                               void *workspace, size_t workspace_bytes,
                               dkv_event_t *stage_events, dkv_stream_t stream);

/*
 * dkv_decode_append -- one decode step that first encodes each sequence's
 * newest key: for every sequence s with N = seq_lens[s] >= 1 and every KV
 * head, the key at position N-1 (already written to k_pool by the caller)
 * gets its code and radius in codes/radii exactly as dkv_encode over
 * [N-1, N) would write them, then the step runs as dkv_decode.  The
 * encode happens inside the decode's first kernel, so a decode step costs
 * one call and no extra launch ([SPHERICAL KV, §2.3]: dense keys are
 * mapped to codes as they are written to the paged cache).
 *   codes, radii  device, written at position N-1 of every sequence
 *   stage_events  optional (NULL: none), as for dkv_decode_profiled
 * Every other argument and every output as for dkv_decode.  Positions
 * before N-1 must already hold their codes.
 */
dkv_status dkv_decode_append(const dkv_config *cfg, const void *q,
                             const void *k_pool, const void *v_pool,
                             uint32_t *codes, uint8_t *radii,
                             int64_t num_blocks, const int32_t *block_table,
                             int32_t max_blocks_per_seq,
                             const int32_t *seq_lens, int32_t batch,
                             int32_t max_seq_len, const void *proj,
                             float *out, int32_t *sel_idx, int32_t *sel_cnt,
                             void *workspace, size_t workspace_bytes,
                             dkv_event_t *stage_events, dkv_stream_t stream);

/*
 * dkv_decode_append_noalloc -- dkv_decode_append for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the workspace is the library's
 * own static device array of DKV_NOALLOC_SCRATCH_BYTES bytes (one per GPU,
 * held until the process ends) instead of a caller buffer.
 *   Arguments and outputs as for dkv_decode_append, without workspace and
 *   stage events; call it with the stream's device current.
 *   The call allocates nothing (no hipMalloc, hipFree or allocating library
 *   routine).  Its first call on a device looks up that device's copy of
 *   the array (hipGetSymbolAddress); DKV_ERR_LAUNCH if that fails.
 *   DKV_ERR_WORKSPACE when dkv_decode_workspace_size(cfg, batch,
 *   max_seq_len) exceeds DKV_NOALLOC_SCRATCH_BYTES (for example 16 x 128K
 *   tokens of 8 KV heads; about 64 (sequence, KV head) pairs of 128K tokens
 *   fit).  The array needs no initialisation.
 *   Every call on one GPU uses that GPU's single array: calls that overlap
 *   on one GPU (concurrent streams, or threads) race and give undefined
 *   results; serialise them on one stream.
 */
#define DKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
dkv_status dkv_decode_append_noalloc(const dkv_config *cfg, const void *q,
                                     const void *k_pool, const void *v_pool,
                                     uint32_t *codes, uint8_t *radii,
                                     int64_t num_blocks,
                                     const int32_t *block_table,
                                     int32_t max_blocks_per_seq,
                                     const int32_t *seq_lens, int32_t batch,
                                     int32_t max_seq_len, const void *proj,
                                     float *out, int32_t *sel_idx,
                                     int32_t *sel_cnt, dkv_stream_t stream);

/*
 * Multi-table LSH candidate retrieval ([DASH], "from quadratic to linear":
 * several hash tables split the space into buckets; a query looks only in
 * its own buckets, and the candidates found there are pruned to the top-k
 * that enter exact attention).
 *
 * Definition (with T = lsh_tables, m = lsh_bits, W = b/32):
 *   bucket of a key in table t   code bits t*m .. t*m+m-1 (bit t*m+i is
 *                                bit i of the bucket number)
 *   bucket of query head h       the same bits of the query's own sign
 *                                code: bit j = [p_hj > 0], p_h = q_h.P in
 *                                double precision, index order (the key
 *                                code's definition applied to q_h)
 *   candidates                   keys in [sigma, N-w) that share a bucket
 *                                with some head of the KV group in some
 *                                table
 *   selection                    sinks + window + the min(top_k,
 *                                candidates) best candidates by
 *                                (S descending, position ascending)
 *
 * The index is an acceleration structure only: keys at positions it does
 * not hold (appended after dkv_lsh_build) are tested directly, so the
 * result never depends on when the index was built.
 *
 * dkv_lsh_index_size -- bytes of the index for `batch` sequences of at most
 * max_seq_len tokens (0 on invalid arguments or lsh_tables == 0).
 */
size_t dkv_lsh_index_size(const dkv_config *cfg, int32_t batch,
                          int32_t max_seq_len);

/*
 * dkv_lsh_build -- (re)builds the bucket index of positions
 * [0, seq_lens[s]) of every sequence s from the codes dkv_encode wrote.
 *   codes, num_blocks, block_table, max_blocks_per_seq, batch, seq_lens,
 *   max_seq_len   as for dkv_decode (seq_lens on the device)
 *   index         device, dkv_lsh_index_size(cfg, batch, max_seq_len)
 *                 bytes, 256-byte aligned; owned by the caller, read by
 *                 dkv_decode_lsh with the same cfg, batch and max_seq_len.
 *                 Layout per (sequence, KV head): the indexed length, then
 *                 per table bucket offsets [2^m + 1] and positions
 *                 [max_seq_len] (int32), grouped by bucket.
 * Errors as dkv_decode (DKV_ERR_WORKSPACE for a short or misaligned index).
 */
dkv_status dkv_lsh_build(const dkv_config *cfg, const uint32_t *codes,
                         int64_t num_blocks, const int32_t *block_table,
                         int32_t max_blocks_per_seq, int32_t batch,
                         const int32_t *seq_lens, int32_t max_seq_len,
                         void *index, size_t index_bytes, dkv_stream_t stream);

/*
 * dkv_decode_lsh -- dkv_decode with the LSH candidate selection above
 * (cfg->lsh_tables > 0; max_seq_len <= 2^19).  Arguments as dkv_decode,
 * plus the index built by dkv_lsh_build and optional stage_events as in
 * dkv_decode_append (the bucket probe counts to the score stage).
 * sel_cnt = min(N, sinks + window) + min(top_k, candidates).
 */
dkv_status dkv_decode_lsh(const dkv_config *cfg, const void *q,
                          const void *k_pool, const void *v_pool,
                          const uint32_t *codes, const uint8_t *radii,
                          int64_t num_blocks, const int32_t *block_table,
                          int32_t max_blocks_per_seq, const int32_t *seq_lens,
                          int32_t batch, int32_t max_seq_len, const void *proj,
                          const void *index, size_t index_bytes, float *out,
                          int32_t *sel_idx, int32_t *sel_cnt, void *workspace,
                          size_t workspace_bytes, dkv_event_t *stage_events,
                          dkv_stream_t stream);

/* Number of decode stages and the static name of stage i ("" if out of
 * range). */
int32_t dkv_decode_num_stages(void);
const char *dkv_decode_stage_name(int32_t stage);

/* Static, NUL-terminated description of a status code. */
const char *dkv_status_string(dkv_status status);

/* ABI version of this header (bumped on any signature or layout change). */
#define DKV_ABI_VERSION 6
int32_t dkv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DKV_H_ */
