// qprep.hip -- int8 query codes for one decode step, and the matrix-core
// operand the score kernel multiplies them with.
//
// [DASH-KV, asymmetric hashing / dynamic mixed precision]: the query side
// keeps the deeper, higher-precision encoder.  Here: p_hj = q_h . P_:j in
// double precision, index order; one symmetric scale per (sequence, KV
// group): M = max |p| over the group's G heads and all b columns;
// q8 = round_half_even((p * 127) / M) clamped to +-127 (0 when M == 0).
//
// Score operand.  The score kernel computes, per key and query head,
//   D_h = sum_j q8_hj * bit_j   on a 16x16x128 fp8 x fp4 matrix core op,
// with s_h = 2 D_h - Q_h, Q_h = sum_j q8_hj.  The code bits enter as fp4
// nibbles (see score.hip: the nibble for bit j carries the value f_m, m =
// j mod 4, f = {0.5, 1, 2, 0.5}); the query enters as fp8 (e4m3) rows
// 2h (high part) and 2h+1 (low part) with q8 = 16*hi + lo, hi in [-8,7],
// lo in [0,15], each pre-multiplied by 2/f_m so every product is the exact
// even integer 2*hi*bit or 2*lo*bit.  All values are integers of at most
// four significant bits, so they are exact in e4m3 and every partial sum is
// exact in fp32.
//
// Register layout of the 16x16x128 f8f6f4 operation on gfx950 (measured):
//   fp8 operand: lane L holds row L%16; byte p of its 8 dwords is
//     k = 16*(L/16) + p (p < 16) or 64 + 16*(L/16) + (p-16) (p >= 16);
//   fp4 operand: lane L holds column L%16; nibble p of its 4 dwords is
//     k = 32*(L/16) + p;
//   result: lane L holds rows 4*(L/16)+i, i = 0..3, of column L%16.
// The code word (4*ks + L/16) of key L%16 expands into nibble slots
// p = 8m + e <-> bit j = 32*(4*ks + L/16) + 4e + m.
//
// Candidate threshold.  The same workgroup then scores a deterministic
// sample of the (sequence, KV head)'s candidate pages -- every SP-th page
// from the first candidate page, SP the largest power of two <= 64 with
// 2*SP <= k_eff/16 (about 64 sampled keys at the cut), doubled while the
// sample would hold more than 512 pages -- and sets L from the k_s-th
// largest sampled biased score, k_s = ceil(2 * k_eff * n_sample /
// n_candidates), so about 2*k_eff keys are expected to reach L.  The streaming pass keeps every key
// with u >= L; the merge checks that at least k_eff did (then the exact
// top-k is among them) and otherwise rescans exactly.  L = 0 keeps every
// candidate (used when k_eff covers all of them or the sample is too small
// to say more).
#include <type_traits>

// Window attention.  The window rows of a (sequence, KV head) are part of
// its list whatever the scores are ([DeepSeek CSA]: the sliding window of
// recent tokens is kept), so when the units leave compute units free, the
// launch carries one more workgroup per unit that attends over them,
// beside the prep workgroups, and leaves its state as the unit's first
// attention split.  (The few sink rows go with the top-k rows: with them a
// 512-row window would not split into whole tiles over the eight waves.)
#include "attend_common.h"
#include "encode_common.h"
#include "score_common.h"
#include "select_common.h"

namespace dkv {
namespace {

constexpr int kThreads = 512;
constexpr int kMaxPairs = 4;      // G*b <= 8*256 = 4*512
constexpr int kSamplePages = 512; // sample pages per (sequence, KV head)
constexpr int kWv = kThreads / 64;
constexpr int kWavePages = kSamplePages / kWv; // sample pages per wave (<= 64)
constexpr int kWaveQuads = kWavePages / 4;     // their page quads
static_assert(kWavePages <= 64, "one page per lane");

// e4m3 (bias 7) byte of a small integer v, |v| <= 60 with at most four
// significant bits (exactly representable).
__device__ __forceinline__ uint32_t e4m3_of_int(int v) {
  if (v == 0) return 0u;
  const uint32_t sign = v < 0 ? 0x80u : 0u;
  const uint32_t a = (uint32_t)(v < 0 ? -v : v);
  const int e = 31 - __clz(a);                 // floor(log2 a)
  const uint32_t mant = ((a << 3) >> e) - 8u;  // 3 fraction bits, exact
  return sign | ((uint32_t)(e + 7) << 3) | mant;
}

// window tiles of a wave whose rows are in flight together (fewer at G = 8,
// whose accumulators take 64 registers), and the batches whose row ids are
// requested at the start
template <int G> constexpr int kWinBatch = G <= 4 ? 4 : 2;
constexpr int kWinIdBatches = 2;

// The workgroup of unit `unit` that attends over its window rows (the
// positions [ws, N)): wave v takes their 16-row tiles v, v + 8, v + 16,
// ..., kWinBatch<G> tiles' rows requested at once; the eight wave states
// merge in LDS (scratch, >= 38 KB) into part split 0.
template <int G>
__device__ __forceinline__ void window_attend(
    int unit, const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_pool,
    const uint16_t *__restrict__ v_pool, const int32_t *__restrict__ block_table,
    int max_blocks, int64_t num_blocks, const int32_t *__restrict__ seq_lens, int n_max,
    int Hq, int Hkv, int w, int sigma, float *__restrict__ part, int nsplit,
    uint32_t *scratch) {
  constexpr int nb = kWinBatch<G>;
  const int s = unit / Hkv, g = unit % Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int N = seq_len_clamped(seq_lens, s, n_max);
  const SinkWindow sw(N, w, sigma);
  const int nwin = N - sw.ws;
  const int nt = (nwin + kAttnTileRows - 1) / kAttnTileRows;
  const int ntw = nt > wave ? (nt - wave + kWv - 1) / kWv : 0; // this wave's tiles
  auto sp = reinterpret_cast<float(*)[kAttnTileRows][kAttnPStride]>(scratch);
  auto sc = reinterpret_cast<float(*)[kAttnPStride]>(scratch + kWv * kAttnTileRows * kAttnPStride);
  auto sm = reinterpret_cast<float(*)[G][kAttnPartStride]>(
      scratch + kWv * (kAttnTileRows + 1) * kAttnPStride);
  const int32_t *bt = block_table + (int64_t)s * max_blocks;
  // Row ids, one per lane: register q of batch j holds in lane L row L%16
  // of the wave's tile nb*j + 4q + L/16 (-1 for none).  Loads at clamped
  // in-bounds addresses; unused values are dropped where used.
  constexpr int nq = (nb + 3) / 4;
  auto tile_of = [&](int j, int qq) { return nb * j + 4 * qq + lane / kAttnTileRows; };
  auto row_of = [&](int jt) { return (wave + kWv * jt) * kAttnTileRows + lane % kAttnTileRows; };
  auto id_load = [&](int j, int qq) {
    return bt[clamp_int(sw.ws + row_of(tile_of(j, qq)), 0, max(N - 1, 0)) / kPage];
  };
  auto row_id = [&](int j, int qq, int raw) {
    const int jt = tile_of(j, qq);
    const int r = row_of(jt);
    return (4 * qq + lane / kAttnTileRows < nb && jt < ntw && r < nwin && raw >= 0 &&
            raw < num_blocks)
               ? raw * kPage + (sw.ws + r) % kPage : -1;
  };
  // the first batches' block ids are all requested at once
  int raw[kWinIdBatches][nq];
#pragma unroll
  for (int j = 0; j < kWinIdBatches; ++j)
#pragma unroll
    for (int qq = 0; qq < nq; ++qq) raw[j][qq] = id_load(j, qq);
  AttnWave<G> aw;
  aw.init(q + ((int64_t)s * Hq + (int64_t)g * G) * kHeadDim, lane, sp[wave], sc[wave]);
  const int nbw = (ntw + nb - 1) / nb; // this wave's batches (wave-uniform)
  for (int j = 0; j < nbw; ++j) {
    int ids[nq];
#pragma unroll
    for (int qq = 0; qq < nq; ++qq) {
      int v;
      if (j < kWinIdBatches) { // (unrolled selection: no indexed register array)
        v = raw[0][qq];
#pragma unroll
        for (int i = 1; i < kWinIdBatches; ++i) v = j == i ? raw[i][qq] : v;
      } else {
        v = id_load(j, qq);
      }
      ids[qq] = row_id(j, qq, v);
    }
    uint4 kt[nb][4], vt[nb][4];
    uint32_t ok[nb], vok[nb];
#pragma unroll
    for (int t = 0; t < nb; ++t)
      aw.load_tile(ids[t / 4], (t % 4) * kAttnTileRows, k_pool, v_pool, Hkv, g, kt[t], vt[t],
                   ok[t], vok[t]);
#pragma unroll
    for (int t = 0; t < nb; ++t) aw.use_tile(kt[t], vt[t], ok[t], vok[t]);
  }
  aw.store(sm[wave]);
  __syncthreads();
  attn_merge_waves<G, kWv, kThreads>(sm, part + (int64_t)unit * nsplit * G * kAttnPartStride);
}

// WC: code words per key (b/32: 2, 4 or 8), fixed at compile time so the
// sample loads need no branch on it; KS: 128-bit matrix-core K-steps.
// Workgroups [0, nseq*Hkv) prepare a unit each; with v_pool, workgroups
// [nseq*Hkv, 2*nseq*Hkv) attend over a unit's sinks and window each.
template <int WC, int G, int KS = (WC > 4 ? WC / 4 : 1)>
__global__ __launch_bounds__(kThreads) void prep_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ proj,
    const uint32_t *codes, const uint8_t *radii, const uint16_t *__restrict__ k_pool,
    uint32_t *codes_w, uint8_t *radii_w, // non-null: encode the newest key
    int64_t num_blocks, uint32_t code_bytes, uint32_t radius_bytes,
    const int32_t *__restrict__ block_table, int max_blocks,
    const int32_t *__restrict__ seq_lens, int n_max, int8_t *__restrict__ q8,
    uint32_t *__restrict__ qop, float *__restrict__ qneg,
    uint32_t *__restrict__ lthr, uint32_t *__restrict__ qbits,
    uint32_t *__restrict__ tasks, int Hq, int Hkv, int k, int w,
    int sigma, bool lin, bool pages, int nseq, const uint16_t *__restrict__ v_pool,
    float *__restrict__ part, int nsplit) {
  constexpr int W = WC, b = 32 * WC;
  const int unit = blockIdx.x;
  const int s = unit / Hkv;
  const int g = unit % Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); // uniform
  // the group's query rows as doubles, and P: fp32 for b <= 128, bf16 for
  // b = 256 (64 KB either way); each holds the exact bf16 values
  __shared__ __align__(16) double sQd[8 * kHeadDim];
  __shared__ __align__(16) uint32_t sP[kHeadDim * 128];
  __shared__ int sq8[8 * 256];
  __shared__ uint32_t sOp[2 * 512];
  // each wave's sample radius lines: 16 bytes per page, page order
  __shared__ __align__(16) uint8_t sRad[kWv][kWavePages * kPage];
  __shared__ double sMax[kThreads / 64];
  __shared__ int sSum[8];
  __shared__ uint32_t sCount[3][kThreads / 64];
  __shared__ __align__(16) SelectShared<kThreads> sel;
  __shared__ uint16_t sWlin[256]; // linear radius weights (the sample)
  static_assert(sizeof(sP) >= 4 * kWv * ((kAttnTileRows + 1) * kAttnPStride +
                                         8 * kAttnPartStride),
                "window attention scratch");
  if (unit >= nseq * Hkv) { // workgroup-uniform
    window_attend<G>(unit - nseq * Hkv, q, k_pool, v_pool, block_table, max_blocks,
                     num_blocks, seq_lens, n_max, Hq, Hkv, w, sigma, part, nsplit, sP);
    return;
  }

  // ---- sample plan: every SP-th candidate page from page pc0, nsp pages
  struct Plan {
    int nc, keff, pc0, SP, nsp;
  };
  auto plan_for = [&](int n) {
    Plan P;
    P.nc = max(0, n - w - sigma);
    P.keff = min(k, P.nc);
    P.pc0 = 0;
    P.SP = 1;
    P.nsp = 0;
    if (!pages && qbits == nullptr && P.keff > 0 && P.keff < P.nc) {
      P.pc0 = sigma / kPage;
      const int ncp = (n - w + kPage - 1) / kPage - P.pc0;
      while (P.SP < 64 && 2 * P.SP <= P.keff / 16) P.SP *= 2;
      while ((ncp + P.SP - 1) / P.SP > kSamplePages) P.SP *= 2;
      P.nsp = (ncp + P.SP - 1) / P.SP;
    }
    return P;
  };
  // The loads of this prologue are issued by every thread, at clamped
  // in-bounds addresses, and unused values are dropped only where they are
  // used: a load inside a lane-dependent branch, or a select on a loaded
  // value, makes the compiler wait for it -- and for every load issued
  // before it -- right there.
  //
  // First the sample pages' block ids (the sample loads need them soonest):
  // read with the plan of the longest length (n_max) before the sequence's
  // own length has arrived, and read again only when the sequence's plan
  // differs (ragged batches).  Wave v samples pages t = v + 8*i; lane i
  // holds the block id of its i-th page.
  const int32_t *bt = block_table + (int64_t)s * max_blocks;
  const int tl = wave + kWv * lane;
  const Plan spec = plan_for(n_max);
  // (page pc0 + t*SP < max_blocks for every t < nsp)
  int blk_raw = bt[spec.nsp > 0 ? spec.pc0 + min(tl, spec.nsp - 1) * spec.SP : 0];
  // then P and the group's query rows, into registers
  constexpr int kPLoads = 4 * KS; // uint4 of P per thread (b <= 128 * KS)
  uint4 pv[kPLoads];
  constexpr int pn = kHeadDim * b / 8;
  {
    const uint4 *psrc = reinterpret_cast<const uint4 *>(proj); // 16-byte aligned
#pragma unroll
    for (int r = 0; r < kPLoads; ++r)
      pv[r] = psrc[min((int)threadIdx.x + r * kThreads, pn - 1)];
  }
  const uint4 *qsrc = reinterpret_cast<const uint4 *>(
      q + ((int64_t)s * Hq + (int64_t)g * G) * kHeadDim);
  const uint4 qv4 = qsrc[min((int)threadIdx.x, G * kHeadDim / 8 - 1)];
  // The streaming filter's task list is written by the workgroups of KV
  // head 0: the lengths of the sequences before s (the first kThreads of
  // them, one per thread) are requested now and summed at the end.
  const int len_before_raw = seq_lens[min((int)threadIdx.x, s)];
  const int N = seq_len_clamped(seq_lens, s, n_max);
  const Plan pl = plan_for(N);
  const int nc = pl.nc, keff = pl.keff, pc0 = pl.pc0, SP = pl.SP, nsp = pl.nsp;
  const bool sample = nsp > 0;
  if (SP != spec.SP || pc0 != spec.pc0 || nsp > spec.nsp) // workgroup-uniform
    blk_raw = bt[nsp > 0 ? pc0 + min(tl, nsp - 1) * SP : 0]; // (ragged lengths)

  // ---- append: the workgroup also encodes position N-1 of sequence s for
  // KV head g (the key the caller has just written), as the encode kernel
  // would.  Its row is requested now (three dependent loads: the length,
  // the block id, the row) and used only after the threshold: the newest
  // key lies in the window, and with no window the filter reads its code
  // after this kernel anyway.
  __shared__ __align__(16) double sKd[3 * kHeadDim]; // a copy per wave that needs it
  int a_blk = -1;
  if (codes_w != nullptr && N > 0) { // workgroup-uniform
    const int blk = bt[(N - 1) / kPage];
    if (blk >= 0 && blk < num_blocks) a_blk = blk;
  }
  const int a_slot = (N - 1) % kPage;
  // (block 0 stands in when there is no key to encode; threads past the
  // row's 64 dwords re-read them)
  const uint32_t *krow = reinterpret_cast<const uint32_t *>(
      k_pool + (((int64_t)max(a_blk, 0) * kPage + max(a_slot, 0)) * Hkv + g) * kHeadDim);
  const uint32_t krow_w = krow[threadIdx.x & (kHeadDim / 2 - 1)];

  if ((int)threadIdx.x < G * kHeadDim / 8) {
    const uint32_t w4[4] = {qv4.x, qv4.y, qv4.z, qv4.w};
    double2 *dst = reinterpret_cast<double2 *>(sQd + 8 * threadIdx.x);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      dst[u] = make_double2((double)bf16_to_float(w4[u] & 0xFFFFu),
                            (double)bf16_to_float(w4[u] >> 16));
  }
#pragma unroll
  for (int r = 0; r < kPLoads; ++r) {
    const int i = (int)threadIdx.x + r * kThreads;
    if (i < pn) {
      if (KS == 1) { // 8 columns as fp32
        const uint32_t w4[4] = {pv[r].x, pv[r].y, pv[r].z, pv[r].w};
        uint4 *dst = reinterpret_cast<uint4 *>(sP + 8 * i);
        dst[0] = make_uint4(w4[0] << 16, w4[0] & 0xFFFF0000u, w4[1] << 16, w4[1] & 0xFFFF0000u);
        dst[1] = make_uint4(w4[2] << 16, w4[2] & 0xFFFF0000u, w4[3] << 16, w4[3] & 0xFFFF0000u);
      } else {
        reinterpret_cast<uint4 *>(sP)[i] = pv[r];
      }
    }
  }
  if (threadIdx.x < 8) sSum[threadIdx.x] = 0;
  if (lin) fill_linear_weights(sWlin, kThreads); // (workgroup-uniform)
  __syncthreads();

  // ---- the sample pages' loads, in flight while the query is projected
  // (issued after the staging barrier: their addresses need the block ids,
  // which have arrived by now, while waiting for those ids earlier would
  // also have waited for every load issued before them).
  // Page quads as in the streaming filter: lane 16j+c loads the code words
  // of key c of page 4a+j of the wave; lane i loads the radius line of page
  // i.  Pages past the wave's share or with an invalid block id read past
  // the pools (zeros) and count as no sample.
  const int npw = sample ? (nsp - wave + kWv - 1) / kWv : 0; // wave-uniform
  const uint32_t ph_none = (uint32_t)(num_blocks * Hkv);
  const uint32_t ph_l = (lane < npw && blk_raw >= 0 && blk_raw < num_blocks)
                            ? (uint32_t)blk_raw * (uint32_t)Hkv + (uint32_t)g : ph_none;
  const uint32_t page_bytes = (uint32_t)(kPage * W * 4);
  const uint32_t key_byte = (uint32_t)((lane & 15) * W * 4);
  const __amdgpu_buffer_rsrc_t code_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t *>(codes), 0, code_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rad_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(radii), 0, radius_bytes, kBufferWord3);
  // (Issued by every workgroup: with no sample npw is 0, so every page id
  // is ph_none and the loads read zeros.  Under a branch, the copies of the
  // loaded values at its end would wait for the loads right there.)
  uint32_t qx[kWaveQuads][KS][4];
  uint4 rline;
  {
    const auto rv = __builtin_amdgcn_raw_buffer_load_b128(rad_rsrc, (int)(ph_l * (uint32_t)kPage), 0, 0);
    rline = make_uint4(rv[0], rv[1], rv[2], rv[3]);
    auto load_quad = [&](int a) __attribute__((always_inline)) {
      const uint32_t mine = (uint32_t)__shfl((int)ph_l, 4 * a + (lane >> 4));
      const int voff = (int)(mine * page_bytes + key_byte);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (W == 2) {
          const auto v = __builtin_amdgcn_raw_buffer_load_b64(code_rsrc, voff, 0, 0);
          qx[a][ks][0] = v[0];
          qx[a][ks][1] = v[1];
          qx[a][ks][2] = 0u;
          qx[a][ks][3] = 0u;
        } else {
          const auto v = __builtin_amdgcn_raw_buffer_load_b128(code_rsrc, voff + 16 * ks, 0, 0);
          qx[a][ks][0] = v[0];
          qx[a][ks][1] = v[1];
          qx[a][ks][2] = v[2];
          qx[a][ks][3] = v[3];
        }
      }
    };
    // The first half of the quads are loaded unconditionally (pages past the
    // wave's share read zeros), the second half, under one branch, only when
    // the sample needs them (its loaded words are copied, and so waited for,
    // at the branch's end).
#pragma unroll
    for (int a = 0; a < kWaveQuads / 2; ++a) load_quad(a);
    if (npw > 2 * kWaveQuads) { // wave-uniform
#pragma unroll
      for (int a = kWaveQuads / 2; a < kWaveQuads; ++a) load_quad(a);
    }
  }

  // p_hj in double precision, index order (one chain per (h, j) pair).
  // P_ij (exact in fp32 or as bf16) and q_hi (a double in LDS, the same for
  // the whole wave) go into one fused multiply-add per term: the product of
  // two bf16 values is exact in double, so this is the definition's chain.
  // Batches of 8 terms: the next batch's LDS reads are issued before the
  // current batch's multiply-adds, which stay in index order.
  const int npairs = G * b;
  // P_ij as a double
  auto p_at = [&](int i, int j) -> double {
    if (KS == 1) return (double)__uint_as_float(sP[i * b + j]);
    const uint16_t *ph = reinterpret_cast<const uint16_t *>(sP);
    return (double)bf16_to_float(ph[i * b + j]);
  };
  // sum_i x_i P_ij in index order, x a row of doubles in LDS
  auto chain = [&](const double *x, int j) -> double {
    double pa[8], xa[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      pa[u] = p_at(u, j);
      xa[u] = x[u];
    }
    double acc = 0.0;
#pragma unroll 2
    for (int i0 = 0; i0 < kHeadDim; i0 += 8) {
      double pn[8], xn[8];
      const int i1 = i0 + 8 < kHeadDim ? i0 + 8 : i0; // last batch reloads itself
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        pn[u] = p_at(i1 + u, j);
        xn[u] = x[i1 + u];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc = fma(xa[u], pa[u], acc);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        pa[u] = pn[u];
        xa[u] = xn[u];
      }
    }
    return acc;
  };
  // The query chains: thread t < HS*b runs the CPT chains of column
  // j = t % b for heads (t / b) * CPT ..., each term's P_ij read and
  // widened once for all of them (same terms, same order, same fused
  // multiply-add per chain); HS = 2 keeps a wave on every SIMD.  The
  // results go through LDS (the threshold histogram's space, cleared after)
  // to the pair layout below: pair idx = h*b + j in thread idx % kThreads.
  constexpr int HS = (G >= 2 && 2 * b <= kThreads) ? 2 : 1;
  constexpr int CPT = G / HS;
  double *hand = reinterpret_cast<double *>(sel.hist); // G*b <= 2048 doubles
  static_assert(G * b * sizeof(double) <= sizeof(sel.hist), "hand-off space");
  // The newest key's code (append): its projection chains (one column a
  // thread) and its |k|^2 chain run on the waves past the query chains when
  // there are enough of them (b <= 128), each wave with its own copy of the
  // row in LDS; otherwise on threads 0..b after the threshold.
  constexpr int kKeyEarly0 = HS * b;
  constexpr bool kKeyEarly = kKeyEarly0 + b + 64 <= kThreads;
  constexpr int kKey0 = kKeyEarly ? kKeyEarly0 : 0; // the key's first thread
  uint64_t key_bits = 0;
  double r2 = 0.0;
  if ((int)threadIdx.x < HS * b) { // whole waves (b is a multiple of 64)
    const int j = (int)threadIdx.x % b, h0 = ((int)threadIdx.x / b) * CPT;
    double acc[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[c] = 0.0;
    constexpr int kUnroll = CPT >= 4 ? 4 : 8;
#pragma unroll kUnroll
    for (int i = 0; i < kHeadDim; ++i) {
      const double pij = p_at(i, j);
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc[c] = fma(sQd[(h0 + c) * kHeadDim + i], pij, acc[c]);
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) hand[(h0 + c) * b + j] = acc[c];
  } else if (kKeyEarly && a_blk >= 0 && (int)threadIdx.x < kKey0 + b + 64) { // whole waves
    double *kd = sKd + (((int)threadIdx.x - kKey0) / 64) * kHeadDim;
    kd[2 * lane] = (double)bf16_to_float(krow_w & 0xFFFFu);
    kd[2 * lane + 1] = (double)bf16_to_float(krow_w >> 16);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if ((int)threadIdx.x < kKey0 + b) {
      const double pk = chain(kd, (int)threadIdx.x - kKey0);
      key_bits = __ballot(pk > 0.0); // columns of this wave's 64 threads
    } else if ((int)threadIdx.x == kKey0 + b) {
      for (int i = 0; i < kHeadDim; ++i) r2 = fma(kd[i], kd[i], r2);
    }
  }
  __syncthreads();
  double p[kMaxPairs];
  double mloc = 0.0;
#pragma unroll
  for (int r = 0; r < kMaxPairs; ++r) {
    const int idx = threadIdx.x + r * kThreads;
    p[r] = idx < npairs ? hand[idx] : 0.0;
    mloc = fmax(mloc, fabs(p[r]));
  }
  // the query heads' own sign codes (LSH buckets): pair idx = h*b + j
  uint64_t qsign[kMaxPairs];
#pragma unroll
  for (int r = 0; r < kMaxPairs; ++r) qsign[r] = __ballot(p[r] > 0.0);
  mloc = wave_max_nonneg_f64(mloc);
  if (lane == 0) sMax[wave] = mloc;
  __syncthreads();
  double M = sMax[0];
  for (int i = 1; i < kThreads / 64; ++i) M = fmax(M, sMax[i]);
  // the threshold histogram, cleared for its first use (the hand-off reads
  // are behind the barrier above)
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) sel.hist[i] = 0;

  // Global stores wait until the end of the kernel: a barrier would
  // otherwise wait for them to complete.
  int qv[kMaxPairs];
#pragma unroll
  for (int r = 0; r < kMaxPairs; ++r) {
    const int idx = threadIdx.x + r * kThreads;
    qv[r] = 0;
    if (idx < npairs) { // wave-uniform: npairs and b are multiples of 64
      int v = 0;
      if (M != 0.0) {
        const double scaled = p[r] * 127.0;
        const double ratio = scaled / M;
        v = (int)fmin(127.0, fmax(-127.0, rint(ratio)));
      }
      qv[r] = v;
      sq8[idx] = v;
      const int sum = (int)wave_sum_u32((uint32_t)v); // one head per wave
      if (lane == 0) atomicAdd(&sSum[idx / b], sum);
    }
  }
  __syncthreads();

  // matrix-core operand dwords: [KS][64 lanes][8 dwords]
  constexpr int kOpWords = KS * 64 * 8;
  uint32_t opw[kOpWords / kThreads];
#pragma unroll
  for (int r = 0; r < kOpWords / kThreads; ++r) {
    const int t = threadIdx.x + r * kThreads;
    const int ks = t / 512, la = (t / 8) % 64, di = t % 8;
    const int row = la % 16, gA = la / 16;
    const int h = row / 2, part = row % 2;
    uint32_t word = 0;
    if (h < G) {
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        const int pA = 4 * di + bi;
        const int kk = pA < 16 ? 16 * gA + pA : 64 + 16 * gA + (pA - 16);
        const int tt = kk / 32, pp = kk % 32, m = pp / 8, e = pp % 8;
        const int j = 32 * (4 * ks + tt) + 4 * e + m;
        int v = 0;
        if (j < b) {
          const int qv = sq8[h * b + j];
          const int x = part == 0 ? (qv >> 4) : (qv & 15);
          v = (m == 2) ? x : (m == 1 ? 2 * x : 4 * x);  // 2x / f_m
        }
        word |= e4m3_of_int(v) << (8 * bi);
      }
    }
    opw[r] = word;
    sOp[t] = word;
  }
  __syncthreads();

  // ---- candidate threshold from the page sample
  // L = ~0 asks for no candidates (k_eff = 0, or every candidate is
  // selected and the merge marks them directly)
  uint32_t L = 0xFFFFFFFFu;
  if (sample) { // workgroup-uniform
    L = 0;
    QueryOperand<KS> op;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i) op.a[ks][i] = (int)sOp[(ks * 64 + lane) * 8 + i];
    {
      const int h0 = 2 * (lane >> 4), h1 = h0 + 1;
      op.cinit = v4f{0.f, h0 < G ? -(float)sSum[h0 < G ? h0 : 0] : 0.f, 0.f,
                     h1 < G ? -(float)sSum[h1 < G ? h1 : 0] : 0.f};
      op.scale = unit_scale();
    }
    // the wave's radius lines, page order, read back one byte per lane
    *reinterpret_cast<uint4 *>(&sRad[wave][16 * lane]) = rline;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // Score the wave's quads: after the transpose, lane L holds key L%16 of
    // page 4a + L/16.  us[a]: its biased score, 0 when it is no valid sample
    // key (a biased score is never 0).
    uint32_t us[kWaveQuads];
    uint32_t nvalid = 0, vlo = 0xFFFFFFFFu, vhi = 0u;
#pragma unroll
    for (int a = 0; a < kWaveQuads; ++a) {
      us[a] = 0u;
      if (4 * a < npw) { // wave-uniform
        uint32_t cw[4][KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          uint32_t x[4] = {qx[a][ks][0], qx[a][ks][1], qx[a][ks][2], qx[a][ks][3]};
          transpose_rows(x);
#pragma unroll
          for (int j = 0; j < 4; ++j) cw[j][ks] = x[j];
        }
        // (256-bit codes: the pages one after another, for the registers)
        const int mx = KS > 1 ? score_quad_max_seq<KS, G>(op, cw) : score_quad_max<KS, G>(op, cw);
        const uint32_t r8 = sRad[wave][64 * a + lane];
        const int i = 4 * a + (lane >> 4);        // the wave's page index
        const int pos = (pc0 + (wave + kWv * i) * SP) * kPage + (lane & 15);
        const uint32_t ph_i = (uint32_t)__shfl((int)ph_l, i);
        const bool valid = i < npw && ph_i != ph_none && pos >= sigma && pos < N - w;
        const uint32_t u = biased_score(__mul24(radius_weight_lut(r8, lin, sWlin), mx));
        if (valid) {
          us[a] = u;
          nvalid += 1;
          vlo = min(vlo, u);
          vhi = max(vhi, u);
        }
      }
    }
    // the count and range of the valid sample keys over the workgroup
    nvalid = wave_sum_u32(nvalid);
    wave_min_max(vlo, vhi);
    if (lane == 0) {
      sCount[0][wave] = nvalid;
      sCount[1][wave] = vlo;
      sCount[2][wave] = vhi;
    }
    __syncthreads();
    uint32_t ns = 0, lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int i = 0; i < kWv; ++i) {
      ns += sCount[0][i];
      lo = min(lo, sCount[1][i]);
      hi = max(hi, sCount[2][i]);
    }
    const uint32_t ks_take = (uint32_t)min((int64_t)ns,
        ((int64_t)2 * keff * ns + nc - 1) / nc);
    if (ks_take > 0 && ks_take < ns) { // workgroup-uniform
      // L = the lower edge of the histogram bin (over (u - lo) >> shift,
      // 4096 bins spanning the sample's range) that holds the ks_take-th
      // largest sample key, so at least ks_take of them reach L
      const uint32_t range = hi - lo;
      const int bits = range == 0 ? 0 : 32 - __clz(range);
      const int shift = bits > kHistBits ? bits - kHistBits : 0;
#pragma unroll
      for (int a = 0; a < kWaveQuads; ++a)
        if (us[a] != 0u) atomicAdd(&sel.hist[(us[a] - lo) >> shift], 1u);
      __syncthreads();
      find_threshold_bin<kThreads>(sel, ks_take);
      L = lo + ((uint32_t)sel.bin << shift);
    }
  }
  if (pages) {
    // page-granular selection: every page meeting [sigma, N - w) is a
    // candidate (L = 0) unless none or all of them are selected
    const int c0 = sigma, c1 = N - w;
    const int npc = c1 > c0 ? (c1 + kPage - 1) / kPage - c0 / kPage : 0;
    const int kp = min(k / kPage, npc);
    L = (kp > 0 && kp < npc) ? 0u : 0xFFFFFFFFu;
  }
  // ---- the newest key's code, if not taken above: threads 0..b-1 run the
  // chain of column j = thread, and thread b |k|^2 (squares summed in index
  // order)
  const bool key_wave = a_blk >= 0 && (int)threadIdx.x >= kKey0 &&
                        (int)threadIdx.x < kKey0 + b; // wave-uniform
  if (!kKeyEarly && a_blk >= 0) { // workgroup-uniform
    if (threadIdx.x < kHeadDim / 2) {
      sKd[2 * threadIdx.x] = (double)bf16_to_float(krow_w & 0xFFFFu);
      sKd[2 * threadIdx.x + 1] = (double)bf16_to_float(krow_w >> 16);
    }
    __syncthreads();
    if (key_wave) {
      const double pk = chain(sKd, (int)threadIdx.x);
      key_bits = __ballot(pk > 0.0); // columns 64*wave .. 64*wave+63
    } else if ((int)threadIdx.x == b) { // the first thread past them: |k|^2
      for (int i = 0; i < kHeadDim; ++i) r2 = fma(sKd[i], sKd[i], r2);
    }
  }
  if (threadIdx.x == 0) lthr[unit] = qbits != nullptr ? 0u : L;
  if (qbits != nullptr) {
#pragma unroll
    for (int r = 0; r < kMaxPairs; ++r) {
      const int idx0 = wave * 64 + r * kThreads; // this wave's 64 pairs
      if (idx0 < npairs && lane < 2) {            // npairs, b: multiples of 64
        const int h = idx0 / b, j0 = idx0 % b;
        qbits[((int64_t)s * Hq + (int64_t)g * G + h) * (b / 32) + j0 / 32 + lane] =
            lane ? (uint32_t)(qsign[r] >> 32) : (uint32_t)qsign[r];
      }
    }
  }
  int8_t *qo = q8 + ((int64_t)s * Hq + (int64_t)g * G) * b;
#pragma unroll
  for (int r = 0; r < kMaxPairs; ++r) {
    const int idx = threadIdx.x + r * kThreads;
    if (idx < npairs) qo[idx] = (int8_t)qv[r];
  }
  uint32_t *dst = qop + (int64_t)unit * kOpWords;
#pragma unroll
  for (int r = 0; r < kOpWords / kThreads; ++r) dst[threadIdx.x + r * kThreads] = opw[r];
  if (threadIdx.x < G)
    qneg[(int64_t)s * Hq + (int64_t)g * G + threadIdx.x] = -(float)sSum[threadIdx.x];
  if (key_wave) {
    const int W32 = b / 32;
    uint32_t *cw = codes_w + (((int64_t)a_blk * Hkv + g) * kPage + a_slot) * W32;
    if (lane < 2)
      cw[2 * (((int)threadIdx.x - kKey0) / 64) + lane] =
          lane ? (uint32_t)(key_bits >> 32) : (uint32_t)key_bits;
  }
  if (a_blk >= 0 && (int)threadIdx.x == kKey0 + b)
    radii_w[((int64_t)a_blk * Hkv + g) * kPage + a_slot] = (uint8_t)radius_code(r2);
  // ---- the filter's task list: one entry (sequence, page group, length)
  // per group of kGroupKeys keys, sequence by sequence, after a count word
  // (padded to 16 bytes).  Only groups that hold keys are listed, so the
  // filter's waves share the real work evenly in ragged batches.
  if (g == 0) { // workgroup-uniform
    auto groups_of = [](int n) { return (uint32_t)((n + kGroupKeys - 1) / kGroupKeys); };
    const int len_before = (int)threadIdx.x < s ? len_before_raw : 0;
    uint32_t local = groups_of(clamp_int(len_before, 0, n_max));
    for (int i = (int)threadIdx.x + kThreads; i < s; i += kThreads)
      local += groups_of(seq_len_clamped(seq_lens, i, n_max));
    __shared__ uint32_t sTaskTmp[kThreads / 64];
    uint32_t before;
    (void)wg_exclusive_scan<kThreads>(local, sTaskTmp, &before);
    const uint32_t ng = groups_of(N);
    uint4 *entries = reinterpret_cast<uint4 *>(tasks + 4);
    for (uint32_t j = threadIdx.x; j < ng; j += kThreads)
      entries[before + j] = make_uint4((uint32_t)s, j, (uint32_t)N, 0u);
    if (s == nseq - 1 && threadIdx.x == 0) tasks[0] = before + ng;
  }
}

} // namespace

hipError_t launch_prep(const DecodeDims &d, const uint16_t *q,
                       const uint16_t *proj, const uint32_t *codes,
                       const uint8_t *radii, const uint16_t *k_pool,
                       const uint16_t *v_pool, uint32_t *codes_w, uint8_t *radii_w,
                       const int32_t *block_table,
                       const int32_t *seq_lens, int8_t *q8, uint32_t *qop,
                       float *qneg, uint32_t *lthr, uint32_t *qbits,
                       uint32_t *tasks, float *part, hipStream_t stream) {
  const int units = d.B * d.Hkv;
  const int nwg = d.window_in_prep ? 2 * units : units;
  const uint32_t code_bytes = (uint32_t)((uint64_t)d.num_blocks * d.Hkv * d.W * kPage * 4);
  const uint32_t radius_bytes = (uint32_t)((uint64_t)d.num_blocks * d.Hkv * kPage);
#define DKV_PREP_CASE(WV, GV)                                                  \
  if (d.W == WV && d.G == GV) {                                                \
    hipLaunchKernelGGL((prep_kernel<WV, GV>), dim3(nwg),                       \
                       dim3(kThreads), 0, stream, q, proj, codes, radii,       \
                       k_pool, codes_w, radii_w,                               \
                       d.num_blocks, code_bytes, radius_bytes, block_table,    \
                       d.max_blocks, seq_lens, d.n_max, q8, qop, qneg, lthr,   \
                       qbits, tasks, d.Hq, d.Hkv, d.k, d.w, d.sigma, d.lin,    \
                       d.pages, d.B, v_pool, part, d.nsplit);                  \
    return hipGetLastError();                                                  \
  }
  DKV_PREP_CASE(2, 1)
  DKV_PREP_CASE(2, 2)
  DKV_PREP_CASE(2, 4)
  DKV_PREP_CASE(2, 8)
  DKV_PREP_CASE(4, 1)
  DKV_PREP_CASE(4, 2)
  DKV_PREP_CASE(4, 4)
  DKV_PREP_CASE(4, 8)
  DKV_PREP_CASE(8, 1)
  DKV_PREP_CASE(8, 2)
  DKV_PREP_CASE(8, 4)
  DKV_PREP_CASE(8, 8)
#undef DKV_PREP_CASE
  return hipErrorInvalidValue;
}

} // namespace dkv
