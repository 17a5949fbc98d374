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
// from the first candidate page, SP a power of two <= 32 chosen so the
// sample holds at most 512 pages -- and sets L = the k_s-th largest sampled
// biased score, k_s = ceil(2 * k_eff * n_sample / n_candidates), so about
// 2*k_eff keys are expected to reach L.  The streaming pass keeps every key
// with u >= L; the merge checks that at least k_eff did (then the exact
// top-k is among them) and otherwise rescans exactly.  L = 0 keeps every
// candidate (used when k_eff covers all of them or the sample is too small
// to say more).
#include <type_traits>

#include "encode_common.h"
#include "score_common.h"
#include "select_common.h"

namespace dkv {
namespace {

constexpr int kThreads = 512;
constexpr int kMaxPairs = 4;      // G*b <= 8*256 = 4*512
constexpr int kSamplePages = 512; // sample pages per (sequence, KV head)
constexpr int kSampleKeys = kSamplePages * kPage;
constexpr int kWv = kThreads / 64;
constexpr int kPre = 32; // sample pages per wave whose loads start first

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

template <int KS, int G>
__global__ __launch_bounds__(kThreads) void prep_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ proj,
    const uint32_t *codes, const uint8_t *radii, const uint16_t *__restrict__ k_pool,
    uint32_t *codes_w, uint8_t *radii_w, // non-null: encode the newest key
    int64_t num_blocks, uint32_t code_bytes, uint32_t radius_bytes,
    const int32_t *__restrict__ block_table, int max_blocks,
    const int32_t *__restrict__ seq_lens, int n_max, int8_t *__restrict__ q8,
    uint32_t *__restrict__ qop, float *__restrict__ qneg,
    uint32_t *__restrict__ lthr, uint32_t *__restrict__ qbits,
    uint32_t *__restrict__ tasks, int Hq, int Hkv, int b, int W, int k, int w,
    int sigma, bool lin, bool pages) {
  const int unit = blockIdx.x;
  const int s = unit / Hkv;
  const int g = unit % Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ __align__(16) uint16_t sQ[8 * kHeadDim];
  __shared__ __align__(16) uint16_t sP[kHeadDim * 256];
  __shared__ int sq8[8 * 256];
  __shared__ uint32_t sOp[2 * 512];
  __shared__ uint32_t sSample[kSampleKeys];
  __shared__ double sMax[kThreads / 64];
  __shared__ int sSum[8];
  __shared__ uint32_t sCount[kThreads / 64];
  __shared__ SelectShared<kThreads> sel;

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
      while (P.SP < 32 && 2 * P.SP <= P.keff / 32) P.SP *= 2;
      while ((ncp + P.SP - 1) / P.SP > kSamplePages) P.SP *= 2;
      P.nsp = (ncp + P.SP - 1) / P.SP;
    }
    return P;
  };
  // P and the group's query rows are requested first, into registers: the
  // staging barrier below then waits only for them and not for the sample
  // pages requested after them (loads count down in order).
  constexpr int kPLoads = 4 * KS; // uint4 of P per thread (b <= 128 * KS)
  uint4 pv[kPLoads];
  const int pn = kHeadDim * b / 8;
  {
    const uint4 *psrc = reinterpret_cast<const uint4 *>(proj); // 16-byte aligned
#pragma unroll
    for (int r = 0; r < kPLoads; ++r) {
      const int i = (int)threadIdx.x + r * kThreads;
      pv[r] = i < pn ? psrc[i] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  const uint4 *qsrc = reinterpret_cast<const uint4 *>(
      q + ((int64_t)s * Hq + (int64_t)g * G) * kHeadDim);
  const uint4 qv4 = (int)threadIdx.x < G * kHeadDim / 8 ? qsrc[threadIdx.x]
                                                         : make_uint4(0u, 0u, 0u, 0u);
  // The streaming filter's task list is written by the workgroups of KV
  // head 0: the lengths of the sequences before s (the first kThreads of
  // them, one per thread) are requested now and summed at the end.
  const int len_before = (g == 0 && (int)threadIdx.x < s) ? seq_lens[threadIdx.x] : 0;
  // The sample pages' loads go next so they are in flight while the query
  // is projected.  Their block ids are read with the plan of the longest
  // length (n_max) before the sequence's own length has arrived; when that
  // length gives another stride or start (ragged batches) they are read
  // again.  Wave v samples pages t = v + 8*i; lane i holds the block id of
  // its i-th page.
  const int32_t *bt = block_table + (int64_t)s * max_blocks;
  const int tl = wave + kWv * lane;
  const Plan spec = plan_for(n_max);
  int blk_l = tl < spec.nsp ? bt[spec.pc0 + tl * spec.SP] : -1;
  const int N = seq_len_clamped(seq_lens, s, n_max);
  const Plan pl = plan_for(N);
  const int nc = pl.nc, keff = pl.keff, pc0 = pl.pc0, SP = pl.SP, nsp = pl.nsp;
  const bool sample = nsp > 0;
  if (SP != spec.SP || pc0 != spec.pc0 || nsp > spec.nsp) // workgroup-uniform
    blk_l = tl < nsp ? bt[pc0 + tl * SP] : -1;
  else if (tl >= nsp)
    blk_l = -1;
  const PoolView view = make_pool_view(codes, radii, code_bytes, radius_bytes,
                                       W, Hkv, g, lane);
  uint32_t pcw[kPre][KS], pr8[kPre];
  uint32_t pokm = 0; // bit u: preloaded page u is a valid sample page
  static_assert(kPre <= 32, "page mask");
  if (nsp > 0) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int blk = __builtin_amdgcn_readlane(blk_l, u);
      const bool ok = wave + kWv * u < nsp && blk >= 0 && blk < num_blocks;
      pokm |= (uint32_t)ok << u;
      load_page<KS>(view, blk, ok, pcw[u], pr8[u]);
    }
  }

  // ---- append: the workgroup also encodes position N-1 of sequence s for
  // KV head g (the key the caller has just written), as the encode kernel
  // would: its projection chains run beside the query's below
  __shared__ __align__(16) uint16_t sK[kHeadDim];
  int a_blk = -1;
  if (codes_w != nullptr && N > 0) {
    const int blk = bt[(N - 1) / kPage];
    if (blk >= 0 && blk < num_blocks) a_blk = blk;
  }
  const int a_slot = (N - 1) % kPage;
  if (a_blk >= 0 && threadIdx.x < kHeadDim / 2) {
    const uint32_t *krow = reinterpret_cast<const uint32_t *>(
        k_pool + (((int64_t)a_blk * kPage + a_slot) * Hkv + g) * kHeadDim);
    reinterpret_cast<uint32_t *>(sK)[threadIdx.x] = krow[threadIdx.x];
  }

  if ((int)threadIdx.x < G * kHeadDim / 8) reinterpret_cast<uint4 *>(sQ)[threadIdx.x] = qv4;
#pragma unroll
  for (int r = 0; r < kPLoads; ++r) {
    const int i = (int)threadIdx.x + r * kThreads;
    if (i < pn) reinterpret_cast<uint4 *>(sP)[i] = pv[r];
  }
  if (threadIdx.x < 8) sSum[threadIdx.x] = 0;
  __syncthreads();

  // p_hj in double precision, index order (one chain per (h, j) pair).
  // Batches of 8 terms: the next batch's LDS reads are issued before the
  // current batch's multiply-adds, which stay in index order.  With KEY,
  // the thread also runs the newest key's chain for the same column j and
  // the key's |k|^2 chain.
  const int npairs = G * b;
  double p[kMaxPairs];
  double mloc = 0.0;
  double pk = 0.0, r2 = 0.0;
  auto project = [&](auto key_tag, int h, int j) {
    constexpr bool KEY = decltype(key_tag)::value;
    const uint4 *qrow = reinterpret_cast<const uint4 *>(sQ + h * kHeadDim);
    const uint4 *krow = reinterpret_cast<const uint4 *>(sK);
    const uint16_t *pcol = sP + j;
    uint4 qa = qrow[0], ka = KEY ? krow[0] : make_uint4(0, 0, 0, 0);
    uint32_t pa[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) pa[u] = pcol[u * b];
    double acc = 0.0;
#pragma unroll 2
    for (int i0 = 0; i0 < kHeadDim; i0 += 8) {
      uint32_t pn[8];
      const int i1 = i0 + 8 < kHeadDim ? i0 + 8 : i0; // last batch reloads itself
      const uint4 qn = qrow[i1 / 8];
      const uint4 kn = KEY ? krow[i1 / 8] : ka;
#pragma unroll
      for (int u = 0; u < 8; ++u) pn[u] = pcol[(i1 + u) * b];
      const uint32_t qw[4] = {qa.x, qa.y, qa.z, qa.w};
      const uint32_t kw[4] = {ka.x, ka.y, ka.z, ka.w};
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t qb = (u & 1) ? (qw[u / 2] >> 16) : (qw[u / 2] & 0xFFFFu);
        const double pd = (double)bf16_to_float(pa[u]);
        acc = fma((double)bf16_to_float(qb), pd, acc);
        if (KEY) {
          const uint32_t kb = (u & 1) ? (kw[u / 2] >> 16) : (kw[u / 2] & 0xFFFFu);
          const double kd = (double)bf16_to_float(kb);
          pk = fma(kd, pd, pk);
          r2 = fma(kd, kd, r2);
        }
      }
      qa = qn;
      ka = kn;
#pragma unroll
      for (int u = 0; u < 8; ++u) pa[u] = pn[u];
    }
    return acc;
  };
  // threads 0..b-1 hold (h = 0, j = thread) at r = 0: the key's columns
  const bool key_wave = a_blk >= 0 && (int)threadIdx.x < b; // wave-uniform
#pragma unroll
  for (int r = 0; r < kMaxPairs; ++r) {
    const int idx = threadIdx.x + r * kThreads;
    p[r] = 0.0;
    if (idx < npairs) {
      const int h = idx / b, j = idx % b;
      const double acc = (r == 0 && key_wave) ? project(std::true_type{}, h, j)
                                             : project(std::false_type{}, h, j);
      p[r] = acc;
      mloc = fmax(mloc, fabs(acc));
    }
  }
  // the newest key's code bits of columns 64*wave .. 64*wave+63
  const uint64_t key_bits = __ballot(pk > 0.0);
  // the query heads' own sign codes (LSH buckets): pair idx = h*b + j
  uint64_t qsign[kMaxPairs];
#pragma unroll
  for (int r = 0; r < kMaxPairs; ++r) qsign[r] = __ballot(p[r] > 0.0);
  for (int off = 32; off > 0; off >>= 1) mloc = fmax(mloc, __shfl_xor(mloc, off));
  if (lane == 0) sMax[wave] = mloc;
  __syncthreads();
  double M = sMax[0];
  for (int i = 1; i < kThreads / 64; ++i) M = fmax(M, sMax[i]);

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
      int sum = v; // one head per wave
      for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
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
  if (sample) {
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
    uint32_t nvalid = 0;
    auto keep = [&](int t, int S) {
      if (lane < kPage && t < nsp) {
        const int pos = (pc0 + t * SP) * kPage + lane;
        const bool valid = pos >= sigma && pos < N - w;
        sSample[t * kPage + lane] = valid ? biased_score(S) : 0u;
        nvalid += valid;
      }
    };
    // the preloaded pages four at a time: after the quad step, lane L holds
    // key L%16 of page 4a + L/16
    const int lq = lane >> 4;
#pragma unroll
    for (int a = 0; a < kPre / 4; ++a) {
      uint32_t cw[4][KS], r8s[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // first use of the loaded words is here (see score_page)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          cw[j][ks] = pcw[4 * a + j][ks];
          asm volatile("" : "+v"(cw[j][ks]));
        }
        r8s[j] = pr8[4 * a + j];
        asm volatile("" : "+v"(r8s[j]));
      }
      const int mx = score_quad_max_seq<KS, G>(op, cw);
      const uint32_t r8 = lq == 0 ? r8s[0] : lq == 1 ? r8s[1] : lq == 2 ? r8s[2] : r8s[3];
      const bool ok = (pokm >> (4 * a + lq)) & 1u;
      const int t = wave + kWv * (4 * a + lq);
      if (t < nsp) {
        const int pos = (pc0 + t * SP) * kPage + (lane & 15);
        const bool valid = ok && pos >= sigma && pos < N - w;
        sSample[t * kPage + (lane & 15)] =
            valid ? biased_score(__mul24(radius_weight(r8, lin), mx)) : 0u;
        nvalid += valid;
      }
    }
    // pages past the first kPre of each wave (long sequences with a small
    // stride): 8 loads in flight per step
    for (int i0 = kPre; wave + kWv * i0 < nsp; i0 += 8) {
      uint32_t cw[8][KS], r8[8];
      bool ok[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u;
        const int blk = __builtin_amdgcn_readlane(blk_l, i & 63);
        ok[u] = wave + kWv * i < nsp && blk >= 0 && blk < num_blocks;
        load_page<KS>(view, blk, ok[u], cw[u], r8[u]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        keep(wave + kWv * (i0 + u), score_page<KS, G>(op, cw[u], r8[u], ok[u], lin));
    }
    for (int off = 32; off > 0; off >>= 1) nvalid += __shfl_xor(nvalid, off);
    if (lane == 0) sCount[wave] = nvalid;
    __syncthreads();
    uint32_t ns = 0;
    for (int i = 0; i < kWv; ++i) ns += sCount[i];
    const uint32_t ks_take = (uint32_t)min((int64_t)ns,
        ((int64_t)2 * keff * ns + nc - 1) / nc);
    if (ks_take > 0 && ks_take < ns) {
      const int nkeys = nsp * kPage;
      L = wg_kth_largest_floor<kThreads>(sel, [&](auto fn) {
        for (int i = threadIdx.x; i < nkeys; i += kThreads) {
          const uint32_t v = sSample[i];
          if (v != 0u) fn(v);
        }
      }, ks_take);
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
    if (lane < 2) cw[2 * wave + lane] = lane ? (uint32_t)(key_bits >> 32) : (uint32_t)key_bits;
    if (threadIdx.x == 0)
      radii_w[((int64_t)a_blk * Hkv + g) * kPage + a_slot] = (uint8_t)radius_code(r2);
  }
  // ---- the filter's task list: one entry (sequence, page group, length)
  // per group of kGroupKeys keys, sequence by sequence, after a count word
  // (padded to 16 bytes).  Only groups that hold keys are listed, so the
  // filter's waves share the real work evenly in ragged batches.
  if (g == 0) { // workgroup-uniform
    auto groups_of = [](int n) { return (uint32_t)((n + kGroupKeys - 1) / kGroupKeys); };
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
    if (s == (int)(gridDim.x / Hkv) - 1 && threadIdx.x == 0) tasks[0] = before + ng;
  }
}

} // namespace

hipError_t launch_prep(const DecodeDims &d, const uint16_t *q,
                       const uint16_t *proj, const uint32_t *codes,
                       const uint8_t *radii, const uint16_t *k_pool,
                       uint32_t *codes_w, uint8_t *radii_w,
                       const int32_t *block_table,
                       const int32_t *seq_lens, int8_t *q8, uint32_t *qop,
                       float *qneg, uint32_t *lthr, uint32_t *qbits,
                       uint32_t *tasks, hipStream_t stream) {
  const uint32_t code_bytes = (uint32_t)((uint64_t)d.num_blocks * d.Hkv * d.W * kPage * 4);
  const uint32_t radius_bytes = (uint32_t)((uint64_t)d.num_blocks * d.Hkv * kPage);
#define DKV_PREP_CASE(KSV, GV)                                                 \
  if (d.KS == KSV && d.G == GV) {                                              \
    hipLaunchKernelGGL((prep_kernel<KSV, GV>), dim3(d.B * d.Hkv),              \
                       dim3(kThreads), 0, stream, q, proj, codes, radii,       \
                       k_pool, codes_w, radii_w,                               \
                       d.num_blocks, code_bytes, radius_bytes, block_table,    \
                       d.max_blocks, seq_lens, d.n_max, q8, qop, qneg, lthr,   \
                       qbits, tasks,                                           \
                       d.Hq, d.Hkv, d.b, d.W, d.k, d.w, d.sigma, d.lin,         \
                       d.pages);                                               \
    return hipGetLastError();                                                  \
  }
  DKV_PREP_CASE(1, 1)
  DKV_PREP_CASE(1, 2)
  DKV_PREP_CASE(1, 4)
  DKV_PREP_CASE(1, 8)
  DKV_PREP_CASE(2, 1)
  DKV_PREP_CASE(2, 2)
  DKV_PREP_CASE(2, 4)
  DKV_PREP_CASE(2, 8)
#undef DKV_PREP_CASE
  return hipErrorInvalidValue;
}

} // namespace dkv
