// lsh.hip -- multi-table LSH candidate retrieval.
//
// [DASH-KV, "from quadratic to linear"]: several hash tables split the
// vector space into buckets so that similar vectors share one; a query
// computes its hash and looks only in its buckets, and the candidates found
// there are pruned to the top-k that enter exact attention.
//
// The key codes are already signs of Gaussian projections (SimHash), so
// table t buckets a key by its code bits t*m .. t*m+m-1, and a query head
// by the same bits of its own sign code (written by the prep kernel).
//
//   build  one workgroup per (sequence, KV head, table): a counting sort of
//          positions [0, n) by bucket -- histogram in LDS, prefix sum,
//          scatter through per-bucket cursors (the order inside a bucket
//          is free: the probe only forms a set);
//   probe  one workgroup per (sequence, KV head): the unit's G*T buckets
//          are read as one flat list of entries (their loads in parallel)
//          and marked in an LDS bitmap of positions; positions past the
//          indexed length are tested directly from their codes; the bitmap
//          goes to the workspace;
//   score  one wave per (sequence, KV head, 1024-position group): only the
//          pages holding candidates are loaded and scored (matrix-core page
//          op, as the streaming filter), and the candidates are written in
//          position order to the group's region with their count -- the
//          merge then takes the exact top-k of them.
#include "score_common.h"

namespace dkv {
namespace {

constexpr int kBuildThreads = 1024;
constexpr int kProbeThreads = 1024;
constexpr int kScoreWaves = 4;
constexpr int kMaxBuckets = 1 << 12;      // m <= 12
constexpr int kMaxProbes = 2048;          // G * T (G <= 8, T <= 256)
constexpr int kMaxWords = DKV_LSH_MAX_SEQ_LEN / 32;

// Bucket of a code (W words) in table t of m bits.
__device__ __forceinline__ uint32_t bucket_of(const uint32_t *code, int t, int m) {
  const int j = t * m, w0 = j >> 5, sh = j & 31;
  uint64_t v = code[w0];
  if (sh + m > 32) v |= (uint64_t)code[w0 + 1] << 32;
  return (uint32_t)(v >> sh) & ((1u << m) - 1u);
}

struct IndexView {
  size_t unit_bytes, off0, off_stride, pos0, pos_stride;
  __device__ const int32_t *offsets(const char *ub, int t) const {
    return reinterpret_cast<const int32_t *>(ub + off0 + (size_t)t * off_stride);
  }
  __device__ const int32_t *positions(const char *ub, int t) const {
    return reinterpret_cast<const int32_t *>(ub + pos0 + (size_t)t * pos_stride);
  }
};

__global__ __launch_bounds__(kBuildThreads) void lsh_build_kernel(
    const uint32_t *__restrict__ codes, int64_t num_blocks,
    const int32_t *__restrict__ block_table, int max_blocks,
    const int32_t *__restrict__ seq_lens, int n_max, int Hkv, int W, int T, int m,
    char *__restrict__ index, IndexView iv) {
  __shared__ uint32_t cnt[kMaxBuckets];
  __shared__ uint32_t red[kBuildThreads / 64];
  const int unit = blockIdx.x / T, t = blockIdx.x % T;
  const int s = unit / Hkv, g = unit % Hkv;
  const int tid = threadIdx.x;
  const int n = seq_len_clamped(seq_lens, s, n_max);
  const int nb = 1 << m;
  char *ub = index + (size_t)unit * iv.unit_bytes;
  int32_t *off = const_cast<int32_t *>(iv.offsets(ub, t));
  int32_t *pos = const_cast<int32_t *>(iv.positions(ub, t));
  const int32_t *bt = block_table + (int64_t)s * max_blocks;
  auto bucket_at = [&](int p) -> uint32_t {
    const int blk = bt[p / kPage];
    if (blk < 0 || blk >= num_blocks) return 0u; // unspecified key: bucket 0
    return bucket_of(codes + (((int64_t)blk * Hkv + g) * kPage + p % kPage) * W, t, m);
  };
  for (int i = tid; i < nb; i += kBuildThreads) cnt[i] = 0;
  __syncthreads();
  for (int p = tid; p < n; p += kBuildThreads) atomicAdd(&cnt[bucket_at(p)], 1u);
  __syncthreads();
  constexpr int kPer = kMaxBuckets / kBuildThreads;
  uint32_t c[kPer], part = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int b = tid * kPer + k;
    c[k] = b < nb ? cnt[b] : 0u;
    part += c[k];
  }
  uint32_t tot;
  uint32_t o = wg_exclusive_scan<kBuildThreads>(part, red, &tot); // ends with a barrier
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int b = tid * kPer + k;
    if (b < nb) {
      off[b] = (int32_t)o;
      cnt[b] = o; // scatter cursor
    }
    o += c[k];
  }
  if (tid == 0) {
    off[nb] = (int32_t)tot;
    if (t == 0) *reinterpret_cast<int32_t *>(ub) = n;
  }
  __syncthreads();
  for (int p = tid; p < n; p += kBuildThreads) {
    const uint32_t slot = atomicAdd(&cnt[bucket_at(p)], 1u);
    pos[slot] = p;
  }
}

__global__ __launch_bounds__(kProbeThreads) void lsh_probe_kernel(
    const uint32_t *__restrict__ codes, int64_t num_blocks,
    const int32_t *__restrict__ block_table, int max_blocks,
    const int32_t *__restrict__ seq_lens, int n_max, int Hkv, int G, int W, int T,
    int m, int w, int sigma, int max_seq_len, const char *__restrict__ index,
    IndexView iv, const uint32_t *__restrict__ qbits, uint32_t *__restrict__ bitmap,
    int bm_stride) {
  __shared__ uint32_t bm[kMaxWords];
  __shared__ uint32_t qb[kMaxProbes];     // bucket of probe h*T + t
  __shared__ uint32_t pstart[kMaxProbes]; // first flat entry of each probe
  __shared__ int32_t pbase[kMaxProbes];   // its first position-list index
  __shared__ uint32_t red[kProbeThreads / 64];
  const int unit = blockIdx.x;
  const int s = unit / Hkv, g = unit % Hkv;
  const int tid = threadIdx.x;
  const int Hq = Hkv * G;
  const int N = seq_len_clamped(seq_lens, s, n_max);
  const int c0 = sigma, c1 = N - w;
  const int nw = (N + 31) / 32;
  const int np = G * T;
  const char *ub = index + (size_t)unit * iv.unit_bytes;
  const int nidx = clamp_int(*reinterpret_cast<const int32_t *>(ub), 0, N);
  for (int i = tid; i < nw; i += kProbeThreads) bm[i] = 0u;
  for (int i = tid; i < np; i += kProbeThreads) {
    const int h = i / T, t = i % T;
    qb[i] = bucket_of(qbits + ((int64_t)s * Hq + (int64_t)g * G + h) * W, t, m);
  }
  __syncthreads();
  if (c1 > c0) { // workgroup-uniform
    // the probes' entry counts and their prefix (two probes per thread)
    uint32_t len[2], part = 0;
    int32_t o0[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = 2 * tid + k;
      len[k] = 0;
      o0[k] = 0;
      if (i < np) {
        const int32_t *off = iv.offsets(ub, i % T);
        const int32_t a = clamp_int(off[qb[i]], 0, max_seq_len);
        const int32_t e = clamp_int(off[qb[i] + 1], a, max_seq_len);
        o0[k] = a;
        len[k] = (uint32_t)(e - a);
      }
      part += len[k];
    }
    uint32_t total;
    uint32_t st = wg_exclusive_scan<kProbeThreads>(part, red, &total);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = 2 * tid + k;
      if (i < np) {
        pstart[i] = st;
        pbase[i] = o0[k];
      }
      st += len[k];
    }
    __syncthreads();
    // every entry of every probe, flat: the probe by binary search
    for (uint32_t e = tid; e < total; e += kProbeThreads) {
      int lo = 0, hi = np - 1; // last probe with pstart <= e
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pstart[mid] <= e) lo = mid; else hi = mid - 1;
      }
      const int32_t *pos = iv.positions(ub, lo % T);
      const int p = pos[pbase[lo] + (int)(e - pstart[lo])];
      if (p >= c0 && p < c1 && p < nidx) atomicOr(&bm[p >> 5], 1u << (p & 31));
    }
    // positions the index does not hold: tested from their codes
    const int32_t *bt = block_table + (int64_t)s * max_blocks;
    for (int p = max(c0, nidx) + tid; p < c1; p += kProbeThreads) {
      const int blk = bt[p / kPage];
      bool hit = false;
      if (blk >= 0 && blk < num_blocks) {
        const uint32_t *code = codes + (((int64_t)blk * Hkv + g) * kPage + p % kPage) * W;
        for (int t = 0; t < T && !hit; ++t) {
          const uint32_t kb = bucket_of(code, t, m);
          for (int h = 0; h < G; ++h) hit |= kb == qb[h * T + t];
        }
      }
      if (hit) atomicOr(&bm[p >> 5], 1u << (p & 31));
    }
  }
  __syncthreads();
  uint32_t *gbm = bitmap + (int64_t)unit * bm_stride;
  for (int i = tid; i < nw; i += kProbeThreads) gbm[i] = bm[i];
}

template <int KS, int G>
__global__ __launch_bounds__(kScoreWaves * 64) void lsh_score_kernel(
    const uint32_t *__restrict__ codes, const uint8_t *__restrict__ radii,
    int64_t num_blocks, uint32_t code_bytes, uint32_t radius_bytes,
    const int32_t *__restrict__ block_table, int max_blocks,
    const int32_t *__restrict__ seq_lens, int n_max, const uint32_t *__restrict__ qop,
    const float *__restrict__ qneg, int B, int Hkv, int W, bool lin,
    const uint32_t *__restrict__ bitmap, int bm_stride, uint2 *__restrict__ cand,
    uint32_t *__restrict__ tcount, int cand_groups, int ntasks) {
  // linear radius weights of the 256 codes (before any wave can leave)
  __shared__ uint16_t wlut[256];
  if (lin) { // workgroup-uniform
    fill_linear_weights(wlut, kScoreWaves * 64);
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int task = blockIdx.x * kScoreWaves + (threadIdx.x >> 6);
  if (task >= ntasks) return; // no barriers below
  const int g = task % Hkv;
  const int r = task / Hkv;
  const int s = r % B, grp = r / B;
  const int unit = s * Hkv + g;
  const int N = seq_len_clamped(seq_lens, s, n_max);
  const int key0 = grp * kGroupKeys;
  if (key0 >= N) return; // the merge reads groups below N only
  // lane j: the candidate bits of page j of the group (16 per page)
  const uint32_t *bmu = bitmap + (int64_t)unit * bm_stride;
  const uint32_t word = key0 + kPage * lane < N ? bmu[key0 / 32 + lane / 2] : 0u;
  const uint32_t pm = (lane & 1) ? (word >> 16) : (word & 0xFFFFu);
  // lane j: the block id of page j of the group, loaded with the bitmap
  const int blkv = key0 + kPage * lane < N
                       ? block_table[(int64_t)s * max_blocks + key0 / kPage + lane] : -1;
  uint64_t pages = __ballot(pm != 0u);
  const QueryOperand<KS> op = load_query_operand<KS, G>(qop, qneg, unit, s, g, Hkv * G, lane);
  const PoolView view = make_pool_view(codes, radii, code_bytes, radius_bytes, W, Hkv, g, lane);
  uint2 *reg = cand + ((int64_t)unit * cand_groups + grp) * kGroupKeys;
  uint32_t nc = 0;
  constexpr int kBatch = 8;
  while (pages) { // wave-uniform
    // up to kBatch candidate pages with their loads in flight together
    int pj[kBatch];
    uint32_t cw[kBatch][KS], r8[kBatch];
    bool ok[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      pj[k] = -1;
      if (pages) {
        pj[k] = __builtin_ctzll(pages);
        pages &= pages - 1;
      }
      const int blk = pj[k] >= 0 ? __builtin_amdgcn_readlane(blkv, pj[k]) : -1;
      ok[k] = blk >= 0 && blk < num_blocks;
      load_page<KS>(view, blk, ok[k], cw[k], r8[k]);
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (pj[k] >= 0) { // wave-uniform
        const int S = score_page<KS, G>(op, cw[k], r8[k], ok[k], lin, wlut);
        const uint32_t mask = (uint32_t)__builtin_amdgcn_readlane((int)pm, pj[k]);
        const bool isc = lane < kPage && ((mask >> lane) & 1u);
        const uint64_t bal = __ballot(isc);
        if (isc) {
          const uint32_t slot = nc + lanes_below(bal);
          reg[slot] = make_uint2(biased_score(S), (uint32_t)(key0 + kPage * pj[k] + lane));
        }
        nc += (uint32_t)__popcll(bal);
      }
    }
  }
  if (lane == 0) tcount[(int64_t)unit * cand_groups + grp] = nc;
}

IndexView view_of(const LshLayout &L) {
  IndexView v;
  v.unit_bytes = L.unit_bytes;
  v.off0 = L.off0;
  v.off_stride = L.off_stride;
  v.pos0 = L.pos0;
  v.pos_stride = L.pos_stride;
  return v;
}

} // namespace

LshLayout lsh_layout(int T, int m, int max_seq_len) {
  LshLayout L;
  auto a256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  L.off0 = 64;
  L.off_stride = ((size_t)(1u << m) + 1) * 4;
  L.pos0 = a256(L.off0 + (size_t)T * L.off_stride);
  L.pos_stride = (size_t)max_seq_len * 4;
  L.unit_bytes = a256(L.pos0 + (size_t)T * L.pos_stride);
  return L;
}

hipError_t launch_lsh_build(const DecodeDims &d, const uint32_t *codes,
                            const int32_t *block_table, const int32_t *seq_lens,
                            char *index, hipStream_t stream) {
  const IndexView iv = view_of(lsh_layout(d.lsh_T, d.lsh_m, d.max_seq_len));
  hipLaunchKernelGGL(lsh_build_kernel, dim3((unsigned)(d.B * d.Hkv * d.lsh_T)),
                     dim3(kBuildThreads), 0, stream, codes, d.num_blocks, block_table,
                     d.max_blocks, seq_lens, d.n_max, d.Hkv, d.W, d.lsh_T, d.lsh_m,
                     index, iv);
  return hipGetLastError();
}

hipError_t launch_lsh_probe(const DecodeDims &d, const uint32_t *codes,
                            const int32_t *block_table, const int32_t *seq_lens,
                            const char *index, const uint32_t *qbits,
                            uint32_t *bitmap, hipStream_t stream) {
  const IndexView iv = view_of(lsh_layout(d.lsh_T, d.lsh_m, d.max_seq_len));
  hipLaunchKernelGGL(lsh_probe_kernel, dim3((unsigned)(d.B * d.Hkv)),
                     dim3(kProbeThreads), 0, stream, codes, d.num_blocks, block_table,
                     d.max_blocks, seq_lens, d.n_max, d.Hkv, d.G, d.W, d.lsh_T,
                     d.lsh_m, d.w, d.sigma, d.max_seq_len, index, iv, qbits, bitmap,
                     d.bm_words);
  return hipGetLastError();
}

hipError_t launch_lsh_score(const DecodeDims &d, const uint32_t *codes,
                            const uint8_t *radii, const int32_t *block_table,
                            const int32_t *seq_lens, const uint32_t *qop,
                            const float *qneg, const uint32_t *bitmap, uint2 *cand,
                            uint32_t *tcount, hipStream_t stream) {
  const int pages = (d.n_max + kPage - 1) / kPage;
  const int64_t ngroups = (pages + kGroupPages - 1) / kGroupPages;
  if (ngroups == 0) return hipSuccess;
  const int64_t ntasks = (int64_t)d.B * ngroups * d.Hkv;
  if (ntasks > 0x7FFFFFFF - 65536) return hipErrorInvalidValue;
  const uint32_t code_bytes = (uint32_t)((uint64_t)d.num_blocks * d.Hkv * d.W * kPage * 4);
  const uint32_t radius_bytes = (uint32_t)((uint64_t)d.num_blocks * d.Hkv * kPage);
  const unsigned nwg = (unsigned)((ntasks + kScoreWaves - 1) / kScoreWaves);
#define DKV_LSH_CASE(KSV, GV)                                                  \
  if (d.KS == KSV && d.G == GV) {                                              \
    hipLaunchKernelGGL((lsh_score_kernel<KSV, GV>), dim3(nwg),                 \
                       dim3(kScoreWaves * 64), 0, stream, codes, radii,        \
                       d.num_blocks, code_bytes, radius_bytes, block_table,    \
                       d.max_blocks, seq_lens, d.n_max, qop, qneg, d.B, d.Hkv, \
                       d.W, d.lin, bitmap, d.bm_words, cand, tcount,           \
                       d.cand_groups, (int)ntasks);                            \
    return hipGetLastError();                                                  \
  }
  DKV_LSH_CASE(1, 1)
  DKV_LSH_CASE(1, 2)
  DKV_LSH_CASE(1, 4)
  DKV_LSH_CASE(1, 8)
  DKV_LSH_CASE(2, 1)
  DKV_LSH_CASE(2, 2)
  DKV_LSH_CASE(2, 4)
  DKV_LSH_CASE(2, 8)
#undef DKV_LSH_CASE
  return hipErrorInvalidValue;
}

} // namespace dkv
