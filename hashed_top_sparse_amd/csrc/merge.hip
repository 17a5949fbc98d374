// merge.hip -- final selection of one decode step per (sequence, KV head).
//
// [DASH-KV Top-K pruning; DeepSeek DSA]: exact attention runs over the
// top-k keys only; [DeepSeek CSA]: plus the sliding window of the most
// recent tokens; [DySCO FAQ 3]: plus the first tokens (attention sinks).
//   sinks   [0, min(sigma, N))
//   window  [max(min(sigma, N), N - w), N)
//   top-k   the k_eff = min(k, |C|) best of C = [sigma, N - w) by
//           (S desc, position asc)
//
// The streaming pass left every candidate with u >= L (the sampled
// threshold) in the region of its group of kGroupKeys positions, with the
// group's count.  If at least k_eff of them exist, the top-k of C is exactly
// the top-k of the candidates:
//   - the k_eff-th largest biased score T and the number of ties at T to
//     keep come from two histogram passes (select_common.h);
//   - if only some ties are kept, the lowest positions win: a second
//     k-th-largest search over the inverted positions of the ties;
//   - the staged candidates are in ascending position order (groups in
//     order, and the streaming pass writes a group's candidates in
//     position order), so the survivors are compacted with a prefix sum
//     over that order: the list is sinks, window, then the top-k in
//     ascending position (deterministic).  Candidate lists too long to
//     stage, and the fallback below, mark survivors in a position bitmap
//     and read it back in order instead.
// Otherwise the workgroup rescans the (sequence, KV head)'s codes itself
// and runs the same exact selection over every candidate score (slow, but
// exact for any input).
//
// Output per unit: physical row ids (page*16 + slot) for the attention
// gather and, when asked, logical positions; -1 past the count.
#include "score_common.h"
#include "select_common.h"

namespace dkv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kStage = 12288;        // candidates staged in LDS as (u, pos)
constexpr int kRowAhead = 8;         // staged entries per thread whose rows are looked up early
constexpr int kStageRound = 8;       // groups per wave whose loads are in flight together
constexpr int kMaxGroupsLds = 4096;  // groups whose count prefix fits in LDS
constexpr uint32_t kPosMax = 0x00FFFFFFu; // positions < 2^24

__device__ __forceinline__ int row_of(const int32_t *bt, int pos,
                                      int64_t num_blocks) {
  const int blk = bt[pos / kPage];
  return (blk >= 0 && blk < num_blocks) ? blk * kPage + pos % kPage : -1;
}

// SEL: 0 keys; 1 pages (the candidates are pages: page-granular
// selection); 2 LSH (the candidates are exactly the LSH candidates, all
// kept when they are k or fewer).
template <int KS, int G, int SEL>
__global__ __launch_bounds__(kThreads) void merge_kernel(
    const uint2 *__restrict__ cand, const uint32_t *__restrict__ tcount,
    int cand_groups,
    const int32_t *__restrict__ seq_lens, int n_max,
    const int32_t *__restrict__ block_table, int max_blocks,
    int64_t num_blocks, int Hkv, int k, int w, int sigma, int cap,
    uint32_t *__restrict__ bitmap, int bm_stride, int32_t *__restrict__ rows,
    int32_t *__restrict__ cnt, int32_t *__restrict__ user_sel,
    int32_t *__restrict__ user_cnt, const uint32_t *__restrict__ codes,
    const uint8_t *__restrict__ radii, uint32_t code_bytes,
    uint32_t radius_bytes, int W, const uint32_t *__restrict__ qop,
    const float *__restrict__ qneg, bool lin) {
  constexpr bool pages = SEL == 1;
  constexpr bool lsh = SEL == 2;
  __shared__ __align__(16) uint2 st[kStage];
  __shared__ uint32_t gpre[kMaxGroupsLds + 1];
  __shared__ SelectShared<kThreads> sel;
  __shared__ uint16_t wlut[256]; // linear radius weights (the exact rescan)

  const int unit = blockIdx.x;
  const int s = unit / Hkv, g = unit % Hkv;
  const int tid = threadIdx.x;
  if (lin) fill_linear_weights(wlut, kThreads); // (many barriers before the rescan)
  const int lane = tid & 63, wave = tid >> 6;
  const int N = seq_len_clamped(seq_lens, s, n_max);
  const int ns = sigma < N ? sigma : N;
  const int ws = (N - w > ns) ? N - w : ns;
  const int nwin = N - ws;
  const int nc = max(0, N - w - sigma);
  const int c0 = sigma, c1 = N - w; // candidate positions [c0, c1)
  // pages: the items ranked are the pages meeting [c0, c1); the number of
  // rows they bring is known only after the selection (edge pages are
  // partial) unless none or all of them are taken
  const int npc = nc > 0 ? (c1 + kPage - 1) / kPage - c0 / kPage : 0;
  const int nitems = pages ? npc : nc;
  // (LSH: an upper bound until the candidates are counted)
  int keff = pages ? min(k / kPage, npc) : min(k, nc);
  const bool rows_known = (!pages && !lsh) || keff == 0 || (pages && keff == npc);
  const int base = ns + nwin;
  int total = base + (keff == nitems && !lsh ? nc : (pages || lsh ? 0 : keff));
  const int32_t *bt = block_table + (int64_t)s * max_blocks;
  int32_t *R = rows + (int64_t)unit * cap;
  int32_t *U = user_sel ? user_sel + (int64_t)unit * cap : nullptr;

  // Loads are issued by every thread at clamped in-bounds addresses and
  // their values dropped where they are used: a load in a lane-dependent
  // branch, or a select on its value, makes the compiler wait for it (and
  // for every load issued before it) right there.
  //
  // The block id of this thread's first sink or window row is requested
  // first; the row is written once the group counts are requested too.
  const int sw_pos = tid < ns ? tid : ws + (tid - ns); // row tid of the list
  const int sw_blk = bt[clamp_int(sw_pos, 0, max(N - 1, 0)) / kPage];
  auto write_sinks_window = [&]() {
    if (tid < base) {
      R[tid] = (sw_blk >= 0 && sw_blk < num_blocks) ? sw_blk * kPage + sw_pos % kPage : -1;
      if (U) U[tid] = sw_pos;
    }
    for (int i = tid + kThreads; i < base; i += kThreads) { // (a window past kThreads)
      const int pos = i < ns ? i : ws + (i - ns);
      R[i] = row_of(bt, pos, num_blocks);
      if (U) U[i] = pos;
    }
    if (rows_known) {
      for (int i = total + tid; i < cap; i += kThreads) {
        R[i] = -1;
        if (U) U[i] = -1;
      }
    }
  };
  bool sw_done = false;

  if (keff > 0) {
    uint32_t *bm = bitmap + (int64_t)unit * bm_stride;
    const int nwords = (N + 31) / 32;
    bool use_bitmap = true;
    // marks the candidate positions of page p
    auto mark_page = [&](int p) {
      const int lo = max(c0, p * kPage), hi = min(c1, (p + 1) * kPage);
      if (hi > lo) // a page's bits never span two words
        atomicOr(&bm[lo >> 5], ((1u << (hi - lo)) - 1u) << (lo & 31));
    };
    if (!lsh && keff == nitems) {
      write_sinks_window();
      sw_done = true;
      // every candidate is selected, in position order
      for (int i = tid; i < nc; i += kThreads) {
        const int pos = c0 + i;
        R[base + i] = row_of(bt, pos, num_blocks);
        if (U) U[base + i] = pos;
      }
      use_bitmap = false;
    } else {
      // the candidates of the unit's groups (those below N were written):
      // count prefix over the groups, in LDS when it fits.  A count is at
      // most the group's size; it is clamped to it anyway, so a corrupt
      // count cannot send a read past the group's region.
      const int ngs = (N + kGroupKeys - 1) / kGroupKeys;
      const uint32_t *tc = tcount + (int64_t)unit * cand_groups;
      const uint2 *cb = cand + (int64_t)unit * cand_groups * kGroupKeys;
      const bool pre_lds = ngs <= kMaxGroupsLds;
      uint32_t nlist;
      // The first staging round's entries (the first 64 of groups wave,
      // wave + 16, ...) are requested right after the counts: their
      // addresses do not depend on the counts, so both arrive in one round
      // trip (entries past a group's count are dropped when staged).
      uint2 e0[kStageRound];
      {
        constexpr int kPer = kMaxGroupsLds / kThreads;
        uint32_t c[kPer], part = 0;
        if (pre_lds) { // workgroup-uniform; ngs >= 1 here (N > w + sigma)
          uint32_t raw[kPer];
#pragma unroll
          for (int i = 0; i < kPer; ++i) raw[i] = tc[min(tid * kPer + i, ngs - 1)];
#pragma unroll
          for (int r = 0; r < kStageRound; ++r)
            e0[r] = cb[(int64_t)min(wave + r * kWaves, ngs - 1) * kGroupKeys + lane];
          write_sinks_window();
          sw_done = true;
#pragma unroll
          for (int i = 0; i < kPer; ++i) {
            const int gi = tid * kPer + i;
            c[i] = gi < ngs ? min(raw[i], (uint32_t)kGroupKeys) : 0u;
            part += c[i];
          }
        } else {
          write_sinks_window();
          sw_done = true;
          for (int gi = tid; gi < ngs; gi += kThreads)
            part += min(tc[gi], (uint32_t)kGroupKeys);
        }
        uint32_t off = wg_exclusive_scan<kThreads>(part, &sel.red[2][0], &nlist);
        if (pre_lds) {
#pragma unroll
          for (int i = 0; i < kPer; ++i) {
            const int gi = tid * kPer + i;
            if (gi < ngs) gpre[gi] = off;
            off += c[i];
          }
          if (tid == 0) gpre[ngs] = nlist;
        }
      }
      // fn(u, pos) for every candidate, each once across the workgroup,
      // straight from the group regions (for units too large to stage)
      auto for_each_global = [&](auto fn) {
        for (int gi = wave; gi < ngs; gi += kWaves) {
          const uint32_t n = min(tc[gi], (uint32_t)kGroupKeys);
          const uint2 *reg = cb + (int64_t)gi * kGroupKeys;
          for (uint32_t j = lane; j < n; j += 64) {
            const uint2 e = reg[j];
            fn(e.x, (int)e.y);
          }
        }
      };
      uint32_t T, take_eq, n_eq;
      if (lsh) {
        // the selection is the top min(k, candidates) of the candidates
        keff = min(keff, (int)nlist);
        total = base + keff;
        for (int i = total + tid; i < cap; i += kThreads) {
          R[i] = -1;
          if (U) U[i] = -1;
        }
      }
      if (keff == 0) { // LSH without candidates (workgroup-uniform)
        use_bitmap = false;
      } else if (nlist >= (uint32_t)keff) {
        // ---- normal path: exact top-k of the candidates
        const bool staged = pre_lds && nlist <= (uint32_t)kStage;
        if (!staged) {
          for (int i = tid; i < nwords; i += kThreads) bm[i] = 0u;
        }
        __syncthreads();
        if (staged) {
          // group g's candidates go to st[gpre[g] ..): wave v copies groups
          // v, v+16, ..., kStageRound groups' first 64 entries in flight at
          // once (every lane loads; entries past a group's count, and
          // groups past the unit's, are not stored).  The range of u the
          // cut's histogram needs is taken on the way, and the histogram
          // cleared, before the staging barrier.
          uint32_t lo = 0xFFFFFFFFu, hi = 0u;
          auto stage_round = [&](int g0, const uint2 (&e)[kStageRound])
                                 __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < kStageRound; ++r) {
              const int gi = g0 + r * kWaves;
              if (gi < ngs) { // wave-uniform
                const uint32_t b = gpre[gi], n = gpre[gi + 1] - b;
                if ((uint32_t)lane < n) {
                  st[b + (uint32_t)lane] = e[r];
                  lo = min(lo, e[r].x);
                  hi = max(hi, e[r].x);
                }
              }
            }
            // entries past the first 64 of a group (rare)
#pragma unroll
            for (int r = 0; r < kStageRound; ++r) {
              const int gi = g0 + r * kWaves;
              if (gi < ngs) {
                const uint32_t b = gpre[gi], n = gpre[gi + 1] - b;
                for (uint32_t j = 64u + (uint32_t)lane; j < n; j += 64u) {
                  const uint2 x = cb[(int64_t)gi * kGroupKeys + j];
                  st[b + j] = x;
                  lo = min(lo, x.x);
                  hi = max(hi, x.x);
                }
              }
            }
          };
          if (wave < ngs) stage_round(wave, e0); // (its loads were issued with the counts)
          for (int g0 = wave + kStageRound * kWaves; g0 < ngs; g0 += kStageRound * kWaves) {
            uint2 e[kStageRound];
#pragma unroll
            for (int r = 0; r < kStageRound; ++r)
              e[r] = cb[(int64_t)min(g0 + r * kWaves, ngs - 1) * kGroupKeys + lane];
            stage_round(g0, e);
          }
          wave_min_max(lo, hi);
          if (lane == 0) {
            sel.red[0][wave] = lo;
            sel.red[1][wave] = hi;
          }
          for (int i = tid; i < kHistBins; i += kThreads) sel.hist[i] = 0u;
          __syncthreads();
        }
        auto for_each = [&](auto fn) {
          if (staged) {
            for (uint32_t i = tid; i < nlist; i += kThreads) fn(st[i].x, (int)st[i].y);
          } else {
            for_each_global(fn);
          }
        };
        // the compaction below gives thread t the run [i0, i1) of the staged
        // list; the block ids of its first kRowAhead entries are requested
        // now (positions clamped into the sequence), so the block-table
        // loads overlap the cut
        const uint32_t per = (nlist + kThreads - 1) / kThreads;
        const uint32_t i0 = min(nlist, tid * per), i1 = min(nlist, i0 + per);
        int rblk[kRowAhead];
#pragma unroll
        for (int k = 0; k < kRowAhead; ++k) {
          const uint32_t i = min(i0 + (uint32_t)k, (uint32_t)kStage - 1u);
          const int pos = (staged && !pages) ? clamp_int((int)st[i].y, 0, N - 1) : 0;
          rblk[k] = bt[pos / kPage];
        }
        // the row of staged entry i0 + k at position pos
        auto row_ahead = [&](int k, int pos) {
          return (rblk[k] >= 0 && rblk[k] < num_blocks) ? rblk[k] * kPage + pos % kPage : -1;
        };
        // the cut: survivors are u > Tu, or u == Tu and pos <= Tpos
        uint32_t Tu = 0, Tpos = 0;
        bool cut = false;
        if (lsh && (uint32_t)keff == nlist) { // every candidate is kept
          cut = true;
          Tpos = 0xFFFFFFFFu;
        } else if (staged) {
          cut = wg_topk_cut_ranged<kThreads>(sel, for_each, (uint32_t)keff, Tu, Tpos);
        }
        uint32_t Pt = 0; // otherwise: ties with (kPosMax - pos) >= Pt are kept
        if (!cut) {
          wg_kth_largest<kThreads>(sel, [&](auto fn) {
            for_each([&](uint32_t u, int) { fn(u); });
          }, (uint32_t)keff, T, take_eq, n_eq);
          if (take_eq < n_eq) {
            uint32_t t2, n2;
            wg_kth_largest<kThreads>(sel, [&](auto fn) {
              for_each([&](uint32_t u, int pos) {
                if (u == T) fn(kPosMax - (uint32_t)pos);
              });
            }, take_eq, Pt, t2, n2);
          }
        }
        auto keep = [&](uint32_t u, int pos) {
          return cut ? (u > Tu || (u == Tu && (uint32_t)pos <= Tpos))
                     : (u > T || (u == T && kPosMax - (uint32_t)pos >= Pt));
        };
        if (pages && staged) {
          // stable compaction of the selected pages' candidate keys: thread
          // t takes the run [i0, i1) of the staged (page-ordered) list and
          // writes all rows of its kept pages after a prefix sum of their
          // row counts
          auto rows_of_page = [&](int p) {
            return max(0, min(c1, (p + 1) * kPage) - max(c0, p * kPage));
          };
          // The block ids of all kept pages are requested together; after
          // two prefix sums (rows, pages) every kept page goes to an LDS list
          // (block id, page, first row) that reuses the staging buffer, and
          // 16 lanes write each page's rows side by side.
          constexpr int kPer = kStage / kThreads; // >= i1 - i0
          uint32_t c = 0, kept = 0;
          int blk[kPer], pg[kPer];
#pragma unroll
          for (int j = 0; j < kPer; ++j) {
            const uint32_t i = i0 + j;
            blk[j] = -1;
            pg[j] = 0;
            if (i < i1 && keep(st[i].x, (int)st[i].y)) {
              pg[j] = (int)st[i].y;
              c += (uint32_t)rows_of_page(pg[j]);
              kept |= 1u << j;
              blk[j] = bt[pg[j]];
            }
          }
          uint32_t tot, npk;
          uint32_t o = wg_exclusive_scan<kThreads>(c, &sel.red[3][0], &tot);
          uint32_t e = wg_exclusive_scan<kThreads>((uint32_t)__popc(kept), &sel.red[3][0], &npk);
          // (the scans' barriers: no thread reads the staged list any more)
          const uint32_t room = (uint32_t)(cap - base);
          uint4 *lst = reinterpret_cast<uint4 *>(st);
          const bool listed = npk <= (uint32_t)(kStage / 2); // workgroup-uniform
#pragma unroll
          for (int j = 0; j < kPer; ++j) {
            if ((kept >> j) & 1u) {
              const int p = pg[j];
              if (listed) {
                lst[e++] = make_uint4((uint32_t)blk[j], (uint32_t)p, o, 0u);
                o += (uint32_t)rows_of_page(p);
              } else {
                const bool okb = blk[j] >= 0 && blk[j] < num_blocks;
                for (int pos = max(c0, p * kPage); pos < min(c1, (p + 1) * kPage) && o < room;
                     ++pos) {
                  R[base + o] = okb ? blk[j] * kPage + pos % kPage : -1;
                  if (U) U[base + o] = pos;
                  ++o;
                }
              }
            }
          }
          if (listed) {
            __syncthreads();
            const int l = tid & (kPage - 1);
            for (uint32_t x = (uint32_t)(tid / kPage); x < npk; x += kThreads / kPage) {
              const uint4 ent = lst[x];
              const int b = (int)ent.x, p = (int)ent.y;
              const int pos = max(c0, p * kPage) + l;
              const uint32_t r = ent.z + (uint32_t)l;
              if (pos < min(c1, (p + 1) * kPage) && r < room) {
                R[base + r] = (b >= 0 && b < num_blocks) ? b * kPage + pos % kPage : -1;
                if (U) U[base + r] = pos;
              }
            }
          }
          total = base + (int)min(tot, room);
          for (int i = total + tid; i < cap; i += kThreads) {
            R[i] = -1;
            if (U) U[i] = -1;
          }
          use_bitmap = false;
        } else if (pages) {
          // the selected pages' candidate keys go to the bitmap
          for_each([&](uint32_t u, int p) {
            if (keep(u, p)) mark_page(p);
          });
        } else if (staged) {
          // stable compaction of the survivors: thread t takes the run
          // [i0, i1) of the staged list
          uint32_t c = 0;
          for (uint32_t i = i0; i < i1; ++i) c += keep(st[i].x, (int)st[i].y);
          uint32_t tot;
          uint32_t o = wg_exclusive_scan<kThreads>(c, &sel.red[3][0], &tot);
#pragma unroll
          for (int k = 0; k < kRowAhead; ++k) {
            const uint32_t i = i0 + k;
            if (i < i1) {
              const int pos = (int)st[i].y;
              if (keep(st[i].x, pos)) {
                R[base + o] = row_ahead(k, pos);
                if (U) U[base + o] = pos;
                ++o;
              }
            }
          }
          for (uint32_t i = i0 + kRowAhead; i < i1; ++i) {
            const int pos = (int)st[i].y;
            if (keep(st[i].x, pos)) {
              R[base + o] = row_of(bt, pos, num_blocks);
              if (U) U[base + o] = pos;
              ++o;
            }
          }
          use_bitmap = false;
        } else {
          for_each([&](uint32_t u, int pos) {
            if (keep(u, pos)) atomicOr(&bm[pos >> 5], 1u << (pos & 31));
          });
        }
      } else {
        for (int i = tid; i < nwords; i += kThreads) bm[i] = 0u;
        __syncthreads();
        // ---- exact fallback: rescore every candidate key of the unit
        // (pages: every page, scored by its best candidate key)
        const QueryOperand<KS> op = load_query_operand<KS, G>(
            qop, qneg, unit, s, g, Hkv * G, lane);
        const PoolView view = make_pool_view(codes, radii, code_bytes,
                                             radius_bytes, W, Hkv, g, lane);
        const int pc0 = c0 / kPage, pc1 = (c1 + kPage - 1) / kPage;
        // fn(u, pos) for every candidate, lanes 0..15 of each wave (pages:
        // fn(u, page) in lane 0)
        auto rescan = [&](auto fn) {
          for (int p0 = pc0 + wave * 8; p0 < pc1; p0 += kWaves * 8) {
            uint32_t cw[8][KS], r8[8];
            bool ok[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const int pg = p0 + u;
              const int blk = pg < pc1 ? bt[pg] : -1;
              ok[u] = blk >= 0 && blk < num_blocks;
              load_page<KS>(view, blk, ok[u], cw[u], r8[u]);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const int S = score_page<KS, G>(op, cw[u], r8[u], ok[u], lin, wlut);
              const int pos = (p0 + u) * kPage + lane;
              const bool in_c = lane < kPage && pos >= c0 && pos < c1;
              if (pages) { // workgroup-uniform; the row max needs every lane
                const uint32_t up = row_max16(in_c ? biased_score(S) : 0u);
                if (lane == 0 && up != 0u) fn(up, p0 + u);
              } else if (in_c) {
                fn(biased_score(S), pos);
              }
            }
          }
        };
        wg_kth_largest<kThreads>(sel, [&](auto fn) {
          rescan([&](uint32_t u, int) { fn(u); });
        }, (uint32_t)keff, T, take_eq, n_eq);
        uint32_t Pt = 0;
        if (take_eq < n_eq) {
          uint32_t t2, n2;
          wg_kth_largest<kThreads>(sel, [&](auto fn) {
            rescan([&](uint32_t u, int pos) {
              if (u == T) fn(kPosMax - (uint32_t)pos);
            });
          }, take_eq, Pt, t2, n2);
        }
        rescan([&](uint32_t u, int pos) {
          if (u > T || (u == T && kPosMax - (uint32_t)pos >= Pt)) {
            if (pages)
              mark_page(pos);
            else
              atomicOr(&bm[pos >> 5], 1u << (pos & 31));
          }
        });
      }
    }
    if (use_bitmap) { // workgroup-uniform
      __syncthreads();
      const uint32_t nsel = emit_bitmap<kThreads>(bm, nwords, bt, num_blocks, R + base,
                                                  U ? U + base : nullptr, &sel.red[3][0],
                                                  (uint32_t)(cap - base));
      if (!rows_known) {
        total = base + (int)nsel;
        for (int i = total + tid; i < cap; i += kThreads) {
          R[i] = -1;
          if (U) U[i] = -1;
        }
      }
    }
  }
  if (!sw_done) write_sinks_window(); // keff == 0 (workgroup-uniform)
  if (tid == 0) {
    cnt[unit] = total;
    if (user_cnt) user_cnt[unit] = total;
  }
}

} // namespace

hipError_t launch_merge(const DecodeDims &d, const uint2 *cand,
                        const uint32_t *tcount,
                        const int32_t *seq_lens, const int32_t *block_table,
                        uint32_t *bitmap, int32_t *rows, int32_t *cnt,
                        int32_t *user_sel, int32_t *user_cnt,
                        const uint32_t *codes, const uint8_t *radii,
                        const uint32_t *qop, const float *qneg,
                        hipStream_t stream) {
  const uint32_t code_bytes = (uint32_t)((uint64_t)d.num_blocks * d.Hkv * d.W * kPage * 4);
  const uint32_t radius_bytes = (uint32_t)((uint64_t)d.num_blocks * d.Hkv * kPage);
#define DKV_MERGE_LAUNCH(KSV, GV, PV)                                          \
  {                                                                            \
    hipLaunchKernelGGL((merge_kernel<KSV, GV, PV>), dim3(d.B * d.Hkv),         \
                       dim3(kThreads), 0, stream, cand, tcount,                \
                       d.cand_groups, seq_lens, d.n_max, block_table,          \
                       d.max_blocks, d.num_blocks, d.Hkv, d.k, d.w, d.sigma,   \
                       d.cap, bitmap, d.bm_words, rows, cnt, user_sel,         \
                       user_cnt, codes, radii, code_bytes, radius_bytes, d.W,  \
                       qop, qneg, d.lin);                                      \
    return hipGetLastError();                                                  \
  }
#define DKV_MERGE_CASE(KSV, GV)                                                \
  if (d.KS == KSV && d.G == GV) {                                              \
    if (d.lsh_T > 0) DKV_MERGE_LAUNCH(KSV, GV, 2)                              \
    if (d.pages) DKV_MERGE_LAUNCH(KSV, GV, 1)                                  \
    DKV_MERGE_LAUNCH(KSV, GV, 0)                                               \
  }
  DKV_MERGE_CASE(1, 1)
  DKV_MERGE_CASE(1, 2)
  DKV_MERGE_CASE(1, 4)
  DKV_MERGE_CASE(1, 8)
  DKV_MERGE_CASE(2, 1)
  DKV_MERGE_CASE(2, 2)
  DKV_MERGE_CASE(2, 4)
  DKV_MERGE_CASE(2, 8)
#undef DKV_MERGE_CASE
#undef DKV_MERGE_LAUNCH
  return hipErrorInvalidValue;
}

} // namespace dkv
