// encode.hip -- key codes and radii at KV write time.
//
// [SPHERICAL KV, §2.1 / §2.3]: each key is stored as a quantised radius and
// a packed angle code, computed when the key is written to the paged cache.
// [DASH-KV, asymmetric hashing]: the key side takes the light encoder and
// its code is reused by every later query.
//
// Code bit j = [p_j > 0] with p_j = sum_i k_i * P_ij accumulated in double
// precision in index order (bf16 x bf16 products are exact in double, so a
// fused multiply-add equals a multiply then an add).  Radius code r8 =
// largest m in 1..255 with |k|^2 >= 2^((m-64)/8), else 0.  The kernel below
// reaches exactly these values through fp32 matrix ops whose signs are
// certified, with the fp64 chains only where they are not.

#include <algorithm>
#include <type_traits>
#include <utility>

#include "encode_common.h"

namespace dkv {
namespace {

// ---------------------------------------------------------------------------
// Matrix-core encode.  p = k.P runs as bf16 x bf16 matrix ops (32 keys x 32
// columns x 16 dims each; the products are exact in fp32, the sums are fp32).
// A sign is certain when |p32| exceeds a bound on the fp32 summation error
// in any order (Cauchy-Schwarz: sum |k_i P_ij| <= |k| |P_j|):
//   |p32 - p| <= (d+2) 2^-23 |k| max_j |P_j| + 2^-100.
// A sum of d exact products with at most d roundings, each off by less than
// 2^-23 of its result (an accumulator that truncates; round-to-nearest
// halves that), errs by at most d 2^-23 (1 + 2^-15) sum |k_i P_ij|; the
// factor (d+2)/d covers the fp32 norms (sums of d squares, each within
// 2^-16 of the exact one) and the bound's own roundings.  The 2^-100 term
// covers products that underflow; the largest column norm of the
// workgroup's columns stands in for |P_j|, which only widens the bound.  Uncertain bits are recomputed with the index-order fp64
// chain of the definition.  Likewise |k|^2: an fp32 sum gives the radius
// code unless it lies near a code threshold (radius_code_certain); then the
// fp64 chain decides.
//
// Work.  A unit is 16 consecutive key rows of a page (the page's rows are
// stored position-major, [16][Hkv][d], so a unit is 4 KB of contiguous
// memory: slice q holds rows 16q..16q+15, row m being position m / Hkv of
// KV head m % Hkv).  A workgroup of four waves walks a run of units, 2X per
// step (X = 1 for b >= 128, 2 for b = 64), as 32X rows:
//  - each wave loads 8X of the rows (whole 256-byte rows, four per load
//    instruction), three steps ahead, then writes them to the step's LDS
//    tile, with their |k|^2 (fp32), row bound and radius code;
//  - after one barrier, each wave takes the 32 rows of its row group in
//    the matrix layout (lane L: row L%32, dims 64h..64h+63, h = L/32;
//    matrix K-step c takes dims 64h+8c..64h+8c+7 of each half, so every dim
//    is used once, and column L%32 of P is arranged the same way) and scores
//    them against its 32 or 64 columns of P, whose fragments stay in its
//    registers.
// In the 32x32 result, lane L holds column L%32 of rows 8(j/4) + 4h + j%4:
// a ballot of one result register is the 32-bit code word of two rows,
// moved into the lane that stores it.  The units' block ids, slices and row
// masks are prepared a window of 256 units at a time into LDS (block ids
// loaded a window ahead), so the step loop walks nothing itself.
typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));
typedef float v16f32 __attribute__((ext_vector_type(16)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
typedef float v4f32 __attribute__((ext_vector_type(4)));

constexpr int kEncThreads = 256; // four waves
constexpr int kEncWaves = kEncThreads / 64;
constexpr int kRangeLds = 512;   // sequences whose encode range sits in LDS
constexpr int kQueue = 64;       // uncertain signs queued per wave
constexpr int kTileRow = 272;    // LDS bytes per tile row (256 + 16: the
                                 // matrix-layout reads are conflict-free)
constexpr int kWin = 256;        // units per window of unit info
constexpr int kAhead = 3;        // steps of rows in flight

__device__ __forceinline__ uint32_t lanes_below_u64(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ v8bf16 as_v8bf16(const uint4 &u) {
  return __builtin_bit_cast(v8bf16, u);
}

// The compiler's lane write (v_writelane_b32), which clang exposes under no
// builtin name; as an intrinsic call the hazard pass sees it and spaces it
// from the compare that wrote its scalar source.
extern "C" __device__ int dkv_amdgcn_writelane(int val, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

// Places a wave-uniform value in one lane of a register (lane fixed at
// compile time).
template <int LANE>
__device__ __forceinline__ uint32_t write_lane(uint32_t old, uint32_t val) {
  return (uint32_t)dkv_amdgcn_writelane((int)val, LANE, (int)old);
}

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(std::integral_constant<int, i>) for i = 0..N-1
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Sum over each row of 16 lanes, in every lane of the row (DPP: quad
// swaps, then the mirrors of half rows and rows).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);  // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);  // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v); // row_half_mirror
  v += dpp_f32<0x140>(v); // row_mirror
  return v;
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Index-order fp64 sums over one key row in global memory: its projection
// on column col of P ([d][b] row-major, global), or its squared norm
// (proj null).
__device__ double row_chain_fp64(const uint16_t *krow_g, const uint16_t *proj, int b, int col) {
  const uint4 *krow = reinterpret_cast<const uint4 *>(krow_g);
  double acc = 0.0;
#pragma unroll 2
  for (int c = 0; c < kHeadDim / 8; ++c) {
    const uint4 k8 = krow[c];
    const uint32_t kw[4] = {k8.x, k8.y, k8.z, k8.w};
    uint32_t pw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) pw[u] = proj ? proj[(int64_t)(8 * c + u) * b + col] : 0u;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const double x = (double)bf16_to_float((u & 1) ? (kw[u / 2] >> 16) : (kw[u / 2] & 0xFFFFu));
      acc = fma(x, proj ? (double)bf16_to_float(pw[u]) : x, acc);
    }
  }
  return acc;
}

// The radius code of an fp32 |k|^2 when it is certain, else -1.  With
// L = 8 log2 |k|^2 the code is floor(L) + 64 clamped to [0, 255]; it is
// certain when L lies farther than 2^-11 from an integer (the fp32 sum is
// within 2^-17 of |k|^2 relatively, 8.8e-5 in L, and the hardware log2
// within a few ulps), when L < -64 (code 0), and when |k|^2 is 0 or at least
// 2^24 (code 255).
__device__ __forceinline__ int radius_code_certain(float r2) {
  if (!(r2 > 0.f)) return r2 == 0.f ? 0 : -1;
  if (r2 >= 0x1p24f) return 255;
  const float L = 8.f * __builtin_amdgcn_logf(r2);
  if (L < -64.f) return 0;
  const float fl = floorf(L);
  const float fr = L - fl;
  if (!(fr > 0x1p-11f && fr < 1.f - 0x1p-11f)) return -1;
  return clamp_int((int)fl + 64, 0, 255);
}

template <int NCB>
struct EncShape {
  static constexpr int b = 32 * NCB, W = NCB;
  static constexpr int X = NCB >= 4 ? 1 : 2;         // row groups of 32 per step
  static constexpr int BPW = NCB >= 8 ? 2 : 1;       // column blocks per wave
  static constexpr int CW = NCB / BPW;               // waves across the columns
  static constexpr int RGW = X * CW / kEncWaves;     // row groups per wave
  static constexpr int ROWS = 32 * X;                // rows per step
  static constexpr int UPS = 2 * X;                  // units per step
  static constexpr int LPW = 2 * X;                  // row loads (4 rows) per wave and step
  static constexpr int PT_BYTES = (b < 128 ? b : 128) * kHeadDim * 2; // P^T staging
  static constexpr int TILE_BYTES = 2 * ROWS * kTileRow;
  static constexpr int BUF_BYTES = PT_BYTES > TILE_BYTES ? PT_BYTES : TILE_BYTES;
  static constexpr int WAVES_PER_EU = NCB == 4 ? 3 : 2;
  static_assert(CW * (X / RGW) == kEncWaves, "the waves tile the step");
  static constexpr int PT_COLS = b < 128 ? b : 128;  // P^T columns staged at once
};

template <int NCB>
__global__ __launch_bounds__(kEncThreads)
__attribute__((amdgpu_waves_per_eu(EncShape<NCB>::WAVES_PER_EU, EncShape<NCB>::WAVES_PER_EU)))
void encode_mfma_kernel(const uint16_t *__restrict__ k_pool, int64_t num_blocks,
                        const int32_t *__restrict__ block_table, int max_blocks,
                        int batch, const int32_t *__restrict__ enc_start,
                        const int32_t *__restrict__ enc_end, int max_encode_len,
                        int pages_max, const uint16_t *__restrict__ proj, int Hkv,
                        uint32_t *__restrict__ codes, uint8_t *__restrict__ radii,
                        int round_wgs) {
  using E = EncShape<NCB>;
  constexpr int b = E::b, W = E::W, X = E::X, CW = E::CW, BPW = E::BPW, RGW = E::RGW;
  constexpr int ROWS = E::ROWS, UPS = E::UPS, LPW = E::LPW;
  // P^T while the fragments are taken, then the two step tiles
  __shared__ __align__(16) unsigned char sBuf[E::BUF_BYTES];
  uint16_t (*sPt)[kHeadDim] = reinterpret_cast<uint16_t (*)[kHeadDim]>(sBuf);
  __shared__ __align__(16) float sKb[2][ROWS];   // row bounds per step slot
  __shared__ __align__(16) int2 sUnit[2][kWin];  // (block id or -1, slice | rows << 16)
  __shared__ uint4 sQ[kEncWaves][kQueue];        // queued fp64 chains
  __shared__ int2 sRange[kRangeLds];
  // units before each sequence's first (balanced mode): sPre[s] = Hkv-free
  // count of the pages the ranges of sequences 0..s-1 meet
  __shared__ int sPre[kRangeLds + 1];
  __shared__ uint32_t sScan[kEncWaves];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int rg0 = RGW == X ? 0 : (wave / CW) * RGW; // the wave's first row group
  const int cb0 = (wave % CW) * BPW;                 // its first column block
  const int hf = lane >> 5, row = lane & 31;
  // positions a block table row reaches (the host keeps max_blocks at or
  // below DKV_MAX_SEQ_LEN / 16, so this fits an int)
  const int limit = (int)min((int64_t)kPage * max_blocks, (int64_t)DKV_MAX_SEQ_LEN);
  auto range_of = [&](int s_) __attribute__((always_inline)) {
    const int st = clamp_int(enc_start[s_], 0, limit);
    int en = clamp_int(enc_end[s_], 0, limit);
    if (en - st > max_encode_len) en = st + max_encode_len;
    return make_int2(st, en);
  };
  for (int i = threadIdx.x; i < batch && i < kRangeLds; i += kEncThreads) sRange[i] = range_of(i);
  __syncthreads();
  // Balanced mode (every sequence's range in LDS): only the pages the
  // ranges meet hold units, numbered sequence by sequence, so the runs hold
  // equal work in ragged batches.  Otherwise every sequence has pages_max
  // page slots, the ones past its range empty.
  const bool bal = batch <= kRangeLds; // workgroup-uniform
  auto pages_met = [](int2 rg_) { return rg_.y > rg_.x ? (rg_.y - 1) / kPage - rg_.x / kPage + 1 : 0; };
  if (bal) {
    constexpr int kPer = (kRangeLds + kEncThreads - 1) / kEncThreads;
    const int i0 = (int)threadIdx.x * kPer;
    uint32_t local = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (i0 + u < batch) local += (uint32_t)pages_met(sRange[i0 + u]);
    uint32_t total;
    uint32_t run = wg_exclusive_scan<kEncThreads>(local, sScan, &total);
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (i0 + u < batch) {
        sPre[i0 + u] = (int)run;
        run += (uint32_t)pages_met(sRange[i0 + u]);
      }
    if (threadIdx.x == 0) sPre[batch] = (int)total;
    __syncthreads();
  }
  // this wave's B fragments (columns 32 (cb0 + i) + L%32) and the largest
  // of their norms; P^T is staged PT_COLS columns at a time
  v8bf16 bfr[BPW][8];
  float n2max = 0.f;
  constexpr int PTC = E::PT_COLS;
  for (int c0 = 0; c0 < b; c0 += PTC) {
    if (c0 > 0) __syncthreads(); // the previous columns are read
    for (int e = threadIdx.x; e < kHeadDim * PTC; e += kEncThreads) {
      const int i = e / PTC, j = e % PTC;
      sPt[j][i] = proj[(int64_t)i * b + c0 + j];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      if (32 * (cb0 + i) < c0 || 32 * (cb0 + i) >= c0 + PTC) continue; // wave-uniform
      const uint16_t *pc = &sPt[32 * (cb0 + i) - c0 + row][64 * hf];
      float n2 = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        bfr[i][c] = as_v8bf16(*reinterpret_cast<const uint4 *>(pc + 8 * c));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (float)bfr[i][c][e];
          n2 = fmaf(x, x, n2);
        }
      }
      n2 += __shfl_xor(n2, 32);
      n2max = fmaxf(n2max, n2);
    }
  }
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) n2max = fmaxf(n2max, __shfl_xor(n2max, o));
  // the bound's factor for every row: (d+2) 2^-23 max_j |P_j| of the
  // workgroup's columns (each wave's own would do; one value keeps the row
  // bounds shareable)
  __shared__ float sCn[kEncWaves];
  if (lane == 0) sCn[wave] = n2max;
  constexpr float kBoundC = (float)(kHeadDim + 2) * 0x1p-23f;
  // m / Hkv = umulhi(m, ceil(2^32 / Hkv)) for m < 2^16 (Hkv > 1)
  const uint32_t hkv_magic = Hkv > 1 ? (uint32_t)((0x100000000ull + (uint32_t)Hkv - 1u) / (uint32_t)Hkv) : 0u;
  __syncthreads(); // P^T read: the buffer becomes the step tiles
  float cnall = 0.f;
#pragma unroll
  for (int i = 0; i < kEncWaves; ++i) cnall = fmaxf(cnall, sCn[i]);
  const float cnmax = sqrtf(cnall) * (1.f + 0x1p-20f);

  // Units u = ((s * pages_max + pi) * Hkv + q) (balanced: (sPre[s] + pi) *
  // Hkv + q): the slices of a page are neighbours.  Each workgroup walks a
  // run of UPS-aligned length.
  const int nunits = bal ? sPre[batch] * Hkv : batch * pages_max * Hkv;
  int u_begin, u_end;
  if (round_wgs > 0) {
    // One workgroup per CU and wave slot: WAVES_PER_EU rounds of round_wgs.
    // The waves of a SIMD issue oldest first, so with equal runs the later
    // rounds ended later (16 x 128K keys: 1236, 1329 and 1447 us on
    // average).  The runs are weighted 35 : 33 : 30 (two rounds: 21 : 19),
    // oldest first; the last round takes what is left.
    constexpr int R = E::WAVES_PER_EU;
    static_assert(R == 2 || R == 3, "two or three rounds");
    constexpr int w0 = R == 3 ? 35 : 21, w1 = R == 3 ? 33 : 19, wsum = R == 3 ? 98 : 40;
    const int r = min((int)blockIdx.x / round_wgs, R - 1);
    const int v = (int)blockIdx.x - r * round_wgs;
    auto run_of = [&](int wr) { // UPS-aligned run of a workgroup of weight wr
      const int64_t per = ((int64_t)nunits * wr + (int64_t)wsum * round_wgs - 1) /
                          ((int64_t)wsum * round_wgs);
      return (int)((per + UPS - 1) / UPS * UPS);
    };
    const int c0 = run_of(w0), c1 = R == 3 ? run_of(w1) : 0;
    const int64_t base_last = (int64_t)(c0 + c1) * round_wgs;
    const int rest = (int)max((int64_t)0, (int64_t)nunits - base_last);
    const int clast = ((rest + round_wgs - 1) / round_wgs + UPS - 1) / UPS * UPS;
    const int c = r == 0 ? c0 : (r == R - 1 ? clast : c1);
    const int64_t base = r == 0 ? 0 : (r == 1 ? (int64_t)c0 * round_wgs : base_last);
    u_begin = (int)min((int64_t)nunits, base + (int64_t)v * c);
    u_end = min(nunits, u_begin + c);
  } else {
    const int chunk = ((nunits + (int)gridDim.x - 1) / (int)gridDim.x + UPS - 1) / UPS * UPS;
    u_begin = min(nunits, (int)blockIdx.x * chunk);
    u_end = min(nunits, u_begin + chunk);
  }
  if (u_begin >= u_end) return; // the whole workgroup: no barrier is left waiting
  const int ntile = (u_end - u_begin + UPS - 1) / UPS;

  // Unit info of unit u (one thread per unit): the block table offset, the
  // slice and the rows to encode (0 past the run or past the range).
  const __amdgpu_buffer_rsrc_t bt_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t *>(block_table), 0, (uint32_t)(batch * max_blocks) * 4u,
      0x00020000u);
  auto unit_plan = [&](int u, int &bt_off, int &q, uint32_t &rows) __attribute__((always_inline)) {
    bt_off = 0;
    q = 0;
    rows = 0u;
    if (u >= u_end) return;
    q = u % Hkv;
    const int r = u / Hkv;
    int s_, pi;
    if (bal) { // the last sequence whose first page slot is at or before r
      int lo = 0, hi = batch; // sPre[lo] <= r < sPre[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sPre[mid] <= r) lo = mid;
        else hi = mid;
      }
      s_ = lo;
      pi = r - sPre[lo];
    } else {
      s_ = r / pages_max;
      pi = r % pages_max;
    }
    const int2 rg_ = s_ < kRangeLds ? sRange[s_] : range_of(s_);
    const int p = rg_.x / kPage + pi;
    bt_off = (int)(((uint32_t)s_ * (uint32_t)max_blocks + (uint32_t)p) * 4u); // past the table: reads 0
    // the page's rows of positions [lo, hi) are rows lo*Hkv .. hi*Hkv-1
    const int lo = max(rg_.x - p * kPage, 0), hi = min(rg_.y - p * kPage, kPage);
    const int a = max(lo * Hkv - kPage * q, 0), e = min(hi * Hkv - kPage * q, kPage);
    rows = e > a ? ((1u << e) - 1u) & ~((1u << a) - 1u) : 0u;
  };
  // window w's unit info: planned and its block id requested (by thread i
  // for unit u_begin + w*kWin + i), then written to LDS a window later
  int win_blk = 0, win_q = 0;
  uint32_t win_rows = 0u;
  auto win_request = [&](int w) __attribute__((always_inline)) {
    int off;
    unit_plan(u_begin + w * kWin + (int)threadIdx.x, off, win_q, win_rows);
    win_blk = __builtin_amdgcn_raw_buffer_load_b32(bt_rsrc, off, 0, 0);
  };
  auto win_store = [&](int w) __attribute__((always_inline)) {
    const bool ok = win_rows != 0u && win_blk >= 0 && win_blk < num_blocks;
    sUnit[w & 1][threadIdx.x] = make_int2(ok ? win_blk : -1, win_q | (int)((ok ? win_rows : 0u) << 16));
  };
  static_assert(kWin == kEncThreads, "one thread per unit of a window");
  static_assert(kWin % UPS == 0, "a step's units lie in one window");
  win_request(0);
  win_store(0);
  win_request(1);
  win_store(1);
  win_request(2);
  __syncthreads();
  // A step's units are read from the window in LDS where needed (index
  // arrays held in registers would be placed in scratch memory): (block id
  // or -1, slice | rows << 16).
  struct StepUnits {
    const int2 *su;
  };
  auto step_units = [&](int t, StepUnits &U) __attribute__((always_inline)) {
    const int i0 = t * UPS;
    U.su = &sUnit[(i0 / kWin) & 1][i0 % kWin];
  };
  // unit j of a step, j the same in every lane
  auto unit_uniform = [&](const StepUnits &U, int j, int &blk, int &q, uint32_t &rows)
      __attribute__((always_inline)) {
    const int2 v = U.su[j];
    blk = __builtin_amdgcn_readfirstlane(v.x);
    const int y = __builtin_amdgcn_readfirstlane(v.y);
    q = y & 0xFFFF;
    rows = (uint32_t)y >> 16;
  };
  // tile row r of a step (unit r / 16; r may differ between lanes) ->
  // (block, key index = the radius index; its code words start at key
  // index * W): the page's row m = 16q + r % 16 is position m / Hkv of
  // head m % Hkv
  auto key_index = [&](const StepUnits &U, int r) __attribute__((always_inline)) -> uint32_t {
    const int2 v = U.su[r >> 4];
    const uint32_t m = (uint32_t)(kPage * (v.y & 0xFFFF) + (r & 15));
    const uint32_t pos = Hkv == 1 ? m : __umulhi(m, hkv_magic);
    const uint32_t h = m - pos * (uint32_t)Hkv;
    return ((uint32_t)v.x * Hkv + h) * kPage + pos;
  };
  auto key_row = [&](const StepUnits &U, int r) __attribute__((always_inline)) -> uint32_t {
    const int2 v = U.su[r >> 4];
    return ((uint32_t)v.x * Hkv + (v.y & 0xFFFF)) * kPage + (r & 15);
  };

  // This wave's rows of a step: load instruction i covers step rows
  // 8X*wave + 4i .. +3, lane l the 16 bytes 16(l%16) of row +l/16.  Each
  // unit is read through a buffer over its 4 KB; a unit without rows has an
  // empty buffer and reads zeros.
  constexpr int row_bytes = kHeadDim * 2;
  auto load_rows = [&](const StepUnits &U, uint4 (&S)[LPW]) __attribute__((always_inline)) {
    // (a wave's rows lie in one unit: rows 8X*wave .. 8X*wave + 8X - 1)
    int blk, q;
    uint32_t rows_;
    unit_uniform(U, (8 * X * wave) >> 4, blk, q, rows_);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int r0 = 8 * X * wave + 4 * i; // wave-uniform
      const uint16_t *base = blk >= 0 ? k_pool + ((int64_t)blk * Hkv + q) * kPage * kHeadDim : k_pool;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t *>(base), 0, blk >= 0 ? (uint32_t)(kPage * row_bytes) : 0u, 0x00020000u);
      S[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs, ((r0 & 15) + (lane >> 4)) * row_bytes + 16 * (lane & 15), 0, 0));
    }
  };

  // the queue of uncertain signs: (key row, code word, column | bit << 8)
  uint32_t qn = 0;
  // The queued chains run one per lane (lanes past the queue do nothing),
  // reading the key row and P from memory (a form that needs few registers:
  // it runs inside the scoring).
  auto flush = [&]() __attribute__((always_inline)) {
    if (qn == 0) return; // wave-uniform
    // the words these entries patch were stored by this wave: let those
    // stores complete first (and the queue's LDS writes)
    wave_lds_sync();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if ((uint32_t)lane < qn) {
      const uint4 ent = sQ[wave][lane];
      const double v = row_chain_fp64(k_pool + (int64_t)ent.x * kHeadDim, proj, b, (int)(ent.z & 0xFFu));
      const uint32_t bit = 1u << (ent.z >> 8);
      if (v > 0.0)
        atomicOr(&codes[ent.y], bit);
      else
        atomicAnd(&codes[ent.y], ~bit);
    }
    qn = 0;
  };

  // Staging of this wave's rows of step t: the LDS tile, |k|^2 (fp32, the
  // 16 lanes of a row combined), the row bound and the radius code.
  auto stage = [&](int t, const StepUnits &U, const uint4 (&S)[LPW]) __attribute__((always_inline)) {
    unsigned char *tile = sBuf + (t & 1) * ROWS * kTileRow;
    float r2[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int r = 8 * X * wave + 4 * i + (lane >> 4);
      *reinterpret_cast<uint4 *>(tile + r * kTileRow + 16 * (lane & 15)) = S[i];
      const uint32_t wv[4] = {S[i].x, S[i].y, S[i].z, S[i].w};
      float a = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const v2bf16 x = __builtin_bit_cast(v2bf16, wv[u]);
        a = __builtin_amdgcn_fdot2_f32_bf16(x, x, a, false);
      }
      r2[i] = a;
    }
#pragma unroll
    for (int i = 0; i < LPW; ++i) r2[i] = row16_sum(r2[i]);
    // lane l: the row of load (l%16) / (16 / LPW), row 4i + l/16 of it
    constexpr int kSub = 16 / LPW;
    float v = r2[0];
#pragma unroll
    for (int i = 1; i < LPW; ++i)
      if ((lane & 15) / kSub == i) v = r2[i];
    const int r = 8 * X * wave + 4 * ((lane & 15) / kSub) + (lane >> 4);
    const bool lead = (lane & 15) % kSub == 0; // one lane per row
    const uint32_t rmask = ((uint32_t)U.su[r >> 4].y >> 16) >> (r & 15);
    const bool rin = (rmask & 1u) != 0u;
    // the row's bound; rows not encoded get -1, so no sign of theirs is
    // ever uncertain
    const float kb = rin ? fmaf(kBoundC * __builtin_amdgcn_sqrtf(v * (1.f + 0x1p-20f)), cnmax, 0x1p-100f) : -1.f;
    if (lead) sKb[t & 1][r] = kb;
    // the radius code, from the fp32 sum unless near a threshold
    int r8 = radius_code_certain(rin ? v : 0.f);
    const bool runc = r8 < 0;
    if (__ballot(runc && lead) != 0u) { // rare: the fp64 chain decides
      if (runc && lead)
        r8 = radius_code(row_chain_fp64(k_pool + (int64_t)key_row(U, r) * kHeadDim, nullptr, b, 0));
    }
    if (rin && lead) radii[key_index(U, r)] = (uint8_t)r8;
  };

  // Scoring of step t: this wave's row groups against its columns (all
  // matrix ops first, so that the groups' chains interleave).
  auto compute = [&](int t, const StepUnits &U) __attribute__((always_inline)) {
    uint32_t rm[RGW]; // rows to encode per row group
#pragma unroll
    for (int rgl = 0; rgl < RGW; ++rgl) {
      int blk_, q_;
      uint32_t lo, hi;
      unit_uniform(U, 2 * (rg0 + rgl), blk_, q_, lo);
      unit_uniform(U, 2 * (rg0 + rgl) + 1, blk_, q_, hi);
      rm[rgl] = lo | (hi << 16);
    }
    uint32_t rany = 0u;
#pragma unroll
    for (int rgl = 0; rgl < RGW; ++rgl) rany |= rm[rgl];
    if (rany == 0u) return; // wave-uniform
    const unsigned char *tile = sBuf + (t & 1) * ROWS * kTileRow;
    uint4 R[RGW][8];
#pragma unroll
    for (int rgl = 0; rgl < RGW; ++rgl)
#pragma unroll
      for (int c = 0; c < 8; ++c)
        R[rgl][c] = *reinterpret_cast<const uint4 *>(
            tile + (32 * (rg0 + rgl) + row) * kTileRow + 128 * hf + 16 * c);
    v16f32 acc[RGW][BPW];
#pragma unroll
    for (int rgl = 0; rgl < RGW; ++rgl)
#pragma unroll
      for (int i = 0; i < BPW; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[rgl][i][j] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int rgl = 0; rgl < RGW; ++rgl)
#pragma unroll
        for (int i = 0; i < BPW; ++i)
          acc[rgl][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_v8bf16(R[rgl][c]), bfr[i][c],
                                                                acc[rgl][i], 0, 0, 0);
    static_for<RGW>([&](auto RG) {
    constexpr int rgl = decltype(RG)::value;
    const int rg = rg0 + rgl;
    const uint32_t rmask = rm[rgl];
    if (rmask == 0u) return; // wave-uniform
    // bounds of result rows 8g + 4h + i (register j = 4g + i)
    v4f32 bq[4];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq)
      bq[gq] = *reinterpret_cast<const v4f32 *>(&sKb[t & 1][32 * rg + 8 * gq + 4 * hf]);
    // code words: lane l holds word l % BPW of the wave's columns for row
    // l / BPW of the row group
    uint32_t out = 0u;
    uint64_t anyu = 0u;
    static_for<16 * BPW>([&](auto I) {
      constexpr int i = decltype(I)::value / 16, j = decltype(I)::value % 16;
      constexpr int r0 = 8 * (j / 4) + (j % 4); // rows r0 (low half) and r0 + 4
      const float p = acc[rgl][i][j];
      const uint64_t m = __ballot(p > 0.f);
      out = write_lane<BPW * r0 + i>(out, (uint32_t)m);
      out = write_lane<BPW * (r0 + 4) + i>(out, (uint32_t)(m >> 32));
      anyu |= __ballot(fabsf(p) <= bq[j / 4][j % 4]);
      asm volatile("" : "+s"(anyu)); // folded in as they come
    });
    {
      const int r32 = lane / BPW;
      if (lane < 32 * BPW && ((rmask >> r32) & 1u))
        codes[key_index(U, 32 * rg + r32) * W + cb0 + lane % BPW] = out;
    }
    // Uncertain signs: the fp32 sign is stored above and the entry joins
    // the wave's queue, whose fp64 chains run 64 at a time (one per lane)
    // and patch the stored words.
    if (anyu != 0u) {
      // (the masks are taken again here rather than kept from above, which
      // would hold many scalar registers through the stores)
#pragma unroll
      for (int i = 0; i < BPW; ++i) asm volatile("" : "+v"(acc[rgl][i]));
      auto unc_of = [&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value / 16, j = decltype(I)::value % 16;
        return __ballot(fabsf(acc[rgl][i][j]) <= bq[j / 4][j % 4]);
      };
      // entry of (block i, register j) for this lane: its result row
      // 8(j/4) + 4h + j%4
      auto entry = [&](int i, int j) __attribute__((always_inline)) {
        const int r = 32 * rg + 8 * (j / 4) + 4 * hf + (j % 4);
        return make_uint4(key_row(U, r), key_index(U, r) * W + cb0 + i,
                          (uint32_t)(32 * (cb0 + i) + row) | ((uint32_t)row << 8), 0u);
      };
      // This lane's uncertain registers (bit 16 i + j for register j of
      // block i), their count, and the lane's place in the queue: the
      // counts of the lanes below, summed bit by bit with ballots (a count
      // is at most 16 * BPW <= 32, six bits).
      uint32_t um = 0u;
      static_for<16 * BPW>([&](auto I) {
        constexpr int i = decltype(I)::value / 16, j = decltype(I)::value % 16;
        um |= (fabsf(acc[rgl][i][j]) <= bq[j / 4][j % 4] ? 1u : 0u) << decltype(I)::value;
      });
      const uint32_t ucount = (uint32_t)__popc(um);
      uint32_t below = 0u, total = 0u;
#pragma unroll
      for (int bit = 0; bit < 6; ++bit) {
        const uint64_t m = __ballot((ucount >> bit) & 1u);
        below += lanes_below_u64(m) << bit;
        total += (uint32_t)__popcll(m) << bit;
      }
      if (qn + total > (uint32_t)kQueue) flush();
      if (total <= (uint32_t)kQueue) {
        // each lane lists its own entries, in register order
        uint32_t slot = qn + below;
        while (um != 0u) {
          const int e = __ffs(um) - 1;
          um &= um - 1u;
          sQ[wave][slot++] = entry(e / 16, e % 16);
        }
        qn += total;
      } else { // more than the queue holds (degenerate rows such as zero
               // keys): one (block, register) at a time
        uint32_t ulo = 0u, uhi = 0u; // lane e: the mask of (e / 16, e % 16)
        static_for<16 * BPW>([&](auto I) {
          const uint64_t unc = unc_of(I);
          ulo = write_lane<decltype(I)::value>(ulo, (uint32_t)unc);
          uhi = write_lane<decltype(I)::value>(uhi, (uint32_t)(unc >> 32));
        });
        for (int e = 0; e < 16 * BPW; ++e) {
          const uint64_t unc = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)ulo, e) |
                               ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)uhi, e) << 32);
          if (unc == 0u) continue; // wave-uniform
          if ((unc >> lane) & 1u) sQ[wave][lanes_below_u64(unc)] = entry(e / 16, e % 16);
          qn = (uint32_t)__popcll(unc);
          flush();
        }
      }
    }
    });
  };

  // The steps.  Rows of steps t+1..t+3 are in flight while step t is
  // scored; their register sets rotate through three slots (the loop is
  // unrolled three times, with one exit, so the load waits at its entry
  // count for every path).  The unit info of window w+1 is written, and
  // that of window w+2 requested, at the first step of window w, after the
  // step's barrier (the other slot's readers are past it).
  uint4 S[kAhead][LPW];
  StepUnits U0;
#pragma unroll
  for (int a = 0; a < kAhead; ++a) {
    StepUnits Ua;
    step_units(a, Ua);
    load_rows(Ua, S[a]);
    if (a == 0) U0 = Ua;
  }
  constexpr int kStepsPerWin = kWin / UPS;
  auto body = [&](auto Xc, int t) __attribute__((always_inline)) {
    constexpr int A = decltype(Xc)::value;
    stage(t, U0, S[A]);
    __syncthreads();
    if (t % kStepsPerWin == 0 && t > 0) { // first step of window w >= 1
      const int w = t / kStepsPerWin;
      win_store(w + 1);
      win_request(w + 2);
    }
    StepUnits Un;
    step_units(t + kAhead, Un); // (past the run: no rows, empty loads)
    load_rows(Un, S[A]);
    compute(t, U0);
    step_units(t + 1, U0);
  };
  int t = 0;
  for (; t + kAhead - 1 < ntile; t += kAhead) {
    body(std::integral_constant<int, 0>{}, t);
    body(std::integral_constant<int, 1>{}, t + 1);
    body(std::integral_constant<int, 2>{}, t + 2);
  }
  if (t < ntile) body(std::integral_constant<int, 0>{}, t);
  if (t + 1 < ntile) body(std::integral_constant<int, 1>{}, t + 1);
  flush();
}

} // namespace

hipError_t launch_encode(const uint16_t *k_pool, int64_t num_blocks,
                         const int32_t *block_table, int max_blocks, int batch,
                         const int32_t *enc_start, const int32_t *enc_end,
                         int max_encode_len, const uint16_t *proj, int Hkv,
                         int b, uint32_t *codes, uint8_t *radii,
                         hipStream_t stream) {
  if (max_encode_len <= 0 || batch <= 0) return hipSuccess;
  if (Hkv <= 0 || Hkv > 4096) return hipErrorInvalidValue; // rows of a page index in 16 bits
  // a range of n positions meets at most ceil(n/16) + 1 pages
  const int pages_max = (max_encode_len + kPage - 1) / kPage + 1;
  const int64_t nunits = (int64_t)batch * pages_max * Hkv;
  if (nunits > 0x7FFFFFFF - 65536) return hipErrorInvalidValue;
  if ((int64_t)batch * max_blocks >= (int64_t)1 << 30) return hipErrorInvalidValue;
  // queued fixes name key rows and code words with 32-bit indices
  if ((uint64_t)num_blocks * kPage * Hkv * (b / 32) >= (uint64_t)1 << 32)
    return hipErrorInvalidValue;
  // persistent workgroups (three per CU, two for b = 256), each walking a
  // run of units
  const int ncu = device_cu_count();
  auto groups = [&](int ups, int per_cu) {
    return std::min<int64_t>((nunits + ups - 1) / ups,
                             std::max<int64_t>(1, (int64_t)per_cu * ncu));
  };
#define DKV_ENCODE_CASE(BV, NCBV)                                              \
  if (b == BV) {                                                               \
    using E = EncShape<NCBV>;                                                  \
    hipLaunchKernelGGL((encode_mfma_kernel<NCBV>),                             \
                       dim3((unsigned)groups(E::UPS, E::WAVES_PER_EU)),        \
                       dim3(kEncThreads), 0, stream, k_pool, num_blocks,       \
                       block_table, max_blocks, batch, enc_start, enc_end,     \
                       max_encode_len, pages_max, proj, Hkv, codes, radii,     \
                       groups(E::UPS, E::WAVES_PER_EU) ==                      \
                               (int64_t)E::WAVES_PER_EU * ncu ? ncu : 0);      \
    return hipGetLastError();                                                  \
  }
  DKV_ENCODE_CASE(64, 2)
  DKV_ENCODE_CASE(128, 4)
  DKV_ENCODE_CASE(256, 8)
#undef DKV_ENCODE_CASE
  return hipErrorInvalidValue;
}

} // namespace dkv
