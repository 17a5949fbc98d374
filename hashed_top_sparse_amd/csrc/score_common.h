// score_common.h -- one wave scores one 16-key page on the gfx950 matrix
// cores (shared by the sampling, streaming and exact-fallback passes).
//
// [SPHERICAL KV, §2.1]: the logit is approximated straight from the stored
// radius and the packed angle code, without rebuilding the dense key.
//   s_h = sum_j q8_hj * (bit_j ? +1 : -1)   for the G heads of a KV group
//   S   = w * max_h s_h                      (exact integer, |S| < 2^31)
// with the key's radius weight w: its code r8 (log weight), or
// rne(2^(r8/16)), linear in the radius the code stands for.
//
// The per-page work is one 16x16x128 fp8 x fp4 matrix-core op per 128 code
// bits (operand layout: see qprep.hip):
//   - lane L holds word L/16 (+4 per K-step) of the key in slot L%16 (code
//     blocks are key-major: a key's b/32 words are contiguous); the word is
//     expanded to fp4 with 5 bit operations (nibble values 0.5/1/2/0.5 for
//     bits 4e+m, m = 0..3);
//   - the query operand holds 2*hi/f_m and 2*lo/f_m per head (q8 = 16*hi +
//     lo), and the accumulator starts at -Q in the low rows, so row 2h gives
//     2*D_hi and row 2h+1 gives 2*D_lo - Q exactly (D = sum_j q8_j*bit_j);
//   - s_h = 16*row(2h) + row(2h+1); the max over the group's heads uses the
//     gfx950 16/32-lane row swaps; S = w * max with a 24-bit integer multiply
//     (|w| < 2^16, |max| < 2^15).
// After scoring, lanes 0..15 hold S of the keys in slots 0..15.
#pragma once

#include "internal.h"

namespace dkv {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// u = S + 2^31 (mod 2^32) orders like S; u = 0 is below every score
constexpr uint32_t kScoreBias = 1u << 31;

__device__ __forceinline__ uint32_t biased_score(int S) {
  return (uint32_t)S + kScoreBias; // unsigned: wraps by definition
}

// Linear radius weight rne(2^(r8/16)) of code r8 (0..255).  2^(r8/16) lies
// at least 1.8e-7 (relative) from the nearest half-integer, so the double
// exp2 (error below 1e-15) rounds to the right integer.
__device__ __forceinline__ int radius_weight_linear(uint32_t r8) {
  return (int)__builtin_rint(exp2((double)r8 * 0.0625));
}

// Radius weight of code r8: the code itself, or linear when lin.
__device__ __forceinline__ int radius_weight(uint32_t r8, bool lin) {
  return lin ? radius_weight_linear(r8) : (int)r8;
}

// The same through wlut, the 256 linear weights in LDS (filled by the
// kernel when lin, before a barrier).  With a runtime `lin`, the compiler
// turns radius_weight's choice into a select that evaluates the fp64 exp2
// for every key, whichever weight is in use; a table read is cheap either
// way.
__device__ __forceinline__ int radius_weight_lut(uint32_t r8, bool lin,
                                                 const uint16_t *wlut) {
  return lin ? (int)wlut[r8 & 255u] : (int)r8;
}

// Fills wlut (LDS, 256 entries) with the linear weights; every thread of a
// workgroup of nt threads calls it, and a barrier must follow.
__device__ __forceinline__ void fill_linear_weights(uint16_t *wlut, int nt) {
  for (int i = threadIdx.x; i < 256; i += nt) wlut[i] = (uint16_t)radius_weight_linear((uint32_t)i);
}
constexpr uint32_t kBufferWord3 = 0x00020000u; // raw buffer, gfx9 family

template <int KS>
struct QueryOperand {
  v8i a[KS];
  v4f cinit;
  int scale; // E8M0 block scale 2^0 (127), held in a register
};

// 127 in a register the compiler cannot see through (a constant operand
// would be rematerialised before every matrix op).
__device__ __forceinline__ int unit_scale() {
  int s = 127;
  asm("" : "+v"(s));
  return s;
}

// The score operand of (sequence s, KV head g): qop [unit][KS][64][8]
// dwords and qneg [B][Hq] = -sum_j q8.
template <int KS, int G>
__device__ __forceinline__ QueryOperand<KS>
load_query_operand(const uint32_t *qop, const float *qneg, int unit, int s,
                   int g, int Hq, int lane) {
  QueryOperand<KS> op;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint4 *src = reinterpret_cast<const uint4 *>(
        qop + (((int64_t)unit * KS + ks) * 64 + lane) * 8);
    const uint4 x0 = src[0], x1 = src[1];
    op.a[ks][0] = (int)x0.x; op.a[ks][1] = (int)x0.y;
    op.a[ks][2] = (int)x0.z; op.a[ks][3] = (int)x0.w;
    op.a[ks][4] = (int)x1.x; op.a[ks][5] = (int)x1.y;
    op.a[ks][6] = (int)x1.z; op.a[ks][7] = (int)x1.w;
  }
  const int h0 = 2 * (lane >> 4), h1 = h0 + 1;
  const float *qn = qneg + (int64_t)s * Hq + (int64_t)g * G;
  const float q0 = qn[h0 < G ? h0 : 0], q1 = qn[h1 < G ? h1 : 0];
  op.cinit = v4f{0.f, h0 < G ? q0 : 0.f, 0.f, h1 < G ? q1 : 0.f};
  op.scale = unit_scale();
  return op;
}

// The operand's loaded parts, kept raw until used (the accumulator's start
// value is selected per lane only then), so a load issued well ahead is not
// waited for at once.
template <int KS>
struct QueryOperandRaw {
  v8i a[KS];
  float q0, q1;
};

template <int KS, int G>
__device__ __forceinline__ void load_query_operand_raw(const uint32_t *qop,
                                                       const float *qneg, int unit,
                                                       int s, int g, int Hq, int lane,
                                                       QueryOperandRaw<KS> &r) {
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint4 *src = reinterpret_cast<const uint4 *>(
        qop + (((int64_t)unit * KS + ks) * 64 + lane) * 8);
    const uint4 x0 = src[0], x1 = src[1];
    r.a[ks][0] = (int)x0.x; r.a[ks][1] = (int)x0.y;
    r.a[ks][2] = (int)x0.z; r.a[ks][3] = (int)x0.w;
    r.a[ks][4] = (int)x1.x; r.a[ks][5] = (int)x1.y;
    r.a[ks][6] = (int)x1.z; r.a[ks][7] = (int)x1.w;
  }
  const int h0 = 2 * (lane >> 4), h1 = h0 + 1;
  const float *qn = qneg + (int64_t)s * Hq + (int64_t)g * G;
  r.q0 = qn[h0 < G ? h0 : 0];
  r.q1 = qn[h1 < G ? h1 : 0];
}

template <int KS, int G>
__device__ __forceinline__ QueryOperand<KS> finish_query_operand(
    const QueryOperandRaw<KS> &r, int lane) {
  QueryOperand<KS> op;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) op.a[ks] = r.a[ks];
  const int h0 = 2 * (lane >> 4), h1 = h0 + 1;
  op.cinit = v4f{0.f, h0 < G ? r.q0 : 0.f, 0.f, h1 < G ? r.q1 : 0.f};
  op.scale = unit_scale();
  return op;
}

__device__ __forceinline__ v8i expand_code_word(uint32_t w) {
  v8i r;
  r[0] = (int)(w & 0x11111111u);
  r[1] = (int)(w & 0x22222222u);
  r[2] = (int)(w & 0x44444444u);
  r[3] = (int)((w >> 3) & 0x11111111u);
  r[4] = r[5] = r[6] = r[7] = 0;
  return r;
}

// max of two scores.  The scores are finite (integers), so the plain
// instruction is enough: fmaxf would first canonicalise operands that come
// from a lane permute.
__device__ __forceinline__ float max_score(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// After v_permlane16_swap(m, m) the two results hold 16-lane rows
// {0,0,2,2} and {1,1,3,3}; after v_permlane32_swap rows {0,1,0,1} and
// {2,3,2,3}.  The max of the pair is the max over the row pair.
__device__ __forceinline__ float max_rows16(float m) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(m),
                                                  __float_as_uint(m), false, false);
  return max_score(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_rows32(float m) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m),
                                                  __float_as_uint(m), false, false);
  return max_score(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Maximum over each 16-lane row, in every lane of the row: DPP swaps of
// neighbours (quad_perm 1,0,3,2), of pairs (quad_perm 2,3,0,1), of the two
// quads of each half-row (row_half_mirror) and of the two half-rows
// (row_mirror).  Every lane must call it.
__device__ __forceinline__ uint32_t row_max16(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false));
  return x;
}

// Lanes 0, 16, 32 and 48: the first lane of each 16-lane row.
constexpr uint64_t kRowHeads = 0x0001000100010001ull;

// Number of set bits of `mask` in lanes below the calling lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// S of the page whose code words (this lane's KS dwords) and radius byte
// are given; valid in lanes 0..15 (slot = lane).  lin selects the linear
// radius weight, read from wlut (radius_weight_lut).  Every lane must call
// it.
template <int KS, int G>
__device__ __forceinline__ int score_page(const QueryOperand<KS> &op,
                                          uint32_t (&cw_in)[KS], uint32_t r8,
                                          bool ok, bool lin, const uint16_t *wlut) {
  // The loaded words are first read here: without this the compiler may
  // move their first use (the radius conversion) up to the loads and wait
  // for each load as it is issued.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(cw_in[ks]));
  asm volatile("" : "+v"(r8));
  const uint32_t (&cw)[KS] = cw_in;
  v4f acc = op.cinit;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        op.a[ks], expand_code_word(cw[ks]), acc, 0, 4, 0, op.scale, 0, op.scale);
  // The matrix op needs all 64 lanes: pin its result in wave-uniform control
  // flow so the compiler cannot sink it into a lane-divergent branch.
  asm volatile("" : "+v"(acc));
  float m = 16.f * acc[0] + acc[1];
  if (G >= 2) m = fmaxf(m, 16.f * acc[2] + acc[3]);
  if (G >= 4) m = max_rows16(m);
  if (G >= 8) m = max_rows32(m);
  int S = ok ? __mul24(radius_weight_lut(r8, lin, wlut), (int)m) : 0;
  // computed in every lane so the radius load is not sunk into a store
  // branch (where it would wait for every outstanding load)
  asm volatile("" : "+v"(S));
  return S;
}

// max_h s_h of four pages at once: page j's 16 results end in lanes
// 16j..16j+15 (integers; exact).  cw[j] are this lane's code words of page
// j.  The per-page maxima sit in 16-lane rows 0 (heads 0,1), 1 (heads 2,3),
// 2 and 3 (heads 4..7 for G = 8); v_permlane16_swap(x0, x1) returns rows
// {x0.0, x1.0, x0.2, x1.2} and {x0.1, x1.1, x0.3, x1.3}, and
// v_permlane32_swap(y01, y23) returns {y01.0, y01.1, y23.0, y23.1}.  Every
// lane must call it.
template <int KS, int G>
__device__ __forceinline__ int score_quad_max(const QueryOperand<KS> &op,
                                              const uint32_t (&cw)[4][KS]) {
  // the four pages' matrix ops first (independent accumulators), then
  // their epilogues
  v4f acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc[j] = op.cinit;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          op.a[ks], expand_code_word(cw[j][ks]), acc[j], 0, 4, 0, op.scale, 0, op.scale);
  }
  int x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float m = 16.f * acc[j][0] + acc[j][1];
    if (G >= 2) m = max_score(m, 16.f * acc[j][2] + acc[j][3]);
    // all 64 lanes take part: keep the ops in wave-uniform control flow
    asm volatile("" : "+v"(m));
    if (G >= 8) m = max_rows32(m);
    x[j] = (int)m;
  }
  const auto a = __builtin_amdgcn_permlane16_swap((uint32_t)x[0], (uint32_t)x[1],
                                                  false, false);
  const auto b = __builtin_amdgcn_permlane16_swap((uint32_t)x[2], (uint32_t)x[3],
                                                  false, false);
  int y01 = (int)a[0], y23 = (int)b[0];
  if (G >= 4) {
    y01 = max(y01, (int)a[1]);
    y23 = max(y23, (int)b[1]);
  }
  const auto c = __builtin_amdgcn_permlane32_swap((uint32_t)y01, (uint32_t)y23,
                                                  false, false);
  return (int)c[0];
}

// score_quad_max with the four pages scored one after another (one
// accumulator and one expanded operand live at a time: fewer registers, for
// kernels that need many waves per SIMD); the maxima stay in fp32 (exact
// integers) through the row swaps and are converted once.
template <int KS, int G>
__device__ __forceinline__ int score_quad_max_seq(const QueryOperand<KS> &op,
                                                  const uint32_t (&cw)[4][KS]) {
  float x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v4f acc = op.cinit;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          op.a[ks], expand_code_word(cw[j][ks]), acc, 0, 4, 0, op.scale, 0,
          op.scale);
    float m = 16.f * acc[0] + acc[1];
    if (G >= 2) m = max_score(m, 16.f * acc[2] + acc[3]);
    // all 64 lanes take part: keep the op in wave-uniform control flow, and
    // in page order
    asm volatile("" : "+v"(m));
    if (G >= 8) m = max_rows32(m);
    x[j] = m;
  }
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[0]),
                                                  __float_as_uint(x[1]), false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[2]),
                                                  __float_as_uint(x[3]), false, false);
  float y01 = __uint_as_float(a[0]), y23 = __uint_as_float(b[0]);
  if (G >= 4) {
    y01 = max_score(y01, __uint_as_float(a[1]));
    y23 = max_score(y23, __uint_as_float(b[1]));
  }
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(y01),
                                                  __float_as_uint(y23), false, false);
  return (int)__uint_as_float(c[0]);
}

// 4x4 transpose across the four 16-lane rows: afterwards x[j] in row a holds
// what x[a] held in row j (for every lane position in the row).  A page
// quad loaded with lane 16j+c holding the code words of key c of page j
// becomes, in x[j], page j's matrix-core operand (lane L: word L/16 of key
// L%16).
__device__ __forceinline__ void transpose_rows(uint32_t (&x)[4]) {
  auto a = __builtin_amdgcn_permlane32_swap(x[0], x[2], false, false);
  auto b = __builtin_amdgcn_permlane32_swap(x[1], x[3], false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  x[0] = c[0];
  x[1] = c[1];
  x[2] = d[0];
  x[3] = d[1];
}

// Raw buffer views of the code and radius pools (byte sizes < 2^32).
struct PoolView {
  __amdgpu_buffer_rsrc_t code, radius;
  uint32_t page_code_bytes; // W*16*4
  int Hkv, g;
  int code_voff, radius_voff; // this lane's byte offsets within a page
};

__device__ __forceinline__ PoolView make_pool_view(const uint32_t *codes,
                                                   const uint8_t *radii,
                                                   uint32_t code_bytes,
                                                   uint32_t radius_bytes, int W,
                                                   int Hkv, int g, int lane) {
  PoolView v;
  v.code = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(codes), 0,
                                             code_bytes, kBufferWord3);
  v.radius = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(radii), 0,
                                               radius_bytes, kBufferWord3);
  const int code_dwords = W * kPage;
  v.page_code_bytes = (uint32_t)code_dwords * 4u;
  v.Hkv = Hkv;
  v.g = g;
  // Lane L: word L/16 of key L%16 (key-major block, W = b/32 words per
  // key).  For b = 64 the upper 32 lanes re-read words 0 and 1: the query
  // operand is zero at those k and fp4 has no NaN/Inf, so they add 0.
  const int W_ = code_dwords / kPage;
  v.code_voff = (lane & 15) * W_ * 4 + ((lane >> 4) & (W_ - 1)) * 4;
  v.radius_voff = lane & (kPage - 1);
  return v;
}

// Loads one page's code dwords and radius byte for this lane (blk must be
// wave-uniform; an invalid page reads page 0 and is flagged not ok).
template <int KS>
__device__ __forceinline__ void load_page(const PoolView &v, int blk, bool ok,
                                          uint32_t (&cw)[KS], uint32_t &r8) {
  const uint32_t ph =
      (uint32_t)__builtin_amdgcn_readfirstlane(ok ? blk : 0) * (uint32_t)v.Hkv +
      (uint32_t)v.g;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    cw[ks] = __builtin_amdgcn_raw_buffer_load_b32(v.code, v.code_voff + 16 * ks,
                                                  ph * v.page_code_bytes, 0);
  r8 = __builtin_amdgcn_raw_buffer_load_b8(v.radius, v.radius_voff,
                                           ph * (uint32_t)kPage, 0);
}

} // namespace dkv
