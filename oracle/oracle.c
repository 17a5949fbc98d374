/*
 * oracle.c -- plain, slow CPU reference for score-then-select sparse decode
 * attention.  TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and
 * the benchmark's CPU-baseline leg call it; the GPU library never links,
 * loads or calls it, and it shares no source with the GPU library.
 *
 * Every step is written the plainest way its definition allows: one key,
 * one bit, one query head at a time, sequential fp64 sums in index order,
 * a full sort for the top-k.  There is no blocking, no fusion and no
 * reordering of arithmetic.  OpenMP only runs independent (sequence,
 * KV-head) units -- or independent keys -- side by side; it never splits a
 * sum.
 *
 * Sources (web pages, cited by title and section):
 *  [SKV]  "SPHERICAL KV: Angle-Domain Attention and Rate-Distortion
 *         Retention for Efficient Long-Context Inference" (gist.science
 *         explainer), technical summary §2.1 Angle-Domain Attention and
 *         §2.3 System integration.
 *  [DASH] "DASH-KV: asymmetric hashing accelerates long-context LLM
 *         inference" (zingnex forum digest), sections on the asymmetric
 *         deep hashing idea, the dynamic mixed-precision architecture and
 *         "from quadratic to linear" (LSH buckets, Top-K pruning).
 *  [DSA]  "DeepSeek: why 1M context cannot be bought with memory -- from
 *         DSA to CSA/HCA" (forum print-out), section "starting from DSA"
 *         (indexer scores history, attention over the top-k only) and the
 *         CSA section (sliding window keeps recent tokens).
 *  [DYS]  DySCO review page, "mathematical model" item 1 (standard
 *         attention softmax(QK^T/sqrt(d))) and FAQ 3 (attention sink = a
 *         few initial tokens kept next to the recent window).
 *
 * The pages leave the concrete code open; the readings taken here are:
 *  - key code: b sign bits of a Gaussian projection p = k.P plus a u8
 *    log-quantised radius; query: int8 projection with one scale per KV
 *    group; score = r8 * max over the group's heads of sum_j q8_j*(+-1).
 *  - every projection is accumulated in double precision, index order.
 *
 * Layouts (all row-major, little-endian):
 *   bf16 values are passed as uint16_t bit patterns.
 *   key / value rows: [n][d]; projection P: [d][b]; code: [b/32] uint32,
 *   bit j of the code is bit (j mod 32) of word (j / 32).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_EXPORT __attribute__((visibility("default")))

/* bf16 -> double, exactly (a bf16 is the top half of an IEEE single). */
static double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* ---------------------------------------------------------------------- */
/* E1 -- key angle code.  [SKV §2.1]: a key is split into a radius and a
 * direction, and the direction is stored as a packed angle code.  [DASH]:
 * keys get the light encoder, computed once when cached.  Reading: bit j is
 * set when the projection of the key on column j of P is positive, where
 * the projection is the double-precision sum of k_i*P_ij taken in index
 * order i = 0..d-1 (each product of two bf16 values is exact in double).
 * A projection of exactly zero gives a clear bit. */
ORC_EXPORT void orc_key_code(const uint16_t *k, const uint16_t *P, int d, int b,
                             uint32_t *code) {
  for (int w = 0; w < b / 32; ++w) code[w] = 0u;
  for (int j = 0; j < b; ++j) {
    double acc = 0.0;
    for (int i = 0; i < d; ++i) {
      double prod = bf16_value(k[i]) * bf16_value(P[(size_t)i * b + j]);
      acc = acc + prod;
    }
    if (acc > 0.0) code[j / 32] |= 1u << (j % 32);
  }
}

/* Nearest doubles to 2^(f/8), f = 0..7 (hex literals). */
static const double ORC_EIGHTH_OCTAVE[8] = {
    0x1.0000000000000p+0, 0x1.172b83c7d517bp+0, 0x1.306fe0a31b715p+0,
    0x1.4bfdad5362a27p+0, 0x1.6a09e667f3bcdp+0, 0x1.8ace5422aa0dbp+0,
    0x1.ae89f995ad3adp+0, 0x1.d5818dcfba487p+0};

static int floor_div(int a, int b) {
  int q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) q -= 1;
  return q;
}

/* Threshold of radius code m (1..255) on the squared norm:
 * T[m] = 2^((m-64)/8), built as C[(m-64) mod 8] * 2^floor((m-64)/8). */
ORC_EXPORT double orc_radius_threshold(int m) {
  int t = m - 64;
  int q = floor_div(t, 8);
  int f = t - 8 * q;
  return ldexp(ORC_EIGHTH_OCTAVE[f], q);
}

/* E2 -- u8 log-quantised radius.  [SKV §2.1]: the scalar radius r = |k| is
 * stored quantised.  Reading: 16 codes per octave of r (8 per octave of
 * r^2), zero point 64; r8 is the largest m in 1..255 with r^2 >= T[m], or 0
 * when r^2 < T[1].  r^2 is the index-order double sum of squares. */
ORC_EXPORT double orc_sq_norm(const uint16_t *k, int d) {
  double acc = 0.0;
  for (int i = 0; i < d; ++i) {
    double x = bf16_value(k[i]);
    acc = acc + x * x;
  }
  return acc;
}

ORC_EXPORT int orc_radius_code(double r2) {
  for (int m = 255; m >= 1; --m)
    if (r2 >= orc_radius_threshold(m)) return m;
  return 0;
}

/* Encode n keys (rows of K, [n][d]) into codes [n][b/32] and radii [n]. */
ORC_EXPORT void orc_encode_keys(int64_t n, int d, int b, const uint16_t *K,
                                const uint16_t *P, uint32_t *codes,
                                uint8_t *radii) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t) {
    orc_key_code(K + t * d, P, d, b, codes + t * (b / 32));
    radii[t] = (uint8_t)orc_radius_code(orc_sq_norm(K + t * d, d));
  }
}

/* ---------------------------------------------------------------------- */
/* Q1 -- query int8 projection.  [DASH]: queries take the deeper, higher
 * precision encoder.  Reading: p_hj = index-order double sum of q_hi*P_ij;
 * one symmetric scale per KV group, M = max |p| over the group's G heads
 * and all b columns; q8 = round-half-even((p*127)/M), clamped to +-127, or
 * 0 when M == 0.  Input q: [G][d]; output q8: [G][b]. */
ORC_EXPORT void orc_query_int8(const uint16_t *q, int G, const uint16_t *P,
                               int d, int b, int8_t *q8) {
  double *p = (double *)malloc(sizeof(double) * (size_t)G * b);
  double M = 0.0;
  for (int h = 0; h < G; ++h) {
    for (int j = 0; j < b; ++j) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i) {
        double prod = bf16_value(q[(size_t)h * d + i]) *
                      bf16_value(P[(size_t)i * b + j]);
        acc = acc + prod;
      }
      p[(size_t)h * b + j] = acc;
      if (fabs(acc) > M) M = fabs(acc);
    }
  }
  for (int t = 0; t < G * b; ++t) {
    if (M == 0.0) {
      q8[t] = 0;
      continue;
    }
    double scaled = p[t] * 127.0;
    double ratio = scaled / M;
    double r = nearbyint(ratio); /* default rounding mode: half to even */
    if (r > 127.0) r = 127.0;
    if (r < -127.0) r = -127.0;
    q8[t] = (int8_t)r;
  }
  free(p);
}

/* ---------------------------------------------------------------------- */
/* W1 -- radius weight of a key in the score.  [SKV §2.1]: the approximate
 * logit multiplies the similarity of the angle codes by the key's radius
 * as decoded from its stored code.  Two readings, chosen per call:
 *   mode 0: the weight is the u8 log code r8 itself;
 *   mode 1: the weight grows linearly with the radius the code stands
 *           for.  Code r8 covers |k| in [2^((r8-64)/16), 2^((r8-63)/16));
 *           its lower edge scaled by 2^4 and rounded to the nearest integer
 *           is w = rne(2^(r8/16)), from 1 (r8 = 0) to 62757 (r8 = 255).
 *           2^4 is the largest power-of-two scale that keeps
 *           |S| <= 62757 * 127 * 256 < 2^31.
 * 2^(r8/16) is irrational unless 16 divides r8, so it is never a tie; it
 * lies at least 1.8e-7 (relative) from the nearest half-integer, far above
 * the error of exp2 in double precision. */
ORC_EXPORT int32_t orc_radius_weight(int r8, int mode) {
  if (mode == 0) return r8;
  return (int32_t)nearbyint(exp2((double)r8 / 16.0));
}

/* ---------------------------------------------------------------------- */
/* S1 -- code-domain score.  [SKV §2.1]: the logit is approximated from the
 * stored radius times a cosine-like similarity computed on the angle codes,
 * with no dense key rebuilt.  [DSA, "starting from DSA"]: a light indexer
 * scores every cached key.  Reading: s_h = sum_j q8_hj * (bit_j ? +1 : -1)
 * per query head of the group, S = wgt * max_h s_h, all exact integers,
 * where wgt is the key's radius weight (W1; r8 itself in mode 0). */
ORC_EXPORT int32_t orc_score(const int8_t *q8, int G, int b,
                             const uint32_t *code, int32_t wgt) {
  int32_t best = 0;
  for (int h = 0; h < G; ++h) {
    int32_t s = 0;
    for (int j = 0; j < b; ++j) {
      int bit = (int)((code[j / 32] >> (j % 32)) & 1u);
      int32_t qv = q8[(size_t)h * b + j];
      s += bit ? qv : -qv;
    }
    if (h == 0 || s > best) best = s;
  }
  return wgt * best;
}

/* ---------------------------------------------------------------------- */
/* T1 -- selection.  [DASH, Top-K pruning] and [DSA]: exact attention only
 * over the best-scored keys; [DSA, CSA section]: a sliding window keeps the
 * most recent tokens; [DYS, FAQ 3]: a few initial tokens (attention sinks)
 * are kept too.  Reading: sinks = [0, min(sigma,N)); window =
 * [max(min(sigma,N), N-w), N); candidates = [sigma, N-w); the top
 * min(k, |candidates|) candidates under (score descending, position
 * ascending) join them.  Returns the count; sel gets positions, sinks
 * first, then the window, then the top-k in rank order. */
typedef struct {
  int32_t score;
  int32_t pos;
} orc_cand;

static int orc_cand_cmp(const void *a, const void *b) {
  const orc_cand *x = (const orc_cand *)a, *y = (const orc_cand *)b;
  if (x->score != y->score) return (x->score > y->score) ? -1 : 1;
  return (x->pos < y->pos) ? -1 : (x->pos > y->pos);
}

ORC_EXPORT int orc_select(const int32_t *S, int N, int k, int w, int sigma,
                          int32_t *sel) {
  int n = 0;
  int ns = sigma < N ? sigma : N;
  for (int i = 0; i < ns; ++i) sel[n++] = i;
  int ws = (N - w > ns) ? N - w : ns;
  for (int i = ws; i < N; ++i) sel[n++] = i;
  int c0 = sigma, c1 = N - w;
  int nc = c1 - c0;
  if (nc <= 0) return n;
  orc_cand *c = (orc_cand *)malloc(sizeof(orc_cand) * (size_t)nc);
  for (int i = 0; i < nc; ++i) {
    c[i].score = S[c0 + i];
    c[i].pos = c0 + i;
  }
  qsort(c, (size_t)nc, sizeof(orc_cand), orc_cand_cmp);
  int keff = k < nc ? k : nc;
  for (int i = 0; i < keff; ++i) sel[n++] = c[i].pos;
  free(c);
  return n;
}

/* ---------------------------------------------------------------------- */
/* T2 -- page-granular selection.  [DSA, CSA section]: several history
 * tokens are first condensed into one entry and the top-k is taken over
 * those entries, not over single tokens; [SKV §2.2]: states grouped into
 * pages are read as one stream instead of scattered rows.  Reading: the
 * entry is the 16-token page.  A page's score is the largest key score S_i
 * over its keys inside the candidate range C = [sigma, N-w); the best
 * min(k/16, pages meeting C) pages by (page score descending, page index
 * ascending) are selected, and every key of theirs inside C joins the sinks
 * and the window (so the list never exceeds sigma + w + k).  Returns the
 * count; sel gets sinks, window, then the selected pages' keys, page by
 * page in rank order, ascending inside a page. */
ORC_EXPORT int orc_select_pages(const int32_t *S, int N, int k, int w,
                                int sigma, int32_t *sel) {
  const int page = 16;
  int n = 0;
  int ns = sigma < N ? sigma : N;
  for (int i = 0; i < ns; ++i) sel[n++] = i;
  int ws = (N - w > ns) ? N - w : ns;
  for (int i = ws; i < N; ++i) sel[n++] = i;
  int c0 = sigma, c1 = N - w;
  if (c1 <= c0) return n;
  int p0 = c0 / page, p1 = (c1 + page - 1) / page; /* pages meeting C */
  int np = p1 - p0;
  orc_cand *c = (orc_cand *)malloc(sizeof(orc_cand) * (size_t)np);
  for (int p = p0; p < p1; ++p) {
    int lo = p * page > c0 ? p * page : c0;
    int hi = (p + 1) * page < c1 ? (p + 1) * page : c1;
    int32_t best = S[lo];
    for (int i = lo + 1; i < hi; ++i)
      if (S[i] > best) best = S[i];
    c[p - p0].score = best;
    c[p - p0].pos = p;
  }
  qsort(c, (size_t)np, sizeof(orc_cand), orc_cand_cmp); /* pos = page */
  int kp = k / page;
  int keff = kp < np ? kp : np;
  for (int r = 0; r < keff; ++r) {
    int p = c[r].pos;
    int lo = p * page > c0 ? p * page : c0;
    int hi = (p + 1) * page < c1 ? (p + 1) * page : c1;
    for (int i = lo; i < hi; ++i) sel[n++] = i;
  }
  free(c);
  return n;
}

/* ---------------------------------------------------------------------- */
/* H1 -- bucket of a code in LSH table t.  [DASH, "from quadratic to
 * linear"]: several hash tables split the vector space into regions, so
 * that similar vectors land in the same bucket.  The code bits are already
 * signs of random projections (SimHash), so table t takes m of them: code
 * bits t*m .. t*m+m-1, bit t*m+i giving bit i of the bucket number. */
ORC_EXPORT int orc_lsh_bucket(const uint32_t *code, int t, int m) {
  int v = 0;
  for (int i = 0; i < m; ++i) {
    int j = t * m + i;
    v |= (int)((code[j / 32] >> (j % 32)) & 1u) << i;
  }
  return v;
}

/* T3 -- selection over the LSH candidates.  [DASH, "from quadratic to
 * linear"]: a new query computes its hash, looks only in its buckets for
 * candidate keys, and the candidates are pruned to the top-k that enter
 * exact attention.  Reading: the query's hash in table t is built from the
 * signs of its own projection on the same columns (qbits: the E1 code of
 * the query row, one per query head of the group); a key in [sigma, N-w)
 * is a candidate when, for some table and some head, its bucket equals the
 * head's; the min(k, candidates) best candidates by (S descending,
 * position ascending) join the sinks and the window.  codes: [N][W];
 * qbits: [G][W].  Returns the count. */
ORC_EXPORT int orc_select_lsh(const int32_t *S, const uint32_t *codes, int W,
                              const uint32_t *qbits, int G, int T, int m,
                              int N, int k, int w, int sigma, int32_t *sel) {
  int n = 0;
  int ns = sigma < N ? sigma : N;
  for (int i = 0; i < ns; ++i) sel[n++] = i;
  int ws = (N - w > ns) ? N - w : ns;
  for (int i = ws; i < N; ++i) sel[n++] = i;
  int c0 = sigma, c1 = N - w;
  if (c1 <= c0) return n;
  orc_cand *c = (orc_cand *)malloc(sizeof(orc_cand) * (size_t)(c1 - c0));
  int nc = 0;
  for (int i = c0; i < c1; ++i) {
    int hit = 0;
    for (int t = 0; t < T && !hit; ++t) {
      int kb = orc_lsh_bucket(codes + (size_t)i * W, t, m);
      for (int h = 0; h < G && !hit; ++h)
        hit = kb == orc_lsh_bucket(qbits + (size_t)h * W, t, m);
    }
    if (hit) {
      c[nc].score = S[i];
      c[nc].pos = i;
      ++nc;
    }
  }
  qsort(c, (size_t)nc, sizeof(orc_cand), orc_cand_cmp);
  int keff = k < nc ? k : nc;
  for (int i = 0; i < keff; ++i) sel[n++] = c[i].pos;
  free(c);
  return n;
}

/* ---------------------------------------------------------------------- */
/* A1 -- exact attention over the selected keys.  [DYS, item 1]:
 * softmax(QK^T / sqrt(d)); [DSA]: the real attention runs only over the
 * selected history.  In double precision: l_t = (q.k_t)/sqrt(d),
 * a = softmax(l) (the maximum is subtracted first, which leaves the
 * softmax unchanged), o = sum_t a_t v_t.  q: [G][d]; K, V: [N][d]; out:
 * [G][d].  An empty selection gives o = 0. */
ORC_EXPORT void orc_attend(const uint16_t *q, int G, const uint16_t *K,
                           const uint16_t *V, int d, const int32_t *sel, int n,
                           double *out) {
  double *l = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int h = 0; h < G; ++h) {
    double *o = out + (size_t)h * d;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    if (n <= 0) continue;
    double mx = -INFINITY;
    for (int t = 0; t < n; ++t) {
      const uint16_t *kr = K + (size_t)sel[t] * d;
      double dot = 0.0;
      for (int i = 0; i < d; ++i)
        dot = dot + bf16_value(q[(size_t)h * d + i]) * bf16_value(kr[i]);
      l[t] = dot / sqrt((double)d);
      if (l[t] > mx) mx = l[t];
    }
    double den = 0.0;
    for (int t = 0; t < n; ++t) den = den + exp(l[t] - mx);
    for (int t = 0; t < n; ++t) {
      double a = exp(l[t] - mx) / den;
      const uint16_t *vr = V + (size_t)sel[t] * d;
      for (int c = 0; c < d; ++c) o[c] = o[c] + a * bf16_value(vr[c]);
    }
  }
  free(l);
}

/* ---------------------------------------------------------------------- */
/* One decode step for one (sequence, KV head) unit: Q1, S1 (with the W1
 * weight of radius_mode) for every cached key, T1 (or T2 when select_pages
 * is non-zero, or T3 over lsh_tables tables of lsh_bits bits when
 * lsh_tables > 0), A1.  q: [G][d] (the
 * group's query heads); codes [N][b/32]; radii [N]; K, V: [N][d] in logical
 * token order.  scores (length N) may be NULL.  sel must hold
 * min(N, sigma+w+k) entries.  Returns the count. */
ORC_EXPORT int orc_decode_unit(int G, int d, int b, int k, int w, int sigma,
                               int radius_mode, int select_pages,
                               int lsh_tables, int lsh_bits,
                               const uint16_t *q, const uint16_t *P,
                               const uint32_t *codes, const uint8_t *radii,
                               const uint16_t *K, const uint16_t *V, int N,
                               int8_t *q8, int32_t *scores, int32_t *sel,
                               double *out) {
  int32_t *S = scores ? scores
                      : (int32_t *)malloc(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
  orc_query_int8(q, G, P, d, b, q8);
  for (int i = 0; i < N; ++i)
    S[i] = orc_score(q8, G, b, codes + (size_t)i * (b / 32),
                     orc_radius_weight(radii[i], radius_mode));
  int n;
  if (lsh_tables > 0) {
    uint32_t *qbits = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)G * (b / 32));
    for (int h = 0; h < G; ++h)
      orc_key_code(q + (size_t)h * d, P, d, b, qbits + (size_t)h * (b / 32));
    n = orc_select_lsh(S, codes, b / 32, qbits, G, lsh_tables, lsh_bits, N, k, w,
                       sigma, sel);
    free(qbits);
  } else {
    n = select_pages ? orc_select_pages(S, N, k, w, sigma, sel)
                     : orc_select(S, N, k, w, sigma, sel);
  }
  orc_attend(q, G, K, V, d, sel, n, out);
  if (!scores) free(S);
  return n;
}

/* U independent units side by side (one OpenMP task each).  Per-unit
 * arrays are packed with stride Nmax along the token axis:
 *   q [U][G][d], codes [U][Nmax][b/32], radii [U][Nmax], K, V [U][Nmax][d],
 *   N [U], q8 [U][G][b], scores [U][Nmax] (or NULL), sel [U][sel_cap],
 *   sel_cnt [U], out [U][G][d]. */
ORC_EXPORT void orc_decode_units(int U, int G, int d, int b, int k, int w,
                                 int sigma, int radius_mode, int select_pages,
                                 int lsh_tables, int lsh_bits, const uint16_t *q,
                                 const uint16_t *P, const uint32_t *codes,
                                 const uint8_t *radii, const uint16_t *K,
                                 const uint16_t *V, const int32_t *N, int Nmax,
                                 int8_t *q8, int32_t *scores, int32_t *sel,
                                 int sel_cap, int32_t *sel_cnt, double *out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int u = 0; u < U; ++u) {
    size_t tok = (size_t)u * (size_t)Nmax;
    sel_cnt[u] = orc_decode_unit(
        G, d, b, k, w, sigma, radius_mode, select_pages, lsh_tables, lsh_bits,
        q + (size_t)u * G * d, P,
        codes + tok * (b / 32), radii + tok, K + tok * d, V + tok * d, N[u],
        q8 + (size_t)u * G * b, scores ? scores + tok : NULL,
        sel + (size_t)u * sel_cap, out + (size_t)u * G * d);
  }
}

/* Number of OpenMP threads a parallel region uses (for reporting). */
ORC_EXPORT int orc_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    {
#ifdef _OPENMP
      extern int omp_get_num_threads(void);
      n = omp_get_num_threads();
#endif
    }
  }
  return n;
}
