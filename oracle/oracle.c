/*
 * oracle.c -- plain, slow, obviously-correct CPU model of the CSA2 sparse-attention
 * step over an FP4 global KV cache.
 *
 * THIS IS TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load it.  It shares no code, header or table with the GPU
 * library; both sides only consume the same seeded input arrays.
 *
 * Sources (web pages on DeepSeek-V4.1-Flash; cited by page title and section):
 *   [EXP]  "DeepSeek-V4.1-Flash, explique pas a pas" (cours-interactifs):
 *            intro (attention = dot products -> softmax -> weighted mean of values),
 *            attention forms (SWA of the last 128 tokens; indexer keeps the best k),
 *            CSA2 section (main KV entries of m tokens, light indexer, main attention),
 *            FP4 KV cache section (E2M1, E4M3 scale per 16 channels, MXFP4 indexer,
 *            448 x 6 = 2688 range bound, 288 B / 68 B entries, 890 B/token).
 *   [RES]  "Resume executif" (mkdocs reaper), "Les quatre mecanismes": CSA2 mode table,
 *            writer layers 2/8/14/20, 4.5 and 4.25 bits per channel; result table.
 *   [VID]  "DeepSeek V4.1 Flash et le cerveau divise", memory section: Full / Reindex /
 *            Reuse semantics (Reuse takes the latest indices).
 *   [LIN]  "La lignee DeepSeek": MLA shares one latent among all heads; DSA = light
 *            indexer + top-K.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - E2M1 magnitudes {0,.5,1,1.5,2,3,4,6}: the only 1/2/1-bit float with max 6.
 *   - E4M3 is the OCP E4M3FN variant (its max is the 448 the pages quote).
 *   - NV16 scale = E4M3FN value nearest to amax/6 (ties to even), saturating at 448.
 *   - MX32 scale = 2^(floor(log2 amax) - 2) (OCP MX rule, E2M1 emax = 2); amax = 0 -> 2^-127.
 *   - element code = nearest of the 8 magnitudes times the scale, ties to the even
 *     index; the sign bit is copied from the input (so -0.3s -> code 0x8).
 *   - a zero NV16 scale (amax/6 rounds to 0) gives signed-zero codes.
 *   - index score: d_h = exact MXFP4 dot rounded once to fp32; r_h = max(d_h, +0);
 *     s = fma chain over h = 0..Hi-1 from +0 (score = sum_h w_h ReLU(q_h . k)).
 *   - top-K: numeric score descending, ties to the lower index; output ascending
 *     by index, -1 padded when fewer than k entries are visible.
 *   - attention: every selected latent row and every window row is both key and
 *     value for all heads; one softmax over the union; fp64 arithmetic.
 *   - FP8 window ([EXP] FP4 KV cache section: the SWA KV stays in FP8): E4M3FN codes
 *     and one E8M0 scale per 512-channel window row, X = the smallest power of two
 *     with amax <= 448 X (no code saturates); code = E4M3FN nearest to x / X, ties
 *     to the even byte, sign copied; amax = 0 -> X = 2^-127.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define LATENT_DIM 512
#define INDEX_DIM 128
#define NV_BLOCK 16
#define MX_BLOCK 32

/* ------------------------------------------------------------------ formats -- */

/* bf16 bits -> exact double. */
double oracle_bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent field 0 is
 * subnormal (m * 0.5).  Built from the bit fields, not from a table. */
double oracle_e2m1_value(uint8_t code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* OCP E4M3FN: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is
 * subnormal (m * 2^-9); S.1111.111 is NaN; there is no infinity. */
double oracle_e4m3_value(uint8_t b) {
  int s = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) mag = ldexp((double)m, -9);
  else mag = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* OCP E8M0: 2^(u-127); 255 is NaN. */
double oracle_e8m0_value(uint8_t u) {
  if (u == 255) return NAN;
  return ldexp(1.0, (int)u - 127);
}

/* Non-negative E4M3FN byte whose value is nearest to target/6 (ties to the even
 * byte, i.e. even mantissa), searched over every finite non-negative byte.  Working
 * with |6v - a| keeps the comparison exact in double (v has 4 significant bits). */
static uint8_t e4m3_nearest_sixth(double a) {
  /* saturation: beyond the largest finite value the nearest finite value is 448
   * (also keeps |6v - a| below from being compared at magnitudes where it rounds) */
  if (a >= 6.0 * 448.0) return 0x7E;
  uint8_t best = 0;
  double bestd = INFINITY;
  for (int b = 0; b <= 0x7E; ++b) {
    double d = fabs(6.0 * oracle_e4m3_value((uint8_t)b) - a);
    if (d < bestd || (d == bestd && (b & 1) == 0 && (best & 1) == 1)) {
      bestd = d;
      best = (uint8_t)b;
    }
  }
  return best;
}

/* Nearest of the 8 E2M1 magnitudes times `scale` to |x| (ties to the even index),
 * with the sign bit of x copied into bit 3.  |x|, M_i and scale are all exact in
 * double; for |x| < 6*scale, M_i*scale - |x| is exact wherever two candidates are
 * close enough to tie (|x| then lies next to a midpoint of similar magnitude). */
static uint8_t e2m1_nearest(double x, double scale) {
  double mag = fabs(x);
  /* at or beyond 6*scale the nearest magnitude is 6 (clipping); the differences
   * below are only compared where they are exact, i.e. |x| within the grid */
  if (mag >= 6.0 * scale) return (uint8_t)((signbit(x) ? 8 : 0) | 7);
  int best = 0;
  double bestd = INFINITY;
  for (int i = 0; i < 8; ++i) {
    double d = fabs(oracle_e2m1_value((uint8_t)i) * scale - mag);
    if (d < bestd || (d == bestd && (i & 1) == 0 && (best & 1) == 1)) {
      bestd = d;
      best = i;
    }
  }
  return (uint8_t)((signbit(x) ? 8 : 0) | best);
}

/* -------------------------------------------------------------- quantisers -- */

/* Main-cache block quantiser ([EXP] FP4 KV cache: E2M1 values, one E4M3 scale per
 * 16 channels, NVFP4 without its global scale).  x: 16 bf16 values.  codes: 16
 * unpacked codes.  Returns the scale byte. */
static uint8_t quant_nv16_block(const uint16_t* x, uint8_t* codes) {
  double a = 0.0;
  for (int i = 0; i < NV_BLOCK; ++i) a = fmax(a, fabs(oracle_bf16_value(x[i])));
  uint8_t sb = e4m3_nearest_sixth(a);
  double s = oracle_e4m3_value(sb);
  for (int i = 0; i < NV_BLOCK; ++i) {
    double v = oracle_bf16_value(x[i]);
    codes[i] = (s == 0.0) ? (uint8_t)(signbit(v) ? 8 : 0) : e2m1_nearest(v, s);
  }
  return sb;
}

/* Indexer block quantiser ([EXP] FP4 KV cache / [RES]: OCP MXFP4 = E2M1 values with
 * one E8M0 scale per 32 channels).  Returns the E8M0 byte. */
static uint8_t quant_mx32_block(const uint16_t* x, uint8_t* codes) {
  double a = 0.0;
  for (int i = 0; i < MX_BLOCK; ++i) a = fmax(a, fabs(oracle_bf16_value(x[i])));
  int u = 0;
  if (a > 0.0) {
    int e;
    frexp(a, &e); /* a = f * 2^e with f in [0.5, 1): floor(log2 a) = e - 1 */
    u = (e - 1) - 2 + 127;
    if (u < 0) u = 0;
    if (u > 254) u = 254;
  }
  double X = oracle_e8m0_value((uint8_t)u);
  for (int i = 0; i < MX_BLOCK; ++i) codes[i] = e2m1_nearest(oracle_bf16_value(x[i]), X);
  return (uint8_t)u;
}

/* Pack unpacked codes two per byte: channel 2k in bits 0-3, channel 2k+1 in 4-7. */
static void pack_nibbles(const uint8_t* codes, int n, uint8_t* out) {
  for (int k = 0; k < n / 2; ++k) out[k] = (uint8_t)(codes[2 * k] | (codes[2 * k + 1] << 4));
}

static uint8_t unpack_nibble(const uint8_t* packed, int c) {
  return (uint8_t)((packed[c >> 1] >> ((c & 1) * 4)) & 15);
}

/* Block quantisers over a flat array of nblk blocks (used by the tests). */
void oracle_quant_nv16(const uint16_t* x, int64_t nblk, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nblk; ++b) scales[b] = quant_nv16_block(x + b * NV_BLOCK, codes + b * NV_BLOCK);
}

void oracle_quant_mx32(const uint16_t* x, int64_t nblk, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nblk; ++b) scales[b] = quant_mx32_block(x + b * MX_BLOCK, codes + b * MX_BLOCK);
}

/* ------------------------------------------------------------ cache write -- */

/* Write n compressed entries into the global cache ([EXP] CSA2 section: entries of
 * the shared main KV and their indexer keys; FP4 KV cache section: quantised after
 * RoPE, same format for all 512 channels).  Row i goes to slot[i].
 * Layout per slot: main codes 256 B, main scales 32 B, indexer codes 64 B, indexer
 * scales 4 B.  Returns 0, or -1 on an out-of-range slot. */
int oracle_fp4_cache_write(uint8_t* main_codes, uint8_t* main_scales, uint8_t* idx_codes,
                           uint8_t* idx_scales, int64_t num_slots, const uint16_t* latent,
                           const uint16_t* idx_key, const int64_t* slot, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (slot[i] < 0 || slot[i] >= num_slots) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    int64_t s = slot[i];
    uint8_t codes[LATENT_DIM];
    for (int g = 0; g < LATENT_DIM / NV_BLOCK; ++g)
      main_scales[s * 32 + g] = quant_nv16_block(latent + i * LATENT_DIM + g * NV_BLOCK, codes + g * NV_BLOCK);
    pack_nibbles(codes, LATENT_DIM, main_codes + s * 256);
    for (int g = 0; g < INDEX_DIM / MX_BLOCK; ++g)
      idx_scales[s * 4 + g] = quant_mx32_block(idx_key + i * INDEX_DIM + g * MX_BLOCK, codes + g * MX_BLOCK);
    pack_nibbles(codes, INDEX_DIM, idx_codes + s * 64);
  }
  return 0;
}

/* Logical entry j of the sequence owning block-table row `row` -> physical slot. */
static int64_t slot_of(const int32_t* block_table, int32_t max_pages, int32_t page_size, int32_t row,
                       int64_t j) {
  return (int64_t)block_table[(int64_t)row * max_pages + j / page_size] * page_size + j % page_size;
}

/* ------------------------------------------------------- causal visibility -- */

/* Entries a query at token t may read ([EXP] CSA2 section: an entry compresses a
 * disjoint group of m consecutive tokens; intro: a token attends only to tokens at or
 * before it).  Entry j covers tokens m*j .. m*j + m - 1, so it exists for the query
 * at t once its last token m*j + m - 1 is at or before t.  The visible entries are
 * the prefix j = 0 .. J - 1 with J the number of j >= 0 satisfying
 *   m*j + m - 1 <= t   <=>   j <= (t + 1)/m - 1   <=>   j < floor((t + 1)/m),
 * so J = floor((t + 1)/m) (0 for t < m - 1).  A decode query is the context's last
 * token (t = ctx - 1); query i of a prefill chunk after a prefix of P tokens is at
 * t = P + i.  out[i] = J for token tok[i] (tok[i] >= -1). */
void oracle_causal_n_visible(const int64_t* tok, int64_t n, int32_t m, int32_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    int64_t t = tok[i];
    out[i] = (int32_t)((t + 1) / m);
  }
}

/* ------------------------------------------------------------ index score -- */

/* Signed E2M1 value times 2, an integer in [-12, 12]. */
static int e2m1_twice(uint8_t c) { return (int)lrint(2.0 * oracle_e2m1_value(c)); }

/* Lightning-indexer score ([EXP] CSA2 section: the indexer combines an indexer query
 * and one indexer key per entry; FP4 KV cache section: indexer queries and keys are
 * MXFP4).  Reading: score_j = sum_h w_h * ReLU(qhat_h . khat_j) with
 *   qhat = MX32 quantisation of q_idx (per head, 4 blocks of 32),
 *   d_h  = exact dot product of the dequantised vectors, rounded once to fp32,
 *   score = fmaf chain over h = 0..Hi-1 starting from +0.
 * Only positions j < n_visible[q] of scores[q] are written.
 * Returns the number of (query, head, entry) dots that were not exactly
 * representable in fp32; *inexact receives the number whose exact value could not
 * be formed in double (both must be 0 for the result to be unambiguous). */
/* The score of one entry (slot s) for a query whose MX32 codes / exponents are qc / qu
 * and whose head weights are wq.  Counts the dots not representable in fp32 and the
 * block sums not exact in double. */
static float score_entry(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t s, const uint8_t* qc,
                         const uint8_t* qu, const float* wq, int32_t Hi, int64_t* not_fp32, int64_t* not_exact) {
  const uint8_t* kp = idx_codes + s * 64;
  float acc = 0.0f;
  for (int h = 0; h < Hi; ++h) {
    double D = 0.0;
    for (int b = 0; b < 4; ++b) {
      long S = 0;
      for (int i = 0; i < MX_BLOCK; ++i) {
        int c = b * MX_BLOCK + i;
        S += (long)e2m1_twice(qc[h * INDEX_DIM + c]) * e2m1_twice(unpack_nibble(kp, c));
      }
      /* value = S/4 * 2^(uq-127) * 2^(uk-127) */
      double term = ldexp((double)S, (int)qu[h * 4 + b] + (int)idx_scales[s * 4 + b] - 254 - 2);
      double sum = D + term;
      double bb = sum - D;
      if ((D - (sum - bb)) + (term - bb) != 0.0) ++*not_exact;
      D = sum;
    }
    float d = (float)D;
    if ((double)d != D) ++*not_fp32;
    float r = d > 0.0f ? d : 0.0f;
    acc = fmaf(wq[h], r, acc);
  }
  return acc;
}

/* MX32 quantisation of query q's Hi heads: codes [Hi][128], exponents [Hi][4]. */
static void quant_query(const uint16_t* q_idx, int32_t Hi, int32_t q, uint8_t* qc, uint8_t* qu) {
  for (int h = 0; h < Hi; ++h)
    for (int b = 0; b < 4; ++b)
      qu[h * 4 + b] = quant_mx32_block(q_idx + ((int64_t)q * Hi + h) * INDEX_DIM + b * MX_BLOCK,
                                       qc + h * INDEX_DIM + b * MX_BLOCK);
}

int64_t oracle_index_score(const uint8_t* idx_codes, const uint8_t* idx_scales, const uint16_t* q_idx,
                           const float* w, int32_t Hi, const int32_t* seq_of_query,
                           const int32_t* n_visible, const int32_t* block_table, int32_t max_pages,
                           int32_t page_size, int32_t nq, float* scores, int64_t ld, int64_t* inexact) {
  int64_t not_fp32 = 0, not_exact = 0;
  for (int32_t q = 0; q < nq; ++q) {
    int32_t row = seq_of_query ? seq_of_query[q] : q;
    uint8_t* qc = (uint8_t*)malloc((size_t)Hi * INDEX_DIM);
    uint8_t* qu = (uint8_t*)malloc((size_t)Hi * 4);
    quant_query(q_idx, Hi, q, qc, qu);
    int64_t nv = n_visible[q];
#pragma omp parallel for schedule(dynamic, 256) reduction(+ : not_fp32, not_exact)
    for (int64_t j = 0; j < nv; ++j) {
      int64_t s = slot_of(block_table, max_pages, page_size, row, j);
      scores[(int64_t)q * ld + j] = score_entry(idx_codes, idx_scales, s, qc, qu, w + (int64_t)q * Hi, Hi,
                                                &not_fp32, &not_exact);
    }
    free(qc);
    free(qu);
  }
  if (inexact) *inexact = not_exact;
  return not_fp32;
}

/* ------------------------------------------------------------------ top-K -- */

typedef struct {
  float s;
  int64_t j;
} scored;

static int by_score_then_index(const void* pa, const void* pb) {
  const scored* a = (const scored*)pa;
  const scored* b = (const scored*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->j < b->j) ? -1 : (a->j > b->j);
}

static int by_index(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

/* Keep the k best entries per query ([EXP] attention forms / CSA2 section: the
 * indexer keeps the best-scoring entries).  Full sort by (score desc, index asc);
 * the first min(k, n) indices are emitted in ascending order, then -1 padding. */
void oracle_topk_select(const float* scores, int64_t ld, const int32_t* n_visible, int32_t nq, int32_t k,
                        int32_t* topk_idx) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t q = 0; q < nq; ++q) {
    int64_t n = n_visible[q];
    scored* all = (scored*)malloc(sizeof(scored) * (size_t)(n > 0 ? n : 1));
    for (int64_t j = 0; j < n; ++j) {
      all[j].s = scores[(int64_t)q * ld + j];
      all[j].j = j;
    }
    qsort(all, (size_t)n, sizeof(scored), by_score_then_index);
    int64_t m = n < k ? n : k;
    int32_t* out = topk_idx + (int64_t)q * k;
    for (int64_t i = 0; i < m; ++i) out[i] = (int32_t)all[i].j;
    qsort(out, (size_t)m, sizeof(int32_t), by_index);
    for (int64_t i = m; i < k; ++i) out[i] = -1;
    free(all);
  }
}

/* --------------------------------------------------------- candidate pool -- */

/* Hierarchical candidate pool ([VID] memory section: the first decoder layer scans the
 * whole global cache and assembles a pool of about 16,000 positions organised as 2048
 * blocks of 8; the layers after it may not search outside the pool).  The rule that
 * builds the pool is not on the pages; the reading here: blocks of POOL_BLOCK
 * consecutive entries are ranked by the largest score among their visible members,
 * ties to the lower block; the npool best form the pool, listed in ascending block
 * order and -1 padded.  That is the top-K rule applied to the block maxima. */
#define POOL_BLOCK 8
void oracle_pool_build(const float* scores, int64_t ld, const int32_t* n_visible, int32_t nq, int32_t npool,
                       int32_t* pool) {
  int64_t ldb = (ld + POOL_BLOCK - 1) / POOL_BLOCK;
  float* bmax = (float*)malloc(sizeof(float) * (size_t)(nq > 0 && ldb > 0 ? nq * ldb : 1));
  int32_t* nb = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nq > 0 ? nq : 1));
  for (int32_t q = 0; q < nq; ++q) {
    int64_t n = n_visible[q];
    nb[q] = (int32_t)((n + POOL_BLOCK - 1) / POOL_BLOCK);
    for (int64_t b = 0; b < nb[q]; ++b) {
      float m = scores[(int64_t)q * ld + b * POOL_BLOCK];
      for (int64_t j = b * POOL_BLOCK + 1; j < (b + 1) * POOL_BLOCK && j < n; ++j)
        if (scores[(int64_t)q * ld + j] > m) m = scores[(int64_t)q * ld + j];
      bmax[q * ldb + b] = m;
    }
  }
  oracle_topk_select(bmax, ldb, nb, nq, npool, pool);
  free(bmax);
  free(nb);
}

/* Scores over the pool: the index score (as in oracle_index_score) of every visible
 * member of the pool's blocks, written at pool position 8r + i for member i of the
 * pool's r-th block.  Positions of -1 blocks and of members at or past n_visible are
 * not written. */
int64_t oracle_index_score_pool(const uint8_t* idx_codes, const uint8_t* idx_scales, const uint16_t* q_idx,
                                const float* w, int32_t Hi, const int32_t* seq_of_query,
                                const int32_t* n_visible, const int32_t* pool, int32_t npool,
                                const int32_t* block_table, int32_t max_pages, int32_t page_size, int32_t nq,
                                float* scores, int64_t* inexact) {
  int64_t not_fp32 = 0, not_exact = 0;
  const int64_t ld = (int64_t)npool * POOL_BLOCK;
  for (int32_t q = 0; q < nq; ++q) {
    int32_t row = seq_of_query ? seq_of_query[q] : q;
    uint8_t* qc = (uint8_t*)malloc((size_t)Hi * INDEX_DIM);
    uint8_t* qu = (uint8_t*)malloc((size_t)Hi * 4);
    quant_query(q_idx, Hi, q, qc, qu);
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : not_fp32, not_exact)
    for (int64_t p = 0; p < ld; ++p) {
      int32_t blk = pool[(int64_t)q * npool + p / POOL_BLOCK];
      int64_t j = (int64_t)blk * POOL_BLOCK + p % POOL_BLOCK;
      if (blk < 0 || j >= n_visible[q]) continue;
      int64_t s = slot_of(block_table, max_pages, page_size, row, j);
      scores[(int64_t)q * ld + p] = score_entry(idx_codes, idx_scales, s, qc, qu, w + (int64_t)q * Hi, Hi,
                                                &not_fp32, &not_exact);
    }
    free(qc);
    free(qu);
  }
  if (inexact) *inexact = not_exact;
  return not_fp32;
}

/* Top-K inside the pool: the k best visible pool members by score, ties to the lower
 * entry, emitted as entry indices in ascending order, -1 padded. */
void oracle_topk_pool(const float* scores, const int32_t* pool, int32_t npool, const int32_t* n_visible,
                      int32_t nq, int32_t k, int32_t* topk_idx) {
  const int64_t ld = (int64_t)npool * POOL_BLOCK;
  for (int32_t q = 0; q < nq; ++q) {
    scored* all = (scored*)malloc(sizeof(scored) * (size_t)(ld > 0 ? ld : 1));
    int64_t m = 0;
    for (int64_t p = 0; p < ld; ++p) {
      int32_t blk = pool[(int64_t)q * npool + p / POOL_BLOCK];
      int64_t j = (int64_t)blk * POOL_BLOCK + p % POOL_BLOCK;
      if (blk < 0 || j >= n_visible[q]) continue;
      all[m].s = scores[(int64_t)q * ld + p];
      all[m].j = j;
      ++m;
    }
    qsort(all, (size_t)m, sizeof(scored), by_score_then_index);
    int64_t c = m < k ? m : k;
    int32_t* out = topk_idx + (int64_t)q * k;
    for (int64_t i = 0; i < c; ++i) out[i] = (int32_t)all[i].j;
    qsort(out, (size_t)c, sizeof(int32_t), by_index);
    for (int64_t i = c; i < k; ++i) out[i] = -1;
    free(all);
  }
}

/* -------------------------------------------------------------- attention -- */

/* Dequantise one main-cache slot exactly: value = E2M1(code) * E4M3(scale). */
static void dequant_main_row(const uint8_t* main_codes, const uint8_t* main_scales, int64_t s, double* x) {
  for (int c = 0; c < LATENT_DIM; ++c)
    x[c] = oracle_e2m1_value(unpack_nibble(main_codes + s * 256, c)) *
           oracle_e4m3_value(main_scales[s * 32 + c / NV_BLOCK]);
}

/* One query: softmax attention of all H heads over the rows X (nrows x 512, fp64).
 * z_x = scale * q_h . x; out_h = sum_x softmax(z)_x x; lse_h = log sum exp z.
 * With no rows at all: out = 0, lse = -inf. */
static void attend_rows(const uint16_t* q, int32_t H, const double* X, int64_t nrows, double scale, float* out,
                        float* lse) {
  double* z = (double*)malloc(sizeof(double) * (size_t)(nrows > 0 ? nrows : 1));
  for (int h = 0; h < H; ++h) {
    const uint16_t* qh = q + (int64_t)h * LATENT_DIM;
    if (nrows == 0) {
      for (int c = 0; c < LATENT_DIM; ++c) out[(int64_t)h * LATENT_DIM + c] = 0.0f;
      lse[h] = -INFINITY;
      continue;
    }
    double m = -INFINITY;
    for (int64_t r = 0; r < nrows; ++r) {
      double dot = 0.0;
      for (int c = 0; c < LATENT_DIM; ++c) dot += oracle_bf16_value(qh[c]) * X[r * LATENT_DIM + c];
      z[r] = scale * dot;
      if (z[r] > m) m = z[r];
    }
    double l = 0.0;
    for (int64_t r = 0; r < nrows; ++r) l += exp(z[r] - m);
    for (int c = 0; c < LATENT_DIM; ++c) {
      double o = 0.0;
      for (int64_t r = 0; r < nrows; ++r) o += exp(z[r] - m) / l * X[r * LATENT_DIM + c];
      out[(int64_t)h * LATENT_DIM + c] = (float)o;
    }
    lse[h] = (float)(m + log(l));
  }
  free(z);
}

/* Gather the selected main-cache rows of one query plus its window rows. */
static int64_t gather_rows(const uint8_t* main_codes, const uint8_t* main_scales, const int32_t* idx, int32_t k,
                           const int32_t* block_table, int32_t max_pages, int32_t page_size, int32_t row,
                           const uint16_t* win, int64_t win_first, int64_t win_end, double* X) {
  int64_t nrows = 0;
  for (int32_t i = 0; i < k; ++i) {
    if (idx[i] < 0) continue;
    dequant_main_row(main_codes, main_scales, slot_of(block_table, max_pages, page_size, row, idx[i]),
                     X + nrows * LATENT_DIM);
    ++nrows;
  }
  for (int64_t r = win_first; r < win_end; ++r, ++nrows)
    for (int c = 0; c < LATENT_DIM; ++c) X[nrows * LATENT_DIM + c] = oracle_bf16_value(win[r * LATENT_DIM + c]);
  return nrows;
}

/* Decode attention ([EXP] CSA2 section: the main query reads the selected entries
 * and the layer's own sliding-window KV; intro: softmax-weighted mean).  Sequence b
 * uses block-table row b, its topk_idx row (-1 = none) and window rows
 * [0, swa_len[b]) of swa[b] (row stride `window`). */
void oracle_sparse_attn_decode(const uint8_t* main_codes, const uint8_t* main_scales, const uint16_t* q,
                               int32_t H, const int32_t* topk_idx, int32_t k, const int32_t* block_table,
                               int32_t max_pages, int32_t page_size, const uint16_t* swa,
                               const int32_t* swa_len, int32_t window, float softmax_scale, int32_t B, float* out,
                               float* lse) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t b = 0; b < B; ++b) {
    double* X = (double*)malloc(sizeof(double) * (size_t)(k + window) * LATENT_DIM);
    int64_t nrows = gather_rows(main_codes, main_scales, topk_idx + (int64_t)b * k, k, block_table, max_pages,
                                page_size, b, swa + (int64_t)b * window * LATENT_DIM, 0, swa_len[b], X);
    attend_rows(q + (int64_t)b * H * LATENT_DIM, H, X, nrows, (double)softmax_scale,
                out + (int64_t)b * H * LATENT_DIM, lse + (int64_t)b * H);
    free(X);
  }
}

/* Prefill-chunk attention: query i sits at token chunk_start + i, uses topk_idx row
 * i and the window rows i .. i+window-1 of the chunk window buffer (buffer row r is
 * token chunk_start - window + 1 + r), skipping rows before swa_first_valid.  Only
 * queries listed in `which` (or all T if which == NULL, count = T) are computed;
 * outputs are written at the query's own row. */
void oracle_sparse_attn_prefill_chunk(const uint8_t* main_codes, const uint8_t* main_scales, const uint16_t* q,
                                      int32_t H, const int32_t* topk_idx, int32_t k, const int32_t* block_table,
                                      int32_t max_pages, int32_t page_size, int32_t T, const uint16_t* swa,
                                      int32_t swa_first_valid, int32_t window, float softmax_scale,
                                      const int32_t* which, int32_t count, float* out, float* lse) {
  if (!which) count = T;
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t w = 0; w < count; ++w) {
    int32_t i = which ? which[w] : w;
    double* X = (double*)malloc(sizeof(double) * (size_t)(k + window) * LATENT_DIM);
    int64_t first = i > swa_first_valid ? i : swa_first_valid;
    int64_t nrows = gather_rows(main_codes, main_scales, topk_idx + (int64_t)i * k, k, block_table, max_pages,
                                page_size, 0, swa, first, (int64_t)i + window, X);
    attend_rows(q + (int64_t)i * H * LATENT_DIM, H, X, nrows, (double)softmax_scale,
                out + (int64_t)i * H * LATENT_DIM, lse + (int64_t)i * H);
    free(X);
  }
}

/* ------------------------------------------------------------- FP8 window -- */

/* Non-negative E4M3FN byte nearest to a (0 <= a <= 448), ties to the even byte,
 * searched over every finite non-negative byte (values and differences exact in
 * double: a has at most 8 significant bits, each candidate 4). */
static uint8_t e4m3_nearest(double a) {
  uint8_t best = 0;
  double bestd = INFINITY;
  for (int b = 0; b <= 0x7E; ++b) {
    double d = fabs(oracle_e4m3_value((uint8_t)b) - a);
    if (d < bestd || (d == bestd && !(b & 1) && (best & 1))) {
      bestd = d;
      best = (uint8_t)b;
    }
  }
  return best;
}

/* Window rows in FP8 ([EXP] FP4 KV cache section: the window KV is kept in FP8 as it
 * is the more quantisation-sensitive part; the format below is the reading stated in
 * the header).  rows x [rows][512] bf16 -> codes [rows][512] E4M3FN, scales [rows]
 * E8M0. */
void oracle_swa_fp8_quant(const uint16_t* x, int64_t rows, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t* xr = x + r * LATENT_DIM;
    double amax = 0.0;
    for (int c = 0; c < LATENT_DIM; ++c) amax = fmax(amax, fabs(oracle_bf16_value(xr[c])));
    int e = -127;
    while (ldexp(448.0, e) < amax) ++e;
    scales[r] = (uint8_t)(e + 127);
    for (int c = 0; c < LATENT_DIM; ++c) {
      double v = oracle_bf16_value(xr[c]);
      codes[r * LATENT_DIM + c] = (uint8_t)((signbit(v) ? 0x80 : 0) | e4m3_nearest(ldexp(fabs(v), -e)));
    }
  }
}

/* FP8 window rows -> bf16 bit patterns of their exact values (E4M3FN x E8M0).
 * Returns the number of values that bf16 cannot hold exactly (0 for any row whose
 * scale is at least 2^-124). */
int64_t oracle_swa_fp8_dequant(const uint8_t* codes, const uint8_t* scales, int64_t rows, uint16_t* out) {
  int64_t bad = 0;
  for (int64_t r = 0; r < rows; ++r)
    for (int c = 0; c < LATENT_DIM; ++c) {
      double v = oracle_e4m3_value(codes[r * LATENT_DIM + c]) * oracle_e8m0_value(scales[r]);
      float f = (float)v;
      uint32_t u;
      memcpy(&u, &f, 4);
      uint16_t b = (uint16_t)(u >> 16);
      if ((double)f != v || oracle_bf16_value(b) != v) ++bad;
      out[r * LATENT_DIM + c] = b;
    }
  return bad;
}

/* -------------------------------------------------------------- footprint -- */

/* Bytes of one stored vector of `dim` channels: 4-bit E2M1 codes plus one 8-bit scale
 * per `block` channels ([EXP] FP4 KV cache section; [RES] bits per channel). */
int64_t oracle_entry_bytes(int64_t dim, int64_t block) { return dim * 4 / 8 + dim / block * 8 / 8; }

double oracle_bits_per_channel(int64_t block) { return 4.0 + 8.0 / (double)block; }

/* Global-cache bytes per token of a layer schedule: only layers that compute their
 * own cache (Full) store one, each holding 1/m entries per token of a 512-channel
 * main entry plus a 128-channel indexer key ([EXP] CSA2 section, 890 B/token
 * reconstruction).  mode: 0 = SWA only, 1 = Full, 2 = Reindex, 3 = Reuse. */
double oracle_global_bytes_per_token(const int32_t* mode, const int32_t* m, int32_t nlayers) {
  double per_entry = (double)(oracle_entry_bytes(LATENT_DIM, NV_BLOCK) + oracle_entry_bytes(INDEX_DIM, MX_BLOCK));
  double total = 0.0;
  for (int32_t l = 0; l < nlayers; ++l)
    if (mode[l] == 1) total += per_entry / (double)m[l];
  return total;
}

/* Number of OpenMP threads a parallel region of the oracle uses. */
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
/* threads of the parallel loops from now on (n <= 0 leaves the OpenMP default) */
void oracle_set_num_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}
