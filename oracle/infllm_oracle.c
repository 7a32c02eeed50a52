/*
 * infllm_oracle.c -- the oracle: a plain, slow, fp64 CPU statement of
 * InfLLM's context-memory attention step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or constant with the HIP
 * library: every rule below is written out again from the method's public
 * description.
 *
 * Sources (page title, section):
 *   [GUIDE]  "InfLLM Guide: Training-Free Long-Context Memory Units"
 *            (aifetchly blog): "Core Innovation 1: Structured Context
 *            Partitioning"; "Core Innovation 2: Semantic Representative Key
 *            Vectors & Dynamic Top-K Selection" (1. construction, 2. query-
 *            aware top-k scoring, 3. exact attention evaluation, Working
 *            Context equation); "Mathematical Modeling" (N_active).
 *   [SUMMARY] "InfLLM: Training-Free Long-Context Extrapolation for LLMs with
 *            an Efficient Context Memory" (atlas.scime.ai summary): "Approach";
 *            "Measured effects" table (representative tokens vs mean of keys;
 *            lookup during encoding and decoding).
 *   [REBUTTAL] the authors' OpenReview replies (paperhub.cn): "Q2:
 *            Representative Tokens"; "Q2: Comparison to Well-trained Long LLM"
 *            (retrieval in pre-filling is block based); "Q5: Latency Across
 *            Different Context Windows" (dot product against all units).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - units are absolute B-aligned blocks j >= floor(n_init/B) lying wholly
 *     inside the context; a unit's keys exclude the initial tokens;
 *   - the score a key earns for representative selection is the raw,
 *     unscaled sum of q.k over the queries of the G query heads of its KV
 *     head at the W positions that follow it (truncated at the context end);
 *   - ties: lower position wins among keys, lower index wins among units;
 *   - the local window of query t is the last W keys including t itself;
 *     a unit key counts only while it is at least W positions behind t;
 *   - a unit is eligible for a chunk once its first key lies at or before
 *     t_last - W; eligible units form a prefix of the unit index range;
 *   - one selection per chunk and KV head, shared by every query of the
 *     chunk and every query head of the group (decode = chunk of one);
 *   - the chunk score is (sum of the chunk's queries over the group) dot
 *     (unit representation), unscaled.
 *
 * Layout: every function works on one (sequence, KV head).  Query arrays
 * hold G heads, head g at q + g*q_head_stride, row i at +i*d.  Key/value
 * arrays are [positions, d] rows with row p = absolute position p.  Element
 * type dt: 0 = fp32, 1 = bf16 (raw 16-bit pattern); all arithmetic is fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Widen one stored element to double.  bf16 is the top half of an IEEE
 * binary32, so the widening is exact. */
static double ld(const void *base, int64_t idx, int32_t dt) {
  if (dt == 0) return (double)((const float *)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static int64_t mini64(int64_t a, int64_t b) { return a < b ? a : b; }
static int64_t maxi64(int64_t a, int64_t b) { return a > b ? a : b; }

int32_t orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------------------- */
/* Unit table.  [GUIDE] Core Innovation 1, item 3: the tokens before the
 * local window, minus the attention sinks, are cut into fixed contiguous
 * blocks of B tokens; its figure labels one unit "Tokens 1024 to 1151",
 * i.e. blocks are aligned to multiples of B.  [SUMMARY] Approach: "block-
 * level memory units".                                                     */

/* Number of units a context of n_ctx tokens holds. */
int64_t orc_num_units(int64_t n_ctx, int32_t B, int32_t n_init) {
  int64_t first_block = n_init / B;
  int64_t full_blocks = n_ctx / B;
  return full_blocks > first_block ? full_blocks - first_block : 0;
}

/* Key range [lo, hi) of unit u: block j = u + floor(n_init/B), without the
 * initial tokens. */
void orc_unit_keys(int64_t u, int32_t B, int32_t n_init, int64_t *lo,
                   int64_t *hi) {
  int64_t j = u + n_init / B;
  *lo = maxi64(j * B, n_init);
  *hi = (j + 1) * B;
}

/* Eligible units for a chunk whose last query sits at t_last: those with a
 * key outside every query's local window, i.e. first key <= t_last - W.   */
int64_t orc_num_eligible(int64_t t_last, int64_t U, int32_t B, int32_t n_init,
                         int32_t W) {
  int64_t e = 0;
  for (int64_t u = 0; u < U; ++u) {
    int64_t lo, hi;
    orc_unit_keys(u, B, n_init, &lo, &hi);
    if (lo <= t_last - W) e = u + 1;
  }
  return e;
}

/* ---------------------------------------------------------------------- */
/* Representative-token score.  [SUMMARY] Approach: each unit is represented
 * by its top-scoring tokens, scored with attention-based scores; [REBUTTAL]
 * Q2 (Representative Tokens): the model selects discrete tokens.  The score
 * of key p is the sum, over the G query heads of its KV head and over the
 * queries at positions p+1 .. min(p+W, n_ctx-1), of the raw product q.k_p. */
double orc_rep_score(const void *q, int64_t q_head_stride, int32_t G,
                     const void *k, int32_t d, int32_t dt, int64_t n_ctx,
                     int32_t W, int64_t p) {
  int64_t last = mini64(p + (int64_t)W, n_ctx - 1);
  double s = 0.0;
  for (int32_t g = 0; g < G; ++g) {
    const int64_t qoff = (int64_t)g * q_head_stride;
    for (int64_t i = p + 1; i <= last; ++i) {
      double dot = 0.0;
      for (int32_t c = 0; c < d; ++c)
        dot += ld(q, qoff + i * d + c, dt) * ld(k, p * d + c, dt);
      s += dot;
    }
  }
  return s;
}

typedef struct {
  double score;
  int64_t pos;
} scored_pos;

/* Order: higher score first; among equal scores the lower position first. */
static int cmp_desc_score_then_pos(const void *a, const void *b) {
  const scored_pos *x = (const scored_pos *)a, *y = (const scored_pos *)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->pos > y->pos) - (x->pos < y->pos);
}

static int cmp_i64(const void *a, const void *b) {
  int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
  return (x > y) - (x < y);
}

/* Build units u_lo .. u_hi-1 in representative-token mode.  For each unit:
 * score every key, keep the r_k best by (score desc, position asc), report
 * them in ascending position order (-1 pads if the unit has fewer keys), and
 * represent the unit by the sum of the kept keys.
 * Outputs, row i = unit u_lo+i:  rep_idx [n, r_k] int32 absolute positions;
 * repr [n, d]; key_scores [n, B] (slot = p - j*B, NaN for the initial-token
 * slots of a partial unit) -- may be NULL.                                   */
void orc_build_tokens(const void *q, int64_t q_head_stride, int32_t G,
                      const void *k, int32_t d, int32_t dt, int64_t n_ctx,
                      int32_t B, int32_t n_init, int32_t W, int32_t r_k,
                      int64_t u_lo, int64_t u_hi, int32_t *rep_idx,
                      double *repr, double *key_scores) {
  int64_t n_units = u_hi - u_lo;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_units; ++i) {
    int64_t lo, hi;
    orc_unit_keys(u_lo + i, B, n_init, &lo, &hi);
    int64_t n_keys = hi - lo;
    scored_pos *cand = (scored_pos *)malloc(sizeof(scored_pos) * n_keys);
    for (int64_t p = lo; p < hi; ++p) {
      cand[p - lo].pos = p;
      cand[p - lo].score = orc_rep_score(q, q_head_stride, G, k, d, dt, n_ctx,
                                         W, p);
    }
    if (key_scores) {
      int64_t block_start = hi - B;
      for (int32_t s = 0; s < B; ++s) key_scores[i * B + s] = NAN;
      for (int64_t m = 0; m < n_keys; ++m)
        key_scores[i * B + (cand[m].pos - block_start)] = cand[m].score;
    }
    qsort(cand, (size_t)n_keys, sizeof(scored_pos), cmp_desc_score_then_pos);
    int64_t n_keep = mini64(r_k, n_keys);
    int64_t kept[n_keep > 0 ? n_keep : 1];
    for (int64_t m = 0; m < n_keep; ++m) kept[m] = cand[m].pos;
    qsort(kept, (size_t)n_keep, sizeof(int64_t), cmp_i64);
    for (int32_t m = 0; m < r_k; ++m)
      rep_idx[i * r_k + m] = m < n_keep ? (int32_t)kept[m] : -1;
    for (int32_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int64_t m = 0; m < n_keep; ++m) acc += ld(k, kept[m] * d + c, dt);
      repr[i * d + c] = acc;
    }
    free(cand);
  }
}

/* Build units u_lo .. u_hi-1 in mean-of-keys mode ([SUMMARY] Measured
 * effects, the "mean key-vector representations" ablation, and Surprising
 * findings): the representation is the mean of the unit's keys.            */
void orc_build_mean(const void *k, int32_t d, int32_t dt, int32_t B,
                    int32_t n_init, int64_t u_lo, int64_t u_hi,
                    double *repr) {
  for (int64_t i = 0; i < u_hi - u_lo; ++i) {
    int64_t lo, hi;
    orc_unit_keys(u_lo + i, B, n_init, &lo, &hi);
    for (int32_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int64_t p = lo; p < hi; ++p) acc += ld(k, p * d + c, dt);
      repr[i * d + c] = acc / (double)(hi - lo);
    }
  }
}

/* ---------------------------------------------------------------------- */
/* Unit relevance.  [GUIDE] Core Innovation 2, item 2: a query is scored
 * against the representation of every unit by a dot product; [REBUTTAL] Q5:
 * the lookup takes the dot product between the query and all unit
 * representations; [REBUTTAL] Q2 (well-trained long LLM): in pre-filling
 * the lookup is done per block of queries.  The chunk score of unit u is
 * (sum over the chunk's L queries and the group's G heads of q) . repr[u];
 * units u >= e (not yet eligible) score -inf.                                */
void orc_score_units(const void *q, int64_t q_head_stride, int32_t G,
                     int32_t d, int32_t dt, int64_t L, const double *repr,
                     int64_t U, int64_t e, double *scores) {
  double *qsum = (double *)calloc((size_t)d, sizeof(double));
  for (int32_t g = 0; g < G; ++g)
    for (int64_t i = 0; i < L; ++i)
      for (int32_t c = 0; c < d; ++c)
        qsum[c] += ld(q, (int64_t)g * q_head_stride + i * d + c, dt);
  for (int64_t u = 0; u < U; ++u) {
    if (u >= e) {
      scores[u] = -INFINITY;
      continue;
    }
    double s = 0.0;
    for (int32_t c = 0; c < d; ++c) s += qsum[c] * repr[u * d + c];
    scores[u] = s;
  }
  free(qsum);
}

/* Top-k selection.  [GUIDE] Core Innovation 2, item 2: keep the k highest-
 * scoring units.  Only the e eligible units compete; min(k_m, e) are kept by
 * (score desc, index asc) and written in ascending index order, -1 pads.   */
void orc_topk(const double *scores, int64_t U, int64_t e, int32_t k_m,
              int32_t *sel) {
  (void)U;
  scored_pos *cand = (scored_pos *)malloc(sizeof(scored_pos) * (e > 0 ? e : 1));
  for (int64_t u = 0; u < e; ++u) {
    cand[u].score = scores[u];
    cand[u].pos = u;
  }
  qsort(cand, (size_t)e, sizeof(scored_pos), cmp_desc_score_then_pos);
  int64_t n_keep = mini64(k_m, e);
  int64_t kept[n_keep > 0 ? n_keep : 1];
  for (int64_t m = 0; m < n_keep; ++m) kept[m] = cand[m].pos;
  qsort(kept, (size_t)n_keep, sizeof(int64_t), cmp_i64);
  for (int32_t m = 0; m < k_m; ++m) sel[m] = m < n_keep ? (int32_t)kept[m] : -1;
  free(cand);
}

/* ---------------------------------------------------------------------- */
/* Working context.  [GUIDE] Core Innovation 2, item 3 (Working Context =
 * sinks + retrieved units + local window) and Core Innovation 1, items 1-2.
 * Key p is attended by query t iff p <= t and
 *   p < n_init                                  (initial tokens), or
 *   p > t - W                                   (local window, t included), or
 *   p >= n_init, p <= t - W, unit(p) selected   (retrieved units).          */
int orc_in_working_context(int64_t p, int64_t t, const int32_t *sel,
                           int32_t k_m, int32_t B, int32_t n_init, int32_t W) {
  if (p > t) return 0;
  if (p < n_init) return 1;
  if (p > t - W) return 1;
  int64_t u = p / B - n_init / B;
  for (int32_t m = 0; m < k_m; ++m)
    if (sel[m] >= 0 && (int64_t)sel[m] == u) return 1;
  return 0;
}

/* Positions attended by query t, ascending; returns their count.  out may be
 * NULL (count only). */
int64_t orc_working_context(int64_t t, const int32_t *sel, int32_t k_m,
                            int32_t B, int32_t n_init, int32_t W,
                            int64_t *out) {
  int64_t n = 0;
  for (int64_t p = 0; p <= t; ++p)
    if (orc_in_working_context(p, t, sel, k_m, B, n_init, W)) {
      if (out) out[n] = p;
      ++n;
    }
  return n;
}

/* Rotary position embedding ([GUIDE] "Operational Checklist", RoPE item:
 * the native base theta is kept): the pairs (c, c + d/2) of x are rotated
 * by the angle pos * theta^(-2c/d), c = 0 .. d/2 - 1 (rotate-half pairing).
 * A negative pos undoes the rotation at -pos. */
static void rope_rotate(double *x, int32_t d, double theta, double pos) {
  const int32_t h = d / 2;
  for (int32_t c = 0; c < h; ++c) {
    const double a = pos * pow(theta, -2.0 * (double)c / (double)d);
    const double cs = cos(a), sn = sin(a);
    const double x0 = x[c], x1 = x[c + h];
    x[c] = x0 * cs - x1 * sn;
    x[c + h] = x1 * cs + x0 * sn;
  }
}

/* Position of token p inside the working context of the chunk whose first
 * query sits at t0 ([GUIDE] "Operational Checklist": local relative
 * positional offsets within memory units keep positions in the pretrained
 * range).  Reading: positions by place in the working context -- the
 * initial tokens keep 0 .. n_init-1; the unit in slot m of the selection
 * occupies n_init + m*B + (offset of p in its block); the local tokens from
 * lo = max(n_init, t0 - W + 1) on (the first query's window and every later
 * position of the chunk, queries included) follow at n_init + k_m*B + (p -
 * lo).  Returns -1 for a token in none of these. */
int64_t orc_context_pos(int64_t p, int64_t t0, const int32_t *sel, int32_t k_m, int32_t B,
                        int32_t n_init, int32_t W) {
  const int64_t lo = maxi64(n_init, t0 - W + 1);
  if (p < n_init) return p;
  if (p >= lo) return n_init + (int64_t)k_m * B + (p - lo);
  const int64_t u = p / B - n_init / B;
  for (int32_t m = 0; m < k_m; ++m)
    if (sel[m] >= 0 && (int64_t)sel[m] == u) return n_init + (int64_t)m * B + (p - (p / B) * B);
  return -1;
}

/* Exact softmax attention of queries at positions t0 .. t0+L-1 (rows 0..L-1
 * of each of the G query-head arrays) over their working contexts, with
 * logits q.k/sqrt(d) ([GUIDE] listing: scaled dot-product attention).
 * out [G, L, d]; lse [G, L] = log sum_p exp(q.k_p/sqrt(d)) (may be NULL).
 * rope_theta > 0: q and k hold vectors rotated at their absolute positions
 * (rope_rotate); each is rotated back from its absolute position and then
 * to its working-context position (orc_context_pos) before the product. */
void orc_attend(const void *q, int64_t q_head_stride, int32_t G, int64_t t0,
                int64_t L, const void *k, const void *v, int32_t d, int32_t dt,
                const int32_t *sel, int32_t k_m, int32_t B, int32_t n_init,
                int32_t W, double rope_theta, double *out, double *lse) {
  const double scale = 1.0 / sqrt((double)d);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < L; ++i) {
    int64_t t = t0 + i;
    int64_t n = orc_working_context(t, sel, k_m, B, n_init, W, NULL);
    int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * (n > 0 ? n : 1));
    double *logit = (double *)malloc(sizeof(double) * (n > 0 ? n : 1));
    orc_working_context(t, sel, k_m, B, n_init, W, pos);
    double *qv = (double *)malloc(sizeof(double) * d);
    double *kv = (double *)malloc(sizeof(double) * d);
    for (int32_t g = 0; g < G; ++g) {
      const int64_t qrow = (int64_t)g * q_head_stride + i * d;
      for (int32_t c = 0; c < d; ++c) qv[c] = ld(q, qrow + c, dt);
      if (rope_theta > 0.0) {
        rope_rotate(qv, d, rope_theta, -(double)t);
        rope_rotate(qv, d, rope_theta, (double)orc_context_pos(t, t0, sel, k_m, B, n_init, W));
      }
      double m = -INFINITY;
      for (int64_t a = 0; a < n; ++a) {
        for (int32_t c = 0; c < d; ++c) kv[c] = ld(k, pos[a] * d + c, dt);
        if (rope_theta > 0.0) {
          rope_rotate(kv, d, rope_theta, -(double)pos[a]);
          rope_rotate(kv, d, rope_theta,
                      (double)orc_context_pos(pos[a], t0, sel, k_m, B, n_init, W));
        }
        double dot = 0.0;
        for (int32_t c = 0; c < d; ++c) dot += qv[c] * kv[c];
        logit[a] = dot * scale;
        if (logit[a] > m) m = logit[a];
      }
      double denom = 0.0;
      for (int64_t a = 0; a < n; ++a) denom += exp(logit[a] - m);
      double *o = out + ((int64_t)g * L + i) * d;
      for (int32_t c = 0; c < d; ++c) o[c] = 0.0;
      for (int64_t a = 0; a < n; ++a) {
        double w = exp(logit[a] - m) / denom;
        for (int32_t c = 0; c < d; ++c) o[c] += w * ld(v, pos[a] * d + c, dt);
      }
      if (lse) lse[(int64_t)g * L + i] = m + log(denom);
    }
    free(qv);
    free(kv);
    free(pos);
    free(logit);
  }
}
