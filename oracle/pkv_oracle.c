/*
 * pkv_oracle.c -- plain, slow, fp64 CPU oracle for paged-KV decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes (sources):
 *  - AstrAI commit d565d44 ("csrc/kernels/attn_paged_decode.cu"), commit
 *    notes: queries attend over K/V held in fixed-size physical pages that a
 *    per-sequence page table addresses; GQA head packing with the query-head
 *    count a multiple of the kv-head count; a unified causal_offset (-1 = off,
 *    >= 0 = position of the first query token); an additive mask of shape
 *    [batch, kv_len] (or [batch, q_len, kv_len]); split-KV partial outputs
 *    (o_part, ml_part) merged by a single combine kernel.
 *  - Nothing on the pages writes out the attention formula; the operation is
 *    ordinary scaled-dot-product softmax attention, so the oracle is that
 *    definition in fp64 over the keys each query may see.
 *
 * Readings of points the pages leave open (each listed in the design notes):
 *  - query head h uses kv head g = h / (Hq / Hkv) (consecutive query heads
 *    share a kv head);
 *  - the mask is added after scaling: s = scale * q.k + mask;
 *  - with causal offset c >= 0, query token i sees key j iff j <= c + i
 *    (and j < kv_len);
 *  - a row that sees no finite score (kv_len = 0, everything masked) is 0;
 *  - split partials store o = (sum_j w_j v_j) / l, m = max score (natural
 *    log units) and l = sum_j exp(s_j - m); an empty partial is
 *    (o = 0, m = -inf, l = 0) and carries no weight in the combine.
 *
 * Arithmetic: bf16 inputs widen exactly to double; the fp32 mask and scale
 * widen exactly to double; every sum, exp and division is in double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

typedef struct {
  int B, q_len, Hq, Hkv, D, page_size, num_pages, max_pages_per_seq;
  const uint16_t *q, *k_cache, *v_cache;
  const int32_t *block_table, *kv_lens, *causal_offsets;
  double scale;
  int causal_offset;
  const float *mask;
  int64_t mask_stride_b, mask_stride_q;
} problem_t;

/* Address of element [page, slot, kv_head, 0] of a paged cache
 * ([num_pages, page_size, Hkv, D], row-major). */
static const uint16_t *cache_row(const problem_t *p, const uint16_t *cache,
                                 int b, int j, int g) {
  int page = p->block_table[(int64_t)b * p->max_pages_per_seq + j / p->page_size];
  int slot = j % p->page_size;
  return cache + (((int64_t)page * p->page_size + slot) * p->Hkv + g) * p->D;
}

/* Number of keys query token i of sequence b may see: kv_len, cut at c + i + 1
 * when a causal offset c >= 0 applies. */
static int visible_keys(const problem_t *p, int b, int i) {
  int L = p->kv_lens[b];
  int c = p->causal_offsets ? p->causal_offsets[b] : p->causal_offset;
  if (c >= 0) {
    int64_t lim = (int64_t)c + i + 1;
    if (lim < L) L = (int)lim;
  }
  return L < 0 ? 0 : L;
}

/* One output row (b, i, h) over keys [j_begin, j_end) intersected with the
 * keys the row may see.  Writes o[D] (normalised), *m_out, *l_out.
 * scores is caller scratch of at least j_end - j_begin doubles. */
static void attend_row(const problem_t *p, int b, int i, int h, int j_begin,
                       int j_end, double *scores, double *o, double *m_out,
                       double *l_out) {
  const int D = p->D;
  const int G = p->Hq / p->Hkv;
  const int g = h / G;
  const int vis = visible_keys(p, b, i);
  if (j_begin < 0) j_begin = 0;
  if (j_end > vis) j_end = vis;
  const uint16_t *qrow = p->q + (((int64_t)b * p->q_len + i) * p->Hq + h) * D;

  /* scores s_j = scale * sum_d q_d k_jd (+ mask) */
  double m = -INFINITY;
  for (int j = j_begin; j < j_end; ++j) {
    const uint16_t *krow = cache_row(p, p->k_cache, b, j, g);
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += bf16_to_double(qrow[d]) * bf16_to_double(krow[d]);
    double s = p->scale * dot;
    if (p->mask) s += (double)p->mask[(int64_t)b * p->mask_stride_b + (int64_t)i * p->mask_stride_q + j];
    scores[j - j_begin] = s;
    if (s > m) m = s;
  }
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  if (m == -INFINITY) { /* no visible finite score */
    *m_out = -INFINITY;
    *l_out = 0.0;
    return;
  }
  /* softmax weights relative to the max, then the weighted sum of V rows */
  double l = 0.0;
  for (int j = j_begin; j < j_end; ++j) {
    double s = scores[j - j_begin];
    if (s == -INFINITY) continue;
    double w = exp(s - m);
    l += w;
    const uint16_t *vrow = cache_row(p, p->v_cache, b, j, g);
    for (int d = 0; d < D; ++d) o[d] += w * bf16_to_double(vrow[d]);
  }
  for (int d = 0; d < D; ++d) o[d] /= l;
  *m_out = m;
  *l_out = l;
}

static int max_keys(const problem_t *p) {
  int mx = 0;
  for (int b = 0; b < p->B; ++b)
    if (p->kv_lens[b] > mx) mx = p->kv_lens[b];
  return mx;
}

/* Shared driver: rows (b, i, h) in parallel, keys [j_begin, j_end) per row.
 * out: [B, q_len, Hq, D]; m_out, l_out: [B, q_len, Hq] or NULL. */
static int run_rows(const problem_t *p, int j_begin, int j_end, double *out,
                    double *m_out, double *l_out, int num_threads) {
  const int64_t rows = (int64_t)p->B * p->q_len * p->Hq;
  const int span = max_keys(p) + 1;
  int rc = 0;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#pragma omp parallel
#endif
  {
    double *scores = (double *)malloc(sizeof(double) * (size_t)span);
    if (!scores) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      rc = -1;
    } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
      for (int64_t r = 0; r < rows; ++r) {
        int h = (int)(r % p->Hq);
        int i = (int)((r / p->Hq) % p->q_len);
        int b = (int)(r / ((int64_t)p->Hq * p->q_len));
        double m, l;
        attend_row(p, b, i, h, j_begin, j_end, scores, out + r * p->D, &m, &l);
        if (m_out) m_out[r] = m;
        if (l_out) l_out[r] = l;
      }
      free(scores);
    }
  }
  return rc;
}

static int fill_problem(problem_t *p, int B, int q_len, int Hq, int Hkv, int D,
                        int page_size, int num_pages, int max_pages_per_seq,
                        const uint16_t *q, const uint16_t *k_cache,
                        const uint16_t *v_cache, const int32_t *block_table,
                        const int32_t *kv_lens, float scale, int causal_offset,
                        const int32_t *causal_offsets, const float *mask,
                        int64_t mask_stride_b, int64_t mask_stride_q) {
  if (B < 0 || q_len < 1 || Hq < 1 || Hkv < 1 || D < 1 || page_size < 1 || Hq % Hkv) return -2;
  if (!q || !k_cache || !v_cache || !block_table || !kv_lens) return -1;
  p->B = B; p->q_len = q_len; p->Hq = Hq; p->Hkv = Hkv; p->D = D;
  p->page_size = page_size; p->num_pages = num_pages;
  p->max_pages_per_seq = max_pages_per_seq;
  p->q = q; p->k_cache = k_cache; p->v_cache = v_cache;
  p->block_table = block_table; p->kv_lens = kv_lens;
  p->causal_offsets = causal_offsets;
  p->scale = (double)scale;
  p->causal_offset = causal_offset;
  p->mask = mask; p->mask_stride_b = mask_stride_b; p->mask_stride_q = mask_stride_q;
  return 0;
}

/* Full decode: out[B, q_len, Hq, D] in fp64.  Returns 0 on success. */
int pkv_oracle_decode(int B, int q_len, int Hq, int Hkv, int D, int page_size,
                      int num_pages, int max_pages_per_seq, const uint16_t *q,
                      const uint16_t *k_cache, const uint16_t *v_cache,
                      const int32_t *block_table, const int32_t *kv_lens,
                      float scale, int causal_offset,
                      const int32_t *causal_offsets, const float *mask,
                      int64_t mask_stride_b, int64_t mask_stride_q,
                      double *out, int num_threads) {
  problem_t p;
  int rc = fill_problem(&p, B, q_len, Hq, Hkv, D, page_size, num_pages, max_pages_per_seq,
                        q, k_cache, v_cache, block_table, kv_lens, scale, causal_offset,
                        causal_offsets, mask, mask_stride_b, mask_stride_q);
  if (rc) return rc;
  if (!out) return -1;
  return run_rows(&p, 0, 0x7fffffff, out, NULL, NULL, num_threads);
}

/* One split-KV partial: every row restricted to keys [j_begin, j_end).
 * o: [B, q_len, Hq, D] normalised partial outputs; m, l: [B, q_len, Hq]
 * (m in natural-log units of the scaled, masked score). */
int pkv_oracle_partial(int B, int q_len, int Hq, int Hkv, int D, int page_size,
                       int num_pages, int max_pages_per_seq, const uint16_t *q,
                       const uint16_t *k_cache, const uint16_t *v_cache,
                       const int32_t *block_table, const int32_t *kv_lens,
                       float scale, int causal_offset,
                       const int32_t *causal_offsets, const float *mask,
                       int64_t mask_stride_b, int64_t mask_stride_q,
                       int j_begin, int j_end, double *o, double *m, double *l,
                       int num_threads) {
  problem_t p;
  int rc = fill_problem(&p, B, q_len, Hq, Hkv, D, page_size, num_pages, max_pages_per_seq,
                        q, k_cache, v_cache, block_table, kv_lens, scale, causal_offset,
                        causal_offsets, mask, mask_stride_b, mask_stride_q);
  if (rc) return rc;
  if (!o || !m || !l) return -1;
  return run_rows(&p, j_begin, j_end, o, m, l, num_threads);
}

/* Log-sum-exp merge of S partials per row (the split-KV combine):
 *   M = max over partials with l_s > 0 of m_s,
 *   w_s = l_s * exp(m_s - M),
 *   out = sum_s w_s o_s / sum_s w_s   (0 when no partial has weight).
 * o_part: [rows, S, D]; m_part, l_part: [rows, S]; out: [rows, D]. */
int pkv_oracle_combine(int64_t rows, int S, int D, const double *o_part,
                       const double *m_part, const double *l_part, double *out) {
  if (rows < 0 || S < 1 || D < 1) return -2;
  if (!o_part || !m_part || !l_part || !out) return -1;
  for (int64_t r = 0; r < rows; ++r) {
    double M = -INFINITY;
    for (int s = 0; s < S; ++s)
      if (l_part[r * S + s] > 0.0 && m_part[r * S + s] > M) M = m_part[r * S + s];
    double *dst = out + r * D;
    for (int d = 0; d < D; ++d) dst[d] = 0.0;
    if (M == -INFINITY) continue;
    double wsum = 0.0;
    for (int s = 0; s < S; ++s) {
      double ls = l_part[r * S + s];
      if (!(ls > 0.0)) continue;
      double w = ls * exp(m_part[r * S + s] - M);
      wsum += w;
      const double *src = o_part + (r * S + s) * D;
      for (int d = 0; d < D; ++d) dst[d] += w * src[d];
    }
    for (int d = 0; d < D; ++d) dst[d] /= wsum;
  }
  return 0;
}

/* Threads OpenMP will use by default (1 without OpenMP). */
int pkv_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
