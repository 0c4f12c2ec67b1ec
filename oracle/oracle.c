/*
 * oracle.c -- the CPU oracle for fused multi-reduction attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library under reduction_attention_amd/,
 * and it never touches a GPU.
 *
 * What it computes.  Every variant the GPU library offers (split-KV decode,
 * causal prefill, block-sparse prefill) is an exact rewrite of one plain
 * definition: masked softmax attention,
 *
 *     O[i,:] = sum_{j in J(i)} softmax_j( scale * q_i . k_j ) v_j
 *     LSE[i] = ln sum_{j in J(i)} exp( scale * q_i . k_j )
 *
 * where J(i) is the set of keys query i may attend to.  The online softmax
 * with iterative tiling and horizontal fusion of the max and sum reductions
 * (Cleave article on tip.co.jp, section "複数リダクションのスケジューリング";
 * Cleave arXiv abstract), the Split operator that cuts the KV reduction into
 * s partial computations (same article, section "Split演算子によるSplit-Kの
 * 対応"), and STOF's skipping of masked outer tiles (STOF explainer on
 * gist.science, "技術概要", section "1. 統合 MHA モジュール") all reach this
 * same value up to rounding.  So the oracle is the definition itself, in
 * fp64, two passes (max, then sum), with no tiling, no online rescale and no
 * reordering.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - GQA: query head h reads KV head floor(h / G), G = Hq / Hkv.
 *   - Causal alignment when n_q != n_kv: bottom-right, j <= i + n_kv - n_q.
 *   - A dense mask entry of 1 means "attend" (STOF's "valid element").
 *   - A query with no valid key gets O = 0 and LSE = -inf.
 *   - LSE is in natural-log units of the scaled scores.
 *   - Split ranges: c = ceil(max_kv_len / s); request b uses ceil(n_b / c)
 *     non-empty chunks of c keys; the merge of partials is the
 *     log-sum-exp-weighted average (the only exact recombination).
 *   - Flat split ranges (the Split operator applied to the packed key
 *     array as one reduction dimension): P pieces of c = ceil(total_kv / P)
 *     consecutive key rows; split i of request b is its intersection with
 *     the i-th piece it touches.
 *
 * Inputs arrive as raw element arrays of type f64, f32, bf16 or f16 and are
 * widened to double exactly, element by element.  Every accumulation is in
 * double.  OpenMP parallelises over independent (query row, head) pairs only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F64 = 0, OR_F32 = 1, OR_BF16 = 2, OR_F16 = 3 };
enum { OR_MASK_NONE = 0, OR_MASK_CAUSAL = 1, OR_MASK_DENSE = 2 };

/* ---- exact widening of stored elements to double ------------------------ */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double f16_bits_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double mag;
  if (e == 0)
    mag = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
  else if (e == 31)
    mag = f ? NAN : INFINITY;
  else
    mag = ldexp((double)(f + 1024), e - 25); /* (1 + f/1024) * 2^(e-15) */
  return sign ? -mag : mag;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float x;
  memcpy(&x, &u, sizeof x);
  return (double)x;
}

/* The two functions above evaluated once for all 65536 bit patterns, so
 * that a 16-bit element is widened by a lookup: the same exact values,
 * memoized.  Filled before any parallel region (widen_tables_init). */
static double g_widen_f16[65536], g_widen_bf16[65536];
static int g_widen_ready = 0;

static void widen_tables_init(void) {
  if (g_widen_ready) return;
  for (uint32_t b = 0; b < 65536u; ++b) {
    g_widen_f16[b] = f16_bits_to_double((uint16_t)b);
    g_widen_bf16[b] = bf16_bits_to_double((uint16_t)b);
  }
  g_widen_ready = 1;
}

static double load_elem(const void* base, int dtype, int64_t idx) {
  switch (dtype) {
    case OR_F64: return ((const double*)base)[idx];
    case OR_F32: return (double)((const float*)base)[idx];
    case OR_BF16: return g_widen_bf16[((const uint16_t*)base)[idx]];
    case OR_F16: return g_widen_f16[((const uint16_t*)base)[idx]];
  }
  return NAN;
}

const char* oracle_version(void) { return "oracle fp64 two-pass v1"; }

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---- the definition ---------------------------------------------------- */

/* Is key j (0-based within its request) valid for query i of the same
 * request?  n_q, n_kv are that request's lengths. */
static int key_valid(int mask_kind, const uint8_t* mask, int64_t mask_ld,
                     int64_t i, int64_t j, int64_t n_q, int64_t n_kv) {
  if (mask_kind == OR_MASK_NONE) return 1;
  if (mask_kind == OR_MASK_CAUSAL) return j <= i + (n_kv - n_q);
  return mask[i * mask_ld + j] != 0;
}

/* One (query row, head): two passes over the valid keys in fp64.  Queries
 * and keys have D elements per head, values Dv (Dv = D for ordinary
 * attention; MLA's absorbed form scores over the latent plus the decoupled
 * rotary dims and averages the latent part only).
 * scores[] is caller scratch of at least n_kv doubles, q_row[] of D doubles
 * (the query row, widened once). */
static void attend_row(const void* q, const void* k, const void* v, int dtype,
                       int64_t tq, int h, int64_t kv0, int64_t n_q, int64_t n_kv,
                       int64_t i_local, int Hq, int Hkv, int D, int Dv, double scale,
                       int mask_kind, const uint8_t* mask, int64_t mask_ld,
                       double* scores, double* q_row, double* o_row, double* lse_out) {
  const int G = Hq / Hkv;
  const int g = h / G; /* contiguous head groups */
  const int64_t q_off = (tq * Hq + h) * (int64_t)D;
  for (int d = 0; d < D; ++d) q_row[d] = load_elem(q, dtype, q_off + d);
  double m = -INFINITY;
  int64_t count = 0;
  for (int64_t j = 0; j < n_kv; ++j) {
    if (!key_valid(mask_kind, mask, mask_ld, i_local, j, n_q, n_kv)) {
      scores[j] = -INFINITY; /* never read below: skipped by the same test */
      continue;
    }
    const int64_t k_off = ((kv0 + j) * Hkv + g) * (int64_t)D;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += q_row[d] * load_elem(k, dtype, k_off + d);
    scores[j] = scale * dot;
    if (scores[j] > m) m = scores[j];
    ++count;
  }
  for (int d = 0; d < Dv; ++d) o_row[d] = 0.0;
  if (count == 0) { /* no valid key: O = 0, LSE = -inf */
    *lse_out = -INFINITY;
    return;
  }
  double l = 0.0;
  for (int64_t j = 0; j < n_kv; ++j) {
    if (!key_valid(mask_kind, mask, mask_ld, i_local, j, n_q, n_kv)) continue;
    const double p = exp(scores[j] - m);
    l += p;
    const int64_t v_off = ((kv0 + j) * Hkv + g) * (int64_t)Dv;
    for (int d = 0; d < Dv; ++d) o_row[d] += p * load_elem(v, dtype, v_off + d);
  }
  for (int d = 0; d < Dv; ++d) o_row[d] /= l;
  *lse_out = m + log(l);
}

/* Find the request b that owns packed query token tq (qo_indptr ascending). */
static int owner_of(const int64_t* indptr, int B, int64_t t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (indptr[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

/*
 * Masked attention over a ragged batch.
 *   q, o : [total_q, Hq, D]; k, v : [total_kv, Hkv, D]; lse : [total_q, Hq]
 *   request b owns query tokens [qo_indptr[b], qo_indptr[b+1]) and keys
 *   [kv_indptr[b], kv_indptr[b+1]).
 *   mask_kind: 0 none, 1 causal (bottom-right), 2 dense mask shared by every
 *   request and head, row i / column j at mask[i * mask_ld + j].
 *   rows, nrows: optional list of (packed query token, head) pairs; when
 *   rows is NULL every pair is computed.  With a list, o holds nrows*D values
 *   and lse nrows values, in list order.
 * Returns 0, or -1 on bad arguments.
 */
int oracle_attention_dv(const void* q, const void* k, const void* v, int dtype,
                        const int64_t* qo_indptr, const int64_t* kv_indptr, int B,
                        int Hq, int Hkv, int D, int Dv, double scale, int mask_kind,
                        const uint8_t* mask, int64_t mask_ld,
                        const int64_t* rows, int64_t nrows, double* o, double* lse,
                        int nthreads) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Dv <= 0 || Hq % Hkv) return -1;
  if (mask_kind == OR_MASK_DENSE && !mask) return -1;
  int64_t max_kv = 0;
  for (int b = 0; b < B; ++b) {
    int64_t n = kv_indptr[b + 1] - kv_indptr[b];
    if (n > max_kv) max_kv = n;
  }
  const int64_t total_q = qo_indptr[B];
  const int64_t npairs = rows ? nrows : total_q * Hq;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int err = 0;
  widen_tables_init();
#pragma omp parallel
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)((max_kv > 0 ? max_kv : 1) + D));
    if (!scores) {
#pragma omp atomic write
      err = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t p = 0; p < npairs; ++p) {
        const int64_t tq = rows ? rows[2 * p] : p / Hq;
        const int h = rows ? (int)rows[2 * p + 1] : (int)(p % Hq);
        const int b = owner_of(qo_indptr, B, tq);
        const int64_t n_q = qo_indptr[b + 1] - qo_indptr[b];
        const int64_t n_kv = kv_indptr[b + 1] - kv_indptr[b];
        const int64_t out = rows ? p : tq * Hq + h;
        attend_row(q, k, v, dtype, tq, h, kv_indptr[b], n_q, n_kv,
                   tq - qo_indptr[b], Hq, Hkv, D, Dv, scale, mask_kind, mask,
                   mask_ld, scores, scores + (max_kv > 0 ? max_kv : 1), o + out * Dv,
                   lse + out);
      }
      free(scores);
    }
  }
  return err ? -1 : 0;
}

/* Ordinary attention: values have the keys' head dim. */
int oracle_attention(const void* q, const void* k, const void* v, int dtype,
                     const int64_t* qo_indptr, const int64_t* kv_indptr, int B,
                     int Hq, int Hkv, int D, double scale, int mask_kind,
                     const uint8_t* mask, int64_t mask_ld,
                     const int64_t* rows, int64_t nrows, double* o, double* lse,
                     int nthreads) {
  return oracle_attention_dv(q, k, v, dtype, qo_indptr, kv_indptr, B, Hq, Hkv, D, D, scale,
                             mask_kind, mask, mask_ld, rows, nrows, o, lse, nthreads);
}

/* ---- the Split operator: split ranges, partials and their merge -------- */

/* Chunk length c = ceil(max_kv_len / s). */
int64_t oracle_chunk_len(int64_t max_kv_len, int s) {
  if (s <= 0) return -1;
  return max_kv_len > 0 ? (max_kv_len + s - 1) / s : 0;
}

/* ranges[(b*s + i)*2 + {0,1}] = [begin, end) of split i of request b, as key
 * offsets within the request; -1, -1 for splits the request does not use. */
int oracle_split_ranges(const int64_t* kv_indptr, int B, int64_t max_kv_len,
                        int s, int64_t* ranges) {
  const int64_t c = oracle_chunk_len(max_kv_len, s);
  if (c < 0) return -1;
  for (int b = 0; b < B; ++b) {
    const int64_t n = kv_indptr[b + 1] - kv_indptr[b];
    if (n > max_kv_len) return -1;
    for (int i = 0; i < s; ++i) {
      int64_t* r = ranges + ((int64_t)b * s + i) * 2;
      const int64_t lo = (int64_t)i * c;
      if (c > 0 && lo < n) {
        r[0] = lo;
        r[1] = lo + c < n ? lo + c : n;
      } else {
        r[0] = -1;
        r[1] = -1;
      }
    }
  }
  return 0;
}

/* Flat split plan.  The packed key rows [0, total_kv) are cut into P
 * pieces of c = ceil(total_kv / P) rows, piece p = [p*c, (p+1)*c).  Request
 * b (rows [kv_indptr[b], kv_indptr[b+1])) is split where the piece
 * boundaries fall inside it: its split i is the request's intersection
 * with the i-th piece it overlaps, written as key offsets within the
 * request.  Empty requests have no split. */
int64_t oracle_flat_piece_len(int64_t total_kv, int P) {
  if (P <= 0 || total_kv < 0) return -1;
  return total_kv > 0 ? (total_kv + P - 1) / P : 0;
}

/* Most splits one request of at most max_kv_len keys can have: it overlaps
 * ceil((n - 1) / c) + 1 pieces at worst, and never more than P. */
int oracle_flat_max_splits(int64_t total_kv, int64_t max_kv_len, int P) {
  const int64_t c = oracle_flat_piece_len(total_kv, P);
  if (c < 0) return -1;
  if (c == 0 || max_kv_len <= 0) return 1;
  int64_t s = (max_kv_len - 1 + c - 1) / c + 1;
  return (int)(s < P ? s : P);
}

/* ranges[(b*s + i)*2 + {0,1}] as in oracle_split_ranges, for the flat plan
 * with s slots per request (fails if a request needs more). */
int oracle_flat_ranges(const int64_t* kv_indptr, int B, int64_t total_kv, int P, int s,
                       int64_t* ranges) {
  const int64_t c = oracle_flat_piece_len(total_kv, P);
  if (c < 0 || s <= 0) return -1;
  for (int64_t e = 0; e < (int64_t)B * s * 2; ++e) ranges[e] = -1;
  for (int b = 0; b < B; ++b) {
    const int64_t r0 = kv_indptr[b], r1 = kv_indptr[b + 1];
    if (r1 < r0 || r0 < 0 || r1 > total_kv) return -1;
    int i = 0;
    for (int64_t pos = r0; pos < r1; ++i) {
      const int64_t piece_end = (pos / c + 1) * c;  /* end of the piece holding pos */
      const int64_t end = piece_end < r1 ? piece_end : r1;
      if (i >= s) return -1;
      ranges[((int64_t)b * s + i) * 2] = pos - r0;
      ranges[((int64_t)b * s + i) * 2 + 1] = end - r0;
      pos = end;
    }
  }
  return 0;
}

/*
 * Merge s partial results of one row.  Partial i is a normalised attention
 * output o_i over its key subset with max score m_i and sum
 * l_i = sum exp(score - m_i).  Unused partials carry m = -inf, l = 0.
 *   M = max_i m_i;  w_i = l_i exp(m_i - M);  O = sum w_i o_i / sum w_i;
 *   LSE = M + ln sum w_i.   No partial with l > 0: O = 0, LSE = -inf.
 * o_part: [s, rows, D]; m_part, l_part: [s, rows]; o: [rows, D]; lse: [rows].
 */
int oracle_merge(const double* o_part, const double* m_part, const double* l_part,
                 int s, int64_t rows, int D, double* o, double* lse) {
  if (s <= 0 || rows < 0 || D <= 0) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double M = -INFINITY;
    for (int i = 0; i < s; ++i)
      if (l_part[(int64_t)i * rows + r] > 0.0 && m_part[(int64_t)i * rows + r] > M)
        M = m_part[(int64_t)i * rows + r];
    for (int d = 0; d < D; ++d) o[r * D + d] = 0.0;
    if (M == -INFINITY) {
      lse[r] = -INFINITY;
      continue;
    }
    double wsum = 0.0;
    for (int i = 0; i < s; ++i) {
      const double li = l_part[(int64_t)i * rows + r];
      if (!(li > 0.0)) continue;
      const double w = li * exp(m_part[(int64_t)i * rows + r] - M);
      wsum += w;
      const double* oi = o_part + ((int64_t)i * rows + r) * D;
      for (int d = 0; d < D; ++d) o[r * D + d] += w * oi[d];
    }
    for (int d = 0; d < D; ++d) o[r * D + d] /= wsum;
    lse[r] = M + log(wsum);
  }
  return 0;
}

/*
 * Split-KV decode by the definition of the Split operator: one query token
 * per request (q: [B, Hq, D]), keys cut into the ranges of
 * oracle_split_ranges, each range attended on its own in fp64 (two-pass),
 * then merged with oracle_merge.
 * Outputs: o [B, Hq, D], lse [B, Hq], and the partials
 * o_part [s, B*Hq, D], m_part / l_part [s, B*Hq] (any may be NULL except o
 * and lse).
 */
int oracle_split_decode_ranges(const void* q, const void* k, const void* v, int dtype,
                               const int64_t* kv_indptr, int B, int Hq, int Hkv, int D,
                               int64_t max_kv_len, double scale, int s,
                               const int64_t* ranges_in, double* o, double* lse,
                               double* o_part_out, double* m_part_out, double* l_part_out,
                               int nthreads);

int oracle_split_decode(const void* q, const void* k, const void* v, int dtype,
                        const int64_t* kv_indptr, int B, int Hq, int Hkv, int D,
                        int64_t max_kv_len, double scale, int s, double* o,
                        double* lse, double* o_part_out, double* m_part_out,
                        double* l_part_out, int nthreads) {
  if (B <= 0 || s <= 0) return -1;
  int64_t* ranges = (int64_t*)malloc(sizeof(int64_t) * 2 * (size_t)B * s);
  int rc = -1;
  if (ranges && !oracle_split_ranges(kv_indptr, B, max_kv_len, s, ranges))
    rc = oracle_split_decode_ranges(q, k, v, dtype, kv_indptr, B, Hq, Hkv, D, max_kv_len, scale,
                                    s, ranges, o, lse, o_part_out, m_part_out, l_part_out,
                                    nthreads);
  free(ranges);
  return rc;
}

/* The same with the split ranges given ([B, s, 2] key offsets within each
 * request, -1 for unused slots; any plan, e.g. oracle_flat_ranges). */
int oracle_split_decode_ranges(const void* q, const void* k, const void* v, int dtype,
                               const int64_t* kv_indptr, int B, int Hq, int Hkv, int D,
                               int64_t max_kv_len, double scale, int s,
                               const int64_t* ranges_in, double* o, double* lse,
                               double* o_part_out, double* m_part_out, double* l_part_out,
                               int nthreads) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv || s <= 0) return -1;
  const int64_t rows = (int64_t)B * Hq;
  const int64_t* ranges = ranges_in;
  double* o_part = (double*)calloc((size_t)(s * rows * D), sizeof(double));
  double* m_part = (double*)malloc(sizeof(double) * (size_t)(s * rows));
  double* l_part = (double*)calloc((size_t)(s * rows), sizeof(double));
  int rc = -1;
  if (!o_part || !m_part || !l_part) goto done;
  for (int64_t e = 0; e < (int64_t)B * s; ++e)
    if (ranges[2 * e] >= 0 && (ranges[2 * e + 1] - ranges[2 * e] > max_kv_len)) goto done;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  widen_tables_init();
#pragma omp parallel
  {
    const int64_t nsc = max_kv_len > 0 ? max_kv_len : 1;
    double* scores = (double*)malloc(sizeof(double) * (size_t)(nsc + D));
#pragma omp for collapse(2) schedule(dynamic, 4)
    for (int64_t r = 0; r < rows; ++r)
      for (int i = 0; i < s; ++i) {
        const int b = (int)(r / Hq), h = (int)(r % Hq);
        const int64_t* rg = ranges + ((int64_t)b * s + i) * 2;
        double* op = o_part + ((int64_t)i * rows + r) * D;
        m_part[(int64_t)i * rows + r] = -INFINITY;
        l_part[(int64_t)i * rows + r] = 0.0;
        if (rg[0] < 0 || !scores) continue;
        /* The range is a request of its own: one query (index 0, n_q = 1),
         * keys [kv_indptr[b] + lo, kv_indptr[b] + hi), no mask. */
        double lse_i;
        attend_row(q, k, v, dtype, b, h, kv_indptr[b] + rg[0], 1, rg[1] - rg[0], 0,
                   Hq, Hkv, D, D, scale, OR_MASK_NONE, NULL, 0, scores, scores + nsc, op,
                   &lse_i);
        /* Recover (m, l) of the partial from its own scores: the two-pass
         * max and sum of exp(score - max). */
        double m = -INFINITY;
        for (int64_t j = 0; j < rg[1] - rg[0]; ++j)
          if (scores[j] > m) m = scores[j];
        double l = 0.0;
        for (int64_t j = 0; j < rg[1] - rg[0]; ++j) l += exp(scores[j] - m);
        m_part[(int64_t)i * rows + r] = m;
        l_part[(int64_t)i * rows + r] = l;
      }
    free(scores);
  }
  rc = oracle_merge(o_part, m_part, l_part, s, rows, D, o, lse);
  if (o_part_out) memcpy(o_part_out, o_part, sizeof(double) * (size_t)(s * rows * D));
  if (m_part_out) memcpy(m_part_out, m_part, sizeof(double) * (size_t)(s * rows));
  if (l_part_out) memcpy(l_part_out, l_part, sizeof(double) * (size_t)(s * rows));
done:
  free(o_part);
  free(m_part);
  free(l_part);
  return rc;
}
