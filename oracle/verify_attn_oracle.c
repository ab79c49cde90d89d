/*
 * Oracle for MLA tree-verify attention over a paged latent KV cache.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, fp64 definition that the GPU
 * path is checked against. Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load it. It shares no code, header or constant with the GPU library.
 *
 * What it computes (sources, by page title and section):
 *  - Absorbed multi-head latent attention: one 512-wide latent row kv_c per token is shared
 *    by every head, the query is already in latent space, q is [num_tok, H, 576] and the
 *    paged cache is [num_slots, 576] ("The Glue That Binds: Wiring a Custom CUDA Kernel into
 *    Production via C-ABI", section "The Broader Engineering Effort"; "The Glue That
 *    Connects: Wiring a Custom Flash Attention Kernel into the C-ABI Layer", section "The
 *    Context: Building a Blackwell-Specific Verify Attention Kernel").
 *  - Keys are reached through kv_indices, segmented per request by kv_indptr / qo_indptr,
 *    and the mask is read at mask_indptr offsets ("The Final Solder Joint: Updating the
 *    C-ABI Layer for CUDA Graph Capture-Safety", sections "The Investigation" and "The
 *    Three-Edits Sequence").
 *  - Visibility is prefix length plus a tree visibility matrix: every prefix key is seen,
 *    tail keys follow the mask ("The Glue That Makes Kernels Run", section "The Context: A
 *    Custom Kernel in Flight"); a masked score is -inf and the mask is indexed by the global
 *    key position, mask[b][i][j] ("The Glue That Connects", section "Design Decisions and
 *    Trade-Offs", paragraph on mask handling).
 *  - Softmax over the visible keys of an arbitrary-length prefix ("The Glue That Connects",
 *    same section, paragraph on online softmax). The oracle computes it in two passes, the
 *    textbook definition; the streaming form is the GPU's business.
 *  - The score uses all Dl + Dr = 576 dims; the value is the Dl = 512 latent dims (the
 *    scalars Dl and Dr are passed separately in "The Final Solder Joint", section "Why the
 *    C-ABI Edit Matters").
 *
 * Two ways to give the key slots (both from "The Final Solder Joint", section "The
 * Three-Edits Sequence": prefix slots from kv_indices, the new tokens' slots from
 * out_cache_loc, told apart by the kv_indptr offsets):
 *  - out_cache_loc == NULL: request r's L_r keys are kv_indices[kv_indptr[r] .. kv_indptr[r+1]),
 *    the last T_r of them being the tree tokens in query order;
 *  - out_cache_loc != NULL: kv_indices[kv_indptr[r] .. kv_indptr[r+1]) holds the P_r prefix
 *    slots only, and tree key P_r + k is out_cache_loc[qo_indptr[r] + k]; L_r = P_r + T_r.
 *
 * Readings where the pages are silent (also listed in the design notes):
 *  - tree keys are the last T_r key positions of each request, in query order;
 *  - the mask of request r is a [T_r, L_r] row-major byte matrix at mask_indptr[r]; prefix
 *    columns are never read; any nonzero byte means visible;
 *  - exponent base e; lse is the natural log of the softmax denominator plus the max score;
 *  - argmax is the smallest key position j in [0, L_r) that attains the max score;
 *  - an empty visible set gives out = 0, lse = -inf, argmax = -1.
 *
 * Per row (request r, tree token i, head h):
 *   s_j    = scale * sum_{d < Dl+Dr} q[t,h,d] * kv[slot_j, d]      for visible j
 *   m      = max_j s_j
 *   w_j    = exp(s_j - m),   Lambda = sum_j w_j
 *   out[c] = sum_j w_j * kv[slot_j, c] / Lambda                      for c < Dl
 *   lse    = m + log(Lambda)
 * Everything in IEEE double, no fast-math, no contraction.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_FP32 = 1 };
enum { ORACLE_OK = 0, ORACLE_ERR_INVALID = 1, ORACLE_ERR_NOMEM = 2 };

/* One input element as a double. bf16 is the upper half of an IEEE binary32. */
static double elem(const void *base, int dtype, int64_t idx) {
  if (dtype == ORACLE_BF16) {
    uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const float *)base)[idx];
}

/* Number of keys L_r of request r (see the two slot layouts above). */
static int64_t req_keys(const int32_t *kv_indptr, const int64_t *qo_indptr,
                        const int64_t *out_cache_loc, int32_t r) {
  const int64_t n = (int64_t)kv_indptr[r + 1] - (int64_t)kv_indptr[r];
  return out_cache_loc ? n + (qo_indptr[r + 1] - qo_indptr[r]) : n;
}

/* Slot of key position j of request r, whose prefix has P keys. */
static int64_t slot_of(const int64_t *kv_indices, const int32_t *kv_indptr,
                       const int64_t *qo_indptr, const int64_t *out_cache_loc, int32_t r,
                       int64_t P, int64_t j) {
  if (out_cache_loc && j >= P) return out_cache_loc[qo_indptr[r] + (j - P)];
  return kv_indices[kv_indptr[r] + j];
}

/* Checks the segment tables: non-decreasing offsets, P_r >= 0, slots in range. */
static int check_tables(int64_t num_slots, const int64_t *kv_indices,
                        const int32_t *kv_indptr, const int64_t *qo_indptr,
                        const int64_t *out_cache_loc, const int64_t *mask_indptr,
                        int64_t mask_len, int32_t bs) {
  for (int32_t r = 0; r < bs; ++r) {
    int64_t T = qo_indptr[r + 1] - qo_indptr[r];
    int64_t n = (int64_t)kv_indptr[r + 1] - (int64_t)kv_indptr[r];
    int64_t L = req_keys(kv_indptr, qo_indptr, out_cache_loc, r);
    if (T < 0 || n < 0 || L - T < 0) return ORACLE_ERR_INVALID;
    if (mask_indptr[r] < 0 || mask_indptr[r] + T * L > mask_len) return ORACLE_ERR_INVALID;
    for (int64_t j = 0; j < L; ++j) {
      int64_t s = slot_of(kv_indices, kv_indptr, qo_indptr, out_cache_loc, r, L - T, j);
      if (s < 0 || s >= num_slots) return ORACLE_ERR_INVALID;
    }
  }
  return ORACLE_OK;
}

/*
 * Computes the rows listed in `rows` (flat ids t*H + h), or all num_tokens*H rows when
 * rows == NULL. out_cache_loc may be NULL (see the two slot layouts above). Outputs are indexed by position in that list: out [n_rows, Dl],
 * lse [n_rows], argmax [n_rows]. Returns ORACLE_OK, ORACLE_ERR_INVALID or ORACLE_ERR_NOMEM.
 */
int oracle_verify_attn_f64(const void *q, const void *kv_buffer, int32_t in_dtype,
                           int64_t num_slots, const int64_t *kv_indices,
                           const int32_t *kv_indptr, const int64_t *qo_indptr,
                           const int64_t *out_cache_loc, const uint8_t *custom_mask,
                           const int64_t *mask_indptr, int64_t mask_len, int32_t bs,
                           int32_t H, int32_t Dl, int32_t Dr,
                           double scale, const int64_t *rows, int64_t n_rows,
                           double *out, double *lse, int64_t *argmax, int32_t nthreads) {
  if (in_dtype != ORACLE_BF16 && in_dtype != ORACLE_FP32) return ORACLE_ERR_INVALID;
  if (bs < 0 || H < 1 || Dl < 1 || Dr < 0) return ORACLE_ERR_INVALID;
  int rc = check_tables(num_slots, kv_indices, kv_indptr, qo_indptr, out_cache_loc, mask_indptr,
                        mask_len, bs);
  if (rc != ORACLE_OK) return rc;
  const int64_t D = (int64_t)Dl + Dr;
  const int64_t num_tokens = bs > 0 ? qo_indptr[bs] : 0;
  const int64_t total = rows ? n_rows : num_tokens * H;
  int64_t max_l = 0;
  for (int32_t r = 0; r < bs; ++r) {
    int64_t L = req_keys(kv_indptr, qo_indptr, out_cache_loc, r);
    if (L > max_l) max_l = L;
  }
  for (int64_t n = 0; n < total; ++n) {
    int64_t row = rows ? rows[n] : n;
    if (row < 0 || row >= num_tokens * H) return ORACLE_ERR_INVALID;
  }

  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double *s = (double *)malloc(sizeof(double) * (size_t)(max_l > 0 ? max_l : 1));
    unsigned char *vis = (unsigned char *)malloc((size_t)(max_l > 0 ? max_l : 1));
    double *acc = (double *)malloc(sizeof(double) * (size_t)Dl);
    if (!s || !vis || !acc) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      failed = 1;
    } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
      for (int64_t n = 0; n < total; ++n) {
        const int64_t row = rows ? rows[n] : n;
        const int64_t t = row / H;
        const int64_t h = row % H;
        /* the request that owns token t */
        int32_t r = 0;
        while (r + 1 < bs && qo_indptr[r + 1] <= t) ++r;
        const int64_t i = t - qo_indptr[r];
        const int64_t T = qo_indptr[r + 1] - qo_indptr[r];
        const int64_t L = req_keys(kv_indptr, qo_indptr, out_cache_loc, r);
        const int64_t P = L - T;
        const uint8_t *mrow = custom_mask + mask_indptr[r] + i * L;
        const int64_t qbase = (t * H + h) * D;

        /* pass 1: visible set, scores, max */
        double m = -INFINITY;
        int64_t am = -1;
        for (int64_t j = 0; j < L; ++j) {
          vis[j] = (unsigned char)(j < P || mrow[j] != 0);
          if (!vis[j]) continue;
          const int64_t kbase =
              slot_of(kv_indices, kv_indptr, qo_indptr, out_cache_loc, r, P, j) * D;
          double dot = 0.0;
          for (int64_t d = 0; d < D; ++d)
            dot += elem(q, in_dtype, qbase + d) * elem(kv_buffer, in_dtype, kbase + d);
          s[j] = scale * dot;
          if (s[j] > m) {
            m = s[j];
            am = j;
          }
        }

        /* pass 2: weights, denominator, weighted sum of latent rows */
        double *o = out + n * (int64_t)Dl;
        if (am < 0) {
          for (int32_t c = 0; c < Dl; ++c) o[c] = 0.0;
          lse[n] = -INFINITY;
          argmax[n] = -1;
          continue;
        }
        for (int32_t c = 0; c < Dl; ++c) acc[c] = 0.0;
        double lam = 0.0;
        for (int64_t j = 0; j < L; ++j) {
          if (!vis[j]) continue;
          const double w = exp(s[j] - m);
          lam += w;
          const int64_t kbase =
              slot_of(kv_indices, kv_indptr, qo_indptr, out_cache_loc, r, P, j) * D;
          for (int32_t c = 0; c < Dl; ++c) acc[c] += w * elem(kv_buffer, in_dtype, kbase + c);
        }
        for (int32_t c = 0; c < Dl; ++c) o[c] = acc[c] / lam;
        lse[n] = m + log(lam);
        argmax[n] = am;
      }
    }
    free(s);
    free(vis);
    free(acc);
  }
  return failed ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/*
 * Score diagnostics for checking an argmax computed in lower precision (same inputs, same
 * tables, same visibility rule and score definition as oracle_verify_attn_f64).
 *
 * For each listed row (flat id t*H + h; every row when rows == NULL):
 *   top1[n]   = m1 = the largest visible score s_j (-inf when no key is visible)
 *   arg1[n]   = the smallest visible key position attaining m1 (-1 when none)
 *   top2[n]   = the largest visible score among keys j != arg1[n] (-inf when none); it equals
 *               m1 when the maximum is attained twice
 *   absmax[n] = the largest visible |scale| * sum_d |q[t,h,d] * kv[slot_j,d]|, the magnitude
 *               that bounds the rounding error of any summation order of s_j
 * For each (row, key position) pair listed in pair_rows / pair_keys:
 *   pair_s[p]   = s_j, and pair_abs[p] = |scale| * sum_d |q[t,h,d] kv[slot_j,d]|
 *   pair_vis[p] = 1 if key j is visible to the row, else 0 (key positions outside [0, L_r)
 *                 report 0 and NaN scores).
 * Returns ORACLE_OK or ORACLE_ERR_INVALID / ORACLE_ERR_NOMEM.
 */
static void row_owner(const int64_t *qo_indptr, int32_t bs, int64_t t, int32_t *r) {
  int32_t k = 0;
  while (k + 1 < bs && qo_indptr[k + 1] <= t) ++k;
  *r = k;
}

/* s_j and its magnitude bound for one (token t, head h, request r, key j). */
static void key_score(const void *q, const void *kv_buffer, int32_t in_dtype,
                      const int64_t *kv_indices, const int32_t *kv_indptr,
                      const int64_t *qo_indptr, const int64_t *out_cache_loc, int32_t r,
                      int64_t P, int64_t t, int64_t h, int32_t H, int64_t D, double scale,
                      int64_t j, double *s, double *sabs) {
  const int64_t qrow = (t * H + h) * D;
  const int64_t krow = slot_of(kv_indices, kv_indptr, qo_indptr, out_cache_loc, r, P, j) * D;
  double dot = 0.0, mag = 0.0;
  for (int64_t e = 0; e < D; e++) {
    const double p = elem(q, in_dtype, qrow + e) * elem(kv_buffer, in_dtype, krow + e);
    dot += p;
    mag += fabs(p);
  }
  *s = scale * dot;
  *sabs = fabs(scale) * mag;
}

int oracle_score_top2_f64(const void *q, const void *kv_buffer, int32_t in_dtype,
                          int64_t num_slots, const int64_t *kv_indices,
                          const int32_t *kv_indptr, const int64_t *qo_indptr,
                          const int64_t *out_cache_loc, const uint8_t *custom_mask,
                          const int64_t *mask_indptr, int64_t mask_len, int32_t bs, int32_t H,
                          int32_t Dl, int32_t Dr, double scale, const int64_t *rows,
                          int64_t n_rows, double *top1, int64_t *arg1, double *top2,
                          double *absmax, const int64_t *pair_rows, const int64_t *pair_keys,
                          int64_t n_pairs, double *pair_s, double *pair_abs, int32_t *pair_vis,
                          int32_t nthreads) {
  if (in_dtype != ORACLE_BF16 && in_dtype != ORACLE_FP32) return ORACLE_ERR_INVALID;
  if (bs < 0 || H < 1 || Dl < 1 || Dr < 0 || n_pairs < 0) return ORACLE_ERR_INVALID;
  int rc = check_tables(num_slots, kv_indices, kv_indptr, qo_indptr, out_cache_loc, mask_indptr,
                        mask_len, bs);
  if (rc != ORACLE_OK) return rc;
  const int64_t D = (int64_t)Dl + Dr;
  const int64_t num_tokens = bs > 0 ? qo_indptr[bs] : 0;
  const int64_t total = rows ? n_rows : num_tokens * H;
  for (int64_t n = 0; n < total; ++n) {
    const int64_t row = rows ? rows[n] : n;
    if (row < 0 || row >= num_tokens * H) return ORACLE_ERR_INVALID;
  }
  for (int64_t p = 0; p < n_pairs; ++p)
    if (pair_rows[p] < 0 || pair_rows[p] >= num_tokens * H) return ORACLE_ERR_INVALID;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t n = 0; n < total; ++n) {
    const int64_t row = rows ? rows[n] : n;
    const int64_t t = row / H, h = row % H;
    int32_t r;
    row_owner(qo_indptr, bs, t, &r);
    const int64_t i = t - qo_indptr[r];
    const int64_t T = qo_indptr[r + 1] - qo_indptr[r];
    const int64_t L = req_keys(kv_indptr, qo_indptr, out_cache_loc, r);
    const int64_t P = L - T;
    const uint8_t *mrow = custom_mask + mask_indptr[r] + i * L;
    double m1 = -INFINITY, m2 = -INFINITY, amag = 0.0;
    int64_t j1 = -1;
    for (int64_t j = 0; j < L; ++j) {
      if (!(j < P || mrow[j] != 0)) continue;
      double s, sabs;
      key_score(q, kv_buffer, in_dtype, kv_indices, kv_indptr, qo_indptr, out_cache_loc, r, P,
                t, h, H, D, scale, j, &s, &sabs);
      if (sabs > amag) amag = sabs;
      if (s > m1) {
        m2 = m1;
        m1 = s;
        j1 = j;
      } else if (s > m2) {
        m2 = s;
      }
    }
    top1[n] = m1;
    arg1[n] = j1;
    top2[n] = m2;
    absmax[n] = amag;
  }
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 16)
#endif
  for (int64_t p = 0; p < n_pairs; ++p) {
    const int64_t t = pair_rows[p] / H, h = pair_rows[p] % H;
    int32_t r;
    row_owner(qo_indptr, bs, t, &r);
    const int64_t i = t - qo_indptr[r];
    const int64_t T = qo_indptr[r + 1] - qo_indptr[r];
    const int64_t L = req_keys(kv_indptr, qo_indptr, out_cache_loc, r);
    const int64_t P = L - T;
    const int64_t j = pair_keys[p];
    if (j < 0 || j >= L) {
      pair_s[p] = NAN;
      pair_abs[p] = NAN;
      pair_vis[p] = 0;
      continue;
    }
    const uint8_t *mrow = custom_mask + mask_indptr[r] + i * L;
    pair_vis[p] = (j < P || mrow[j] != 0) ? 1 : 0;
    key_score(q, kv_buffer, in_dtype, kv_indices, kv_indptr, qo_indptr, out_cache_loc, r, P, t,
              h, H, D, scale, j, &pair_s[p], &pair_abs[p]);
  }
  return ORACLE_OK;
}
