/*
 * sas_oracle.c -- plain fp64 CPU oracle for SAS gated block-sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY: used by the test-suite, the smoke check and the
 * benchmark's CPU baseline; never by the product library.  It shares no code
 * with the HIP kernels.  Every function follows the definition directly:
 * per query row, two-pass softmax, no tiling, no online rescaling.  Loops run
 * in parallel over independent rows / keys with OpenMP, which changes no
 * arithmetic.
 *
 * Sources (page title, part of the page):
 *  [A] "SAS: Simple Attention Sparsification via End-to-End Optimization of
 *      Context Ranking", NeurIPS 2026 poster page, abstract: the selector's
 *      continuous scores are injected into the attention logits; the gate sits
 *      inside the attention softmax in log form; all context units stay active
 *      in training; the budget is the number of attended units per query; a
 *      hard Top-K picks the units at inference.
 *  [B] same paper, Hugging Face papers page, abstract: normalised softmax
 *      gates calibrate the historical context against the always-retained
 *      current block.
 *  [C] "SAS Learns Token Importance for Sparse Attention" (blog),
 *      "The Logit Injection Mechanism": the selector output is added to the
 *      logit before the softmax, so gradients reach the selector through it.
 * Readings where the pages are silent (score function, scales, causal mask
 * inside the current block, tie order of Top-K, bias in sparse mode) are
 * stated at the function that takes them.
 */
#include "sas_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static int64_t nblocks(const oracle_shape* s) { return (s->tk + s->block - 1) / s->block; }

static int check_shape(const oracle_shape* s) {
  if (!s) return -1;
  if (s->batch < 1 || s->hq < 1 || s->hkv < 1 || s->hks < 1 || s->tq < 1 || s->tk < 1 ||
      s->d < 1 || s->ds < 1 || s->block < 1)
    return -1;
  if (s->tq > s->tk) return -1;
  if (s->hq % s->hkv || s->hq % s->hks) return -1;
  return 0;
}

/* Where query row r = (b*hq + h)*tq + i sits. */
typedef struct {
  int64_t b, h, i, t, c, g, sh;
} rowinfo;

static rowinfo row_info(const oracle_shape* s, int64_t r) {
  rowinfo x;
  x.i = r % s->tq;
  int64_t bh = r / s->tq;
  x.h = bh % s->hq;
  x.b = bh / s->hq;
  x.t = (int64_t)(s->tk - s->tq) + x.i; /* absolute position of the query */
  x.c = x.t / s->block;                 /* its (current) block           */
  x.g = x.h * s->hkv / s->hq;           /* kv head                        */
  x.sh = x.h * s->hks / s->hq;          /* selector-key head              */
  return x;
}

static double dot(const double* a, const double* b, int64_t n) {
  double acc = 0.0;
  for (int64_t e = 0; e < n; ++e) acc += a[e] * b[e];
  return acc;
}

/* Step 1 -- selector score of query row x against historical block j:
 * z = sigma * <qs_t, ks_j>.  The pages only say the selector emits a
 * continuous score per context unit ([A], [C]); the bilinear form and the
 * 1/sqrt(ds) scale are this library's reading.  With scores-in (zin) the
 * score is taken as given. */
static double score(const oracle_shape* s, const double* qs, const double* ks, const double* zin,
                    const rowinfo* x, int64_t j) {
  const int64_t nb = nblocks(s);
  const int64_t r = (x->b * s->hq + x->h) * s->tq + x->i;
  if (zin) return zin[r * nb + j];
  const double* a = qs + r * s->ds;
  const double* kk = ks + ((x->b * s->hks + x->sh) * nb + j) * s->ds;
  return s->sel_scale * dot(a, kk, s->ds);
}

/* Step 2 -- log of the softmax normaliser over the historical blocks:
 * lambda = log sum_{j<c} exp(z_j), computed as m + log sum exp(z_j - m).
 * With no history (c = 0) the sum is empty and lambda = -inf ([B]: the gate
 * is a softmax over historical context only). */
static double log_sum_exp(const double* z, int64_t n) {
  if (n <= 0) return -INFINITY;
  double m = z[0];
  for (int64_t j = 1; j < n; ++j)
    if (z[j] > m) m = z[j];
  if (m == -INFINITY) return -INFINITY;
  double acc = 0.0;
  for (int64_t j = 0; j < n; ++j) acc += exp(z[j] - m);
  return m + log(acc);
}

int oracle_gate_scores(const oracle_shape* s, const double* qs, const double* ks, double* z,
                       double* lam, double* beta) {
  if (check_shape(s)) return -1;
  const int64_t nb = nblocks(s);
  const int64_t nrows = (int64_t)s->batch * s->hq * s->tq;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t r = 0; r < nrows; ++r) {
    rowinfo x = row_info(s, r);
    double* zr = (double*)malloc(sizeof(double) * (size_t)(nb > 0 ? nb : 1));
    for (int64_t j = 0; j < x.c; ++j) zr[j] = score(s, qs, ks, NULL, &x, j);
    const double l = log_sum_exp(zr, x.c);
    if (lam) lam[r] = l;
    for (int64_t j = 0; j < nb; ++j) {
      /* Step 3 -- log-gate: beta_j = log softmax_j(z) = z_j - lambda for
       * j < c; the current block keeps bias 0 ([B]); later blocks are never
       * attended (causal) and carry -inf. */
      if (z) z[r * nb + j] = j < x.c ? zr[j] : -INFINITY;
      if (beta) beta[r * nb + j] = j < x.c ? zr[j] - l : (j == x.c ? 0.0 : -INFINITY);
    }
    free(zr);
  }
  return 0;
}

/* Steps 5-8 -- attention of one query row over an explicit key set: every key
 * of the listed historical blocks sel[0..nsel) with bias add[k] on each of its
 * logits, plus the keys of the current block up to and including the query
 * (token-level causal mask; the pages call the attention causal but do not
 * spell out the mask inside a block).  Logit: tau <q_t, k_u> + bias; the bias
 * is not scaled by tau (log gate added to the logit, [A], [C]).
 * Writes o[d] and returns L = log sum_u exp(logit_u). */
static double attend_row(const oracle_shape* s, const double* q, const double* k,
                         const double* v, const rowinfo* x, int64_t nsel, const int64_t* sel,
                         const double* add, double* o) {
  const int64_t d = s->d, B = s->block;
  const double* qr = q + ((x->b * s->hq + x->h) * s->tq + x->i) * d;
  const double* kb = k + (x->b * s->hkv + x->g) * (int64_t)s->tk * d;
  const double* vb = v + (x->b * s->hkv + x->g) * (int64_t)s->tk * d;
  const int64_t cur0 = x->c * B;
  const int64_t nkeys = nsel * B + (x->t - cur0 + 1);
  int64_t* key = (int64_t*)malloc(sizeof(int64_t) * (size_t)nkeys);
  double* lg = (double*)malloc(sizeof(double) * (size_t)nkeys);
  int64_t n = 0;
  for (int64_t a = 0; a < nsel; ++a)
    for (int64_t u = sel[a] * B; u < sel[a] * B + B; ++u) {
      key[n] = u;
      lg[n++] = s->sm_scale * dot(qr, kb + u * d, d) + add[a];
    }
  for (int64_t u = cur0; u <= x->t; ++u) {
    key[n] = u;
    lg[n++] = s->sm_scale * dot(qr, kb + u * d, d);
  }
  /* Step 7 -- two-pass softmax: M = max, L = M + log sum exp(l - M). */
  double M = -INFINITY;
  for (int64_t a = 0; a < n; ++a)
    if (lg[a] > M) M = lg[a];
  double acc = 0.0;
  for (int64_t a = 0; a < n; ++a) acc += exp(lg[a] - M);
  const double L = M + log(acc);
  /* Step 8 -- O = sum_u P_u v_u with P_u = exp(l_u - L). */
  for (int64_t e = 0; e < d; ++e) o[e] = 0.0;
  for (int64_t a = 0; a < n; ++a) {
    const double p = exp(lg[a] - L);
    const double* vr = vb + key[a] * d;
    for (int64_t e = 0; e < d; ++e) o[e] += p * vr[e];
  }
  free(key);
  free(lg);
  return L;
}

/* Dense-active training: every historical block is attended ([A]: all
 * context units stay active so each receives gradients) with bias
 * beta_j = z_j - lambda; returns lambda through *lam_out. */
static double dense_row(const oracle_shape* s, const double* q, const double* k, const double* v,
                        const double* qs, const double* ks, const double* zin, const rowinfo* x,
                        double* o, double* lam_out) {
  const int64_t c = x->c;
  int64_t* sel = (int64_t*)malloc(sizeof(int64_t) * (size_t)(c > 0 ? c : 1));
  double* z = (double*)malloc(sizeof(double) * (size_t)(c > 0 ? c : 1));
  for (int64_t j = 0; j < c; ++j) {
    sel[j] = j;
    z[j] = score(s, qs, ks, zin, x, j);
  }
  const double lam = log_sum_exp(z, c);
  for (int64_t j = 0; j < c; ++j) z[j] -= lam; /* now beta_j */
  const double L = attend_row(s, q, k, v, x, c, sel, z, o);
  free(sel);
  free(z);
  if (lam_out) *lam_out = lam;
  return L;
}

int oracle_attn_fwd(const oracle_shape* s, const double* q, const double* k, const double* v,
                    const double* qs, const double* ks, const double* zin, int64_t nrows,
                    const int64_t* rows, double* o, double* lse) {
  if (check_shape(s)) return -1;
  const int64_t all = (int64_t)s->batch * s->hq * s->tq;
  if (!rows) nrows = all;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t a = 0; a < nrows; ++a) {
    const int64_t r = rows ? rows[a] : a;
    rowinfo x = row_info(s, r);
    double* orow = (double*)malloc(sizeof(double) * (size_t)s->d);
    const double L = dense_row(s, q, k, v, qs, ks, zin, &x, orow, NULL);
    if (o) memcpy(o + a * s->d, orow, sizeof(double) * (size_t)s->d);
    if (lse) lse[a] = L;
    free(orow);
  }
  return 0;
}

/* ------------------------------------------------------------------------
 * Backward of the dense-active forward (gradients reach the selector through
 * the log gate inside the softmax, [A], [C]).  For one row with P_u, O, dO:
 *   D = <dO, O>,  dP_u = <dO, v_u>,  dS_u = P_u (dP_u - D)
 *   dq = tau sum_u dS_u k_u;  dk_u += tau dS_u q;  dv_u += P_u dO
 *   dbeta_j = sum_{u in block j} dS_u  (j < c)
 *   g_j = exp(z_j - lambda);  dz_j = dbeta_j - g_j sum_{j'<c} dbeta_{j'}
 *   dqs = sigma sum_j dz_j ks_j;  dks_j += sigma dz_j qs
 * The per-row statistics (lambda, L, D, sum dbeta) are computed once per row
 * and every pairwise term is recomputed from them where it is needed.
 * ---------------------------------------------------------------------- */
typedef struct {
  double lam, L, D, sdb;
} rowstat;

/* logit of row x at key u; bias by block (0 for the current block). */
static double logit_at(const oracle_shape* s, const double* q, const double* k, const double* qs,
                       const double* ks, const double* zin, const rowinfo* x, const rowstat* st,
                       int64_t u) {
  const int64_t d = s->d;
  const double* qr = q + ((x->b * s->hq + x->h) * s->tq + x->i) * d;
  const double* ku = k + ((x->b * s->hkv + x->g) * (int64_t)s->tk + u) * d;
  const int64_t j = u / s->block;
  const double bias = j == x->c ? 0.0 : score(s, qs, ks, zin, x, j) - st->lam;
  return s->sm_scale * dot(qr, ku, d) + bias;
}

/* dS_{t,u} = P (dP - D) and P for row x at key u. */
static double dS_at(const oracle_shape* s, const double* q, const double* k, const double* v,
                    const double* dout, const double* qs, const double* ks, const double* zin,
                    const rowinfo* x, const rowstat* st, int64_t u, double* p_out) {
  const int64_t d = s->d;
  const double p = exp(logit_at(s, q, k, qs, ks, zin, x, st, u) - st->L);
  const double* dor = dout + ((x->b * s->hq + x->h) * s->tq + x->i) * d;
  const double* vu = v + ((x->b * s->hkv + x->g) * (int64_t)s->tk + u) * d;
  if (p_out) *p_out = p;
  return p * (dot(dor, vu, d) - st->D);
}

int oracle_attn_bwd(const oracle_shape* s, const double* q, const double* k, const double* v,
                    const double* dout, const double* qs, const double* ks, const double* zin,
                    int64_t nrows, const int64_t* rows, double* dq, double* dz, double* dqs,
                    int64_t nkeys, const int64_t* keys, double* dk, double* dv, int64_t nsblk,
                    const int64_t* sblk, double* dks) {
  if (check_shape(s)) return -1;
  const int64_t d = s->d, B = s->block, nb = nblocks(s), ds = s->ds;
  const int64_t all_rows = (int64_t)s->batch * s->hq * s->tq;
  const int64_t all_keys = (int64_t)s->batch * s->hkv * s->tk;
  const int64_t all_sblk = (int64_t)s->batch * s->hks * nb;
  const int64_t qoff = s->tk - s->tq;
  if (nrows < 0) nrows = all_rows;
  if (nkeys < 0) nkeys = all_keys;
  if (nsblk < 0) nsblk = all_sblk;
  if (zin) nsblk = 0; /* no selector vectors to differentiate */

  /* need1: rows whose statistics (lambda, L, D) are needed;
   * need2: rows whose sum dbeta is needed too. */
  unsigned char* need = (unsigned char*)calloc((size_t)all_rows, 1);
  for (int64_t a = 0; a < nrows; ++a) need[rows ? rows[a] : a] = 2;
  for (int64_t a = 0; a < nkeys; ++a) {
    const int64_t key = keys ? keys[a] : a;
    const int64_t u = key % s->tk, bg = key / s->tk, g = bg % s->hkv, b = bg / s->hkv;
    const int64_t per = s->hq / s->hkv;
    for (int64_t h = g * per; h < (g + 1) * per; ++h)
      for (int64_t i = 0; i < s->tq; ++i)
        if (qoff + i >= u) {
          unsigned char* f = &need[(b * s->hq + h) * s->tq + i];
          if (*f < 1) *f = 1;
        }
  }
  for (int64_t a = 0; a < nsblk; ++a) {
    const int64_t sb = sblk ? sblk[a] : a;
    const int64_t j = sb % nb, bs = sb / nb, sh = bs % s->hks, b = bs / s->hks;
    const int64_t per = s->hq / s->hks;
    for (int64_t h = sh * per; h < (sh + 1) * per; ++h)
      for (int64_t i = 0; i < s->tq; ++i)
        if ((qoff + i) / B > j) need[(b * s->hq + h) * s->tq + i] = 2;
  }

  rowstat* st = (rowstat*)calloc((size_t)all_rows, sizeof(rowstat));

  /* Phase 1: forward statistics of each needed row; D = <dO, O>. */
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t r = 0; r < all_rows; ++r) {
    if (!need[r]) continue;
    rowinfo x = row_info(s, r);
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    st[r].L = dense_row(s, q, k, v, qs, ks, zin, &x, o, &st[r].lam);
    st[r].D = dot(dout + r * d, o, d);
    free(o);
  }

  /* Phase 2: per row, dq, dbeta, sum dbeta, dz, dqs. */
  int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)all_rows);
  for (int64_t r = 0; r < all_rows; ++r) pos[r] = -1;
  for (int64_t a = 0; a < nrows; ++a) pos[rows ? rows[a] : a] = a;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t r = 0; r < all_rows; ++r) {
    if (need[r] < 2) continue;
    rowinfo x = row_info(s, r);
    const int64_t a = pos[r];
    double* dqr = (double*)calloc((size_t)d, sizeof(double));
    double* db = (double*)calloc((size_t)(nb > 0 ? nb : 1), sizeof(double));
    const double* kb = k + (x.b * s->hkv + x.g) * (int64_t)s->tk * d;
    for (int64_t u = 0; u <= x.t; ++u) {
      const double g = dS_at(s, q, k, v, dout, qs, ks, zin, &x, &st[r], u, NULL);
      for (int64_t e = 0; e < d; ++e) dqr[e] += s->sm_scale * g * kb[u * d + e];
      if (u / B < x.c) db[u / B] += g;
    }
    double sdb = 0.0;
    for (int64_t j = 0; j < x.c; ++j) sdb += db[j];
    st[r].sdb = sdb;
    if (a >= 0) {
      if (dq) memcpy(dq + a * d, dqr, sizeof(double) * (size_t)d);
      double* dzr = (double*)calloc((size_t)(nb > 0 ? nb : 1), sizeof(double));
      for (int64_t j = 0; j < x.c; ++j) {
        const double gate = exp(score(s, qs, ks, zin, &x, j) - st[r].lam);
        dzr[j] = db[j] - gate * sdb;
      }
      if (dz) memcpy(dz + a * nb, dzr, sizeof(double) * (size_t)nb);
      if (dqs && !zin) {
        const double* kbs = ks + (x.b * s->hks + x.sh) * nb * ds;
        for (int64_t e = 0; e < ds; ++e) {
          double acc = 0.0;
          for (int64_t j = 0; j < x.c; ++j) acc += dzr[j] * kbs[j * ds + e];
          dqs[a * ds + e] = s->sel_scale * acc;
        }
      }
      free(dzr);
    }
    free(dqr);
    free(db);
  }

  /* Phase 3: per key u of kv head g, sum over every query head of the group
   * and every row that sees u. */
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t a = 0; a < nkeys; ++a) {
    const int64_t key = keys ? keys[a] : a;
    const int64_t u = key % s->tk, bg = key / s->tk, g = bg % s->hkv, b = bg / s->hkv;
    const int64_t per = s->hq / s->hkv;
    double* dkr = (double*)calloc((size_t)d, sizeof(double));
    double* dvr = (double*)calloc((size_t)d, sizeof(double));
    for (int64_t h = g * per; h < (g + 1) * per; ++h)
      for (int64_t i = 0; i < s->tq; ++i) {
        if (qoff + i < u) continue;
        const int64_t r = (b * s->hq + h) * s->tq + i;
        rowinfo x = row_info(s, r);
        double p;
        const double gs = dS_at(s, q, k, v, dout, qs, ks, zin, &x, &st[r], u, &p);
        for (int64_t e = 0; e < d; ++e) {
          dkr[e] += s->sm_scale * gs * q[r * d + e];
          dvr[e] += p * dout[r * d + e];
        }
      }
    if (dk) memcpy(dk + a * d, dkr, sizeof(double) * (size_t)d);
    if (dv) memcpy(dv + a * d, dvr, sizeof(double) * (size_t)d);
    free(dkr);
    free(dvr);
  }

  /* Phase 4: per selector block j of selector head s, sum over every query
   * head sharing s and every row with j in its history. */
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t a = 0; a < nsblk; ++a) {
    const int64_t sb = sblk ? sblk[a] : a;
    const int64_t j = sb % nb, bs = sb / nb, sh = bs % s->hks, b = bs / s->hks;
    const int64_t per = s->hq / s->hks;
    double* acc = (double*)calloc((size_t)ds, sizeof(double));
    for (int64_t h = sh * per; h < (sh + 1) * per; ++h)
      for (int64_t i = 0; i < s->tq; ++i) {
        if ((qoff + i) / B <= j) continue;
        const int64_t r = (b * s->hq + h) * s->tq + i;
        rowinfo x = row_info(s, r);
        double db = 0.0;
        for (int64_t u = j * B; u < j * B + B; ++u)
          db += dS_at(s, q, k, v, dout, qs, ks, NULL, &x, &st[r], u, NULL);
        const double gate = exp(score(s, qs, ks, NULL, &x, j) - st[r].lam);
        const double dzv = db - gate * st[r].sdb;
        for (int64_t e = 0; e < ds; ++e) acc[e] += s->sel_scale * dzv * qs[r * ds + e];
      }
    if (dks) memcpy(dks + a * ds, acc, sizeof(double) * (size_t)ds);
    free(acc);
  }

  free(need);
  free(pos);
  free(st);
  return 0;
}

/* ------------------------------------------------------------------------
 * Inference: hard Top-K over the continuous scores ([A]: the budget is the
 * number of attended context units per query).  Reading: K counts historical
 * blocks, the current block is always attended on top; rows with fewer than
 * K historical blocks take all of them; order is z descending, ties to the
 * smaller block index; padding is -1 / -inf.
 * ---------------------------------------------------------------------- */
typedef struct {
  double z;
  int64_t j;
} scored;

static int by_score_desc(const void* pa, const void* pb) {
  const scored* a = (const scored*)pa;
  const scored* b = (const scored*)pb;
  if (a->z > b->z) return -1;
  if (a->z < b->z) return 1;
  return a->j < b->j ? -1 : (a->j > b->j ? 1 : 0);
}

static int topk_impl(const oracle_shape* s, int32_t topk, int64_t fnum, int64_t fden,
                     int32_t renorm, const double* qs, const double* ks, const double* zin,
                     int32_t* idx, double* bias);

int oracle_topk_blocks(const oracle_shape* s, int32_t topk, int32_t renorm, const double* qs,
                       const double* ks, const double* zin, int32_t* idx, double* bias) {
  return topk_impl(s, topk, 0, 1, renorm, qs, ks, zin, idx, bias);
}

/* Budget proportional to the history: row t keeps n_t = min(kmax,
 * ceil(frac_num * c(t) / frac_den)) blocks (frac_num <= 0: n_t = min(kmax,
 * c(t)), the fixed budget).  The blog's "top 25%" of the context at 32k is
 * the ratio 1/4; the ceiling of the exact ratio is taken in integers, so no
 * rounding of the fraction changes a count.  idx / bias have kmax slots per
 * row, padded as for the fixed budget. */
int oracle_topk_budget(const oracle_shape* s, int32_t kmax, int32_t frac_num, int32_t frac_den,
                       int32_t renorm, const double* qs, const double* ks, const double* zin,
                       int32_t* idx, double* bias) {
  if (frac_den < 1) return -1;
  return topk_impl(s, kmax, frac_num, frac_den, renorm, qs, ks, zin, idx, bias);
}

static int topk_impl(const oracle_shape* s, int32_t topk, int64_t fnum, int64_t fden,
                     int32_t renorm, const double* qs, const double* ks, const double* zin,
                     int32_t* idx, double* bias) {
  if (check_shape(s) || topk < 1) return -1;
  const int64_t nrows = (int64_t)s->batch * s->hq * s->tq;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t r = 0; r < nrows; ++r) {
    rowinfo x = row_info(s, r);
    const int64_t c = x.c;
    scored* cand = (scored*)malloc(sizeof(scored) * (size_t)(c > 0 ? c : 1));
    double* z = (double*)malloc(sizeof(double) * (size_t)(c > 0 ? c : 1));
    for (int64_t j = 0; j < c; ++j) {
      z[j] = score(s, qs, ks, zin, &x, j);
      cand[j].z = z[j];
      cand[j].j = j;
    }
    qsort(cand, (size_t)c, sizeof(scored), by_score_desc);
    int64_t n = c < topk ? c : topk;
    if (fnum > 0) {
      const int64_t nb = (fnum * c + fden - 1) / fden; /* ceil(fnum c / fden), c >= 0 */
      if (nb < n) n = nb;
    }
    /* Bias of a selected block.  renorm = 0 (default): the training log-gate
     * z - lambda with lambda over the whole history, i.e. the same logits as
     * dense training with the unselected blocks masked out; renorm = 1: the
     * gate renormalised over the selected set.  The pages do not say which;
     * both give dense == sparse when every block is selected. */
    double norm;
    if (renorm) {
      double* zs = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
      for (int64_t a = 0; a < n; ++a) zs[a] = cand[a].z;
      norm = log_sum_exp(zs, n);
      free(zs);
    } else {
      norm = log_sum_exp(z, c);
    }
    for (int64_t a = 0; a < topk; ++a) {
      if (a < n) {
        if (idx) idx[r * topk + a] = (int32_t)cand[a].j;
        if (bias) bias[r * topk + a] = cand[a].z - norm;
      } else {
        if (idx) idx[r * topk + a] = -1;
        if (bias) bias[r * topk + a] = -INFINITY;
      }
    }
    free(cand);
    free(z);
  }
  return 0;
}

int oracle_sparse_fwd(const oracle_shape* s, int32_t topk, const double* q, const double* k,
                      const double* v, const int32_t* idx, const double* bias, int64_t nrows,
                      const int64_t* rows, double* o, double* lse) {
  if (check_shape(s) || topk < 1) return -1;
  const int64_t all = (int64_t)s->batch * s->hq * s->tq;
  if (!rows) nrows = all;
  /* Every listed block must be a distinct historical block (or -1 = none). */
  for (int64_t a = 0; a < nrows; ++a) {
    const int64_t r = rows ? rows[a] : a;
    rowinfo x = row_info(s, r);
    for (int64_t m = 0; m < topk; ++m) {
      const int64_t j = idx[r * topk + m];
      if (j == -1) continue;
      if (j < 0 || j >= x.c) return -2;
      for (int64_t m2 = 0; m2 < m; ++m2)
        if (idx[r * topk + m2] == j) return -2;
    }
  }
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t a = 0; a < nrows; ++a) {
    const int64_t r = rows ? rows[a] : a;
    rowinfo x = row_info(s, r);
    int64_t* sel = (int64_t*)malloc(sizeof(int64_t) * (size_t)topk);
    double* add = (double*)malloc(sizeof(double) * (size_t)topk);
    int64_t n = 0;
    for (int64_t m = 0; m < topk; ++m) {
      if (idx[r * topk + m] < 0) continue;
      sel[n] = idx[r * topk + m];
      add[n++] = bias[r * topk + m];
    }
    double* orow = (double*)malloc(sizeof(double) * (size_t)s->d);
    const double L = attend_row(s, q, k, v, &x, n, sel, add, orow);
    if (o) memcpy(o + a * s->d, orow, sizeof(double) * (size_t)s->d);
    if (lse) lse[a] = L;
    free(orow);
    free(sel);
    free(add);
  }
  return 0;
}

/* Dynamic-threshold selection [C] ("Implementation and Efficiency": attention
 * is computed only for the blocks whose selector score clears a threshold
 * that moves with the query).  Reading: the threshold applies to the
 * normalised gate g_j = exp(z_j - lambda) of step 2; a historical block j < c
 * is kept when g_j >= theta, i.e. z_j - lambda >= log(theta); theta <= 0
 * keeps every historical block.  Kept blocks are listed in ascending block
 * order: count[r] of them in idx[r, 0 .. count-1], the rest of the nb slots
 * padded with -1 / -inf.  Bias as in Top-K: renorm = 0 gives z - lambda
 * (= log g), renorm = 1 gives z - log sum_{kept} exp z. */
int oracle_threshold_blocks(const oracle_shape* s, float theta, int32_t renorm, const double* qs,
                            const double* ks, const double* zin, int32_t* count, int32_t* idx,
                            double* bias) {
  if (check_shape(s)) return -1;
  const int64_t nb = nblocks(s);
  const int64_t nrows = (int64_t)s->batch * s->hq * s->tq;
  const double th = (double)theta;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t r = 0; r < nrows; ++r) {
    rowinfo x = row_info(s, r);
    const int64_t c = x.c;
    double* z = (double*)malloc(sizeof(double) * (size_t)(c > 0 ? c : 1));
    for (int64_t j = 0; j < c; ++j) z[j] = score(s, qs, ks, zin, &x, j);
    const double lam = log_sum_exp(z, c);
    int64_t n = 0;
    double* kept = (double*)malloc(sizeof(double) * (size_t)(c > 0 ? c : 1));
    for (int64_t j = 0; j < c; ++j) {
      const int keep = th <= 0.0 ? 1 : (z[j] - lam >= log(th));
      if (keep) {
        idx[r * nb + n] = (int32_t)j;
        kept[n] = z[j];
        ++n;
      }
    }
    const double norm = renorm ? log_sum_exp(kept, n) : lam;
    for (int64_t a = 0; a < nb; ++a) {
      if (a < n) {
        bias[r * nb + a] = kept[a] - norm;
      } else {
        idx[r * nb + a] = -1;
        bias[r * nb + a] = -INFINITY;
      }
    }
    count[r] = (int32_t)n;
    free(kept);
    free(z);
  }
  return 0;
}
