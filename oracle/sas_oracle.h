/*
 * sas_oracle.h -- plain fp64 CPU oracle for SAS gated block-sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this code; only the test-suite, the smoke check and the CPU baseline
 * leg of the benchmark do.  It shares no source with the HIP path.
 *
 * Method: "SAS: Simple Attention Sparsification via End-to-End Optimization
 * of Context Ranking" (authors' abstract on the NeurIPS 2026 poster page and
 * on the Hugging Face papers page).  A selector scores every past context
 * block, the scores are normalised with a softmax over the query's historical
 * blocks, and the log of that gate is added to every attention logit of the
 * block inside the attention softmax; the current block is always kept with a
 * zero bias.  The pages leave the score function open; this oracle takes
 * z = sel_scale * <qs_t, ks_j> (bilinear selector), which is the spec.
 *
 * Conventions (every array is dense, row-major, fp64, BHSD):
 *   q   [batch, hq,  tq, d]        k, v [batch, hkv, tk, d]
 *   qs  [batch, hq,  tq, ds]       ks   [batch, hks, nb, ds]
 *   z / beta / dz  [batch, hq, tq, nb]
 *   nb = ceil(tk / block); the last key block may be ragged.
 *   query i sits at absolute position t = (tk - tq) + i, its block is
 *   c(t) = floor(t / block); historical blocks are j < c(t).
 *   kv head of query head h: g = h * hkv / hq; selector head s = h * hks / hq.
 */
#ifndef SAS_ORACLE_H
#define SAS_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t batch, hq, hkv, hks;
  int32_t tq, tk;
  int32_t d, ds, block;
  double sm_scale;  /* tau: attention logit scale            */
  double sel_scale; /* sigma: selector score scale           */
} oracle_shape;

/* Return codes: 0 ok, -1 bad shape. */

/* Selector scores z (j < c(t); -inf elsewhere), gate log-normaliser lambda
 * (-inf when c(t) = 0) and the log-gate beta (z - lambda for j < c(t), 0 at
 * j = c(t), -inf for j > c(t)).  Any output pointer may be NULL. */
int oracle_gate_scores(const oracle_shape* s, const double* qs, const double* ks,
                       double* z, double* lam, double* beta);

/* Dense-active gated attention forward on a list of rows.
 * rows: flat indices (b*hq + h)*tq + i; NULL means every row in order.
 * zin:  NULL -> scores from qs/ks; else scores-in [batch,hq,tq,nb].
 * o [nrows, d] and lse [nrows] hold the results row by row. */
int oracle_attn_fwd(const oracle_shape* s, const double* q, const double* k, const double* v,
                    const double* qs, const double* ks, const double* zin,
                    int64_t nrows, const int64_t* rows, double* o, double* lse);

/* Dense-active backward.  Outputs are computed only where asked:
 *   rows  (flat (b,h,i)):  dq [nrows,d], dz [nrows,nb], dqs [nrows,ds]
 *   keys  (flat (b,g,u)):  dk [nkeys,d], dv [nkeys,d]
 *   sblk  (flat (b,s,j)):  dks [nsblk,ds]
 * A NULL list with count -1 means "all" in natural order.  Any output may be
 * NULL.  dqs/dks are ignored (left untouched) when zin != NULL. */
int oracle_attn_bwd(const oracle_shape* s, const double* q, const double* k, const double* v,
                    const double* dout, const double* qs, const double* ks, const double* zin,
                    int64_t nrows, const int64_t* rows, double* dq, double* dz, double* dqs,
                    int64_t nkeys, const int64_t* keys, double* dk, double* dv,
                    int64_t nsblk, const int64_t* sblk, double* dks);

/* Top-K historical blocks per row by (z desc, j asc), and their bias.
 * idx [batch,hq,tq,topk] (pad -1), bias same shape (pad -inf).
 * renorm = 0: bias = z - lambda (lambda over all history);
 * renorm = 1: bias = z - log sum_{selected} exp(z). */
int oracle_topk_blocks(const oracle_shape* s, int32_t topk, int32_t renorm,
                       const double* qs, const double* ks, const double* zin,
                       int32_t* idx, double* bias);
/* Top-K with a budget proportional to the history: n_t = min(kmax,
 * ceil(frac_num * c(t) / frac_den)) blocks per row, the ceiling of an exact
 * ratio in integers (frac_num <= 0: min(kmax, c(t))); kmax slots per row,
 * padded with -1 / -inf. */
int oracle_topk_budget(const oracle_shape* s, int32_t kmax, int32_t frac_num, int32_t frac_den,
                       int32_t renorm, const double* qs, const double* ks, const double* zin,
                       int32_t* idx, double* bias);

/* Dynamic-threshold selection: a historical block j < c is kept when its
 * normalised gate exp(z_j - lambda) >= theta (theta <= 0 keeps all).
 * count [batch,hq,tq]; idx [batch,hq,tq,nb] lists the kept blocks in
 * ascending order (pad -1), bias the same slots (pad -inf); renorm as for
 * Top-K. */
int oracle_threshold_blocks(const oracle_shape* s, float theta, int32_t renorm, const double* qs,
                            const double* ks, const double* zin, int32_t* count, int32_t* idx,
                            double* bias);

/* Sparse attention forward: each row attends its current block (causal,
 * bias 0) plus the blocks listed in idx with the given bias.
 * rows / o / lse as in oracle_attn_fwd. */
int oracle_sparse_fwd(const oracle_shape* s, int32_t topk, const double* q, const double* k,
                      const double* v, const int32_t* idx, const double* bias,
                      int64_t nrows, const int64_t* rows, double* o, double* lse);

/* Number of OpenMP threads the oracle runs with. */
int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
