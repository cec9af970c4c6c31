/*
 * sas.h -- C ABI of libsas.so: SAS gated block-sparse attention on MI355X
 * (gfx950).
 *
 * Method: "SAS: Simple Attention Sparsification via End-to-End Optimization
 * of Context Ranking" (authors' abstract, NeurIPS 2026 poster page and
 * Hugging Face papers page).  A lightweight selector gives every past context
 * block a continuous score; the scores are normalised with a softmax over the
 * query's historical blocks; the log of that gate is added to every attention
 * logit of the block inside the attention softmax (logit injection, blog
 * "SAS Learns Token Importance for Sparse Attention", section "The Logit
 * Injection Mechanism").  The current block is always kept with zero bias.
 * Training attends every block (dense-active); inference keeps the current
 * block plus the top-K historical blocks (hard Top-K under an attention
 * budget, both abstracts).
 *
 * Score function (the pages leave it open; this library fixes it):
 *   z[t,j]   = sel_scale * <qs[t], ks[s(h), j]>          for j < c(t)
 *   lam[t]   = log sum_{j<c(t)} exp z[t,j]               (-inf if c(t) = 0)
 *   beta[t,j]= z[t,j] - lam[t] (j < c(t)),  0 (j = c(t))
 *   logit[t,u] = sm_scale * <q[t], k[u]> + beta[t, u/block],  u <= t
 *
 * Conventions for every entry point
 *  - Tensors are dense, contiguous BHSD device buffers owned by the caller:
 *      q, o, dq, dout [batch, hq,  tq, d]     k, v, dk, dv [batch, hkv, tk, d]
 *      qs, dqs        [batch, hq,  tq, ds]    ks, dks      [batch, hks, nb, ds]
 *      lse, gate_lse  [batch, hq,  tq]        (float32)
 *      dz, gate_bias  [batch, hq,  tq, nb]    (float32)
 *      idx, bias      [batch, hq,  tq, topk]  (int32 / float32)
 *    with nb = tk / block.  Query row i sits at absolute position
 *    t = (tk - tq) + i; its block is c(t) = t / block.
 *  - Query head h reads kv head h / (hq / hkv) and selector-key head
 *    h / (hq / hks).
 *  - dtype selects the element type of q, k, v, o, dout, dq, dk, dv;
 *    sel_dtype that of qs, ks, dqs, dks (both SAS_BF16 or both SAS_F32).
 *    Softmax statistics and accumulation are float32.
 *  - All pointers must be 16-byte aligned.  `stream` is a hipStream_t
 *    (NULL = the default stream).  Calls only enqueue work: they never
 *    synchronise, never allocate and keep no state between calls, so they are
 *    re-entrant; the results are valid once the stream reaches them.
 *  - Workspace: calls that take (ws, ws_bytes) use a size query.  With
 *    ws == NULL they write the bytes they need to *ws_bytes, return SAS_OK and
 *    launch nothing.  Otherwise *ws_bytes is the size of ws and must be at
 *    least that much (SAS_ERR_WORKSPACE if not).
 *  - Errors: every argument is checked on the host before anything is
 *    enqueued; a failed check returns a status, writes nothing and launches
 *    nothing.  Valid but unsupported shapes return SAS_ERR_UNSUPPORTED (there
 *    is no slow fallback).  A failed launch returns SAS_ERR_HIP; faults inside
 *    kernels surface at the caller's next synchronisation.
 *  - Supported: tk % 64 == 0, d in {64, 128}, ds in {16, 32, 64},
 *    hq % hkv == 0, hq % hks == 0, 1 <= tq <= tk.  batch == 0 is an empty call.
 *  - Context units (block): 64 tokens everywhere; smaller units of 1, 2, 4,
 *    8, 16 or 32 tokens (a unit may be a single token: NeurIPS abstract,
 *    "tokens or blocks") for sas_gate_scores, the Top-K, budget and threshold
 *    selections, sas_sparse_fwd (bf16 or f32), sas_attn_fwd (bf16, or f32
 *    at d = 64) and sas_attn_bwd (f32 at d = 64; bf16 at d = 128 with any
 *    ds for units of 16, 32 or 64 tokens and ds = 32 for units of 1, 2, 4
 *    or 8; bf16 at d = 64 with 64-token units only).  The paged cache takes
 *    64-token units (SAS_ERR_UNSUPPORTED otherwise).  With units under 16
 *    tokens the bf16 backward writes dz only when the caller passes it (its
 *    dks is formed without the dense [rows, nb] matrix).
 */
#ifndef SAS_H
#define SAS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SAS_OK = 0,
  SAS_ERR_NULL = 1,        /* a required pointer is NULL                  */
  SAS_ERR_SHAPE = 2,       /* sizes inconsistent or out of range          */
  SAS_ERR_DTYPE = 3,       /* unknown dtype / dtype combination           */
  SAS_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned            */
  SAS_ERR_UNSUPPORTED = 5, /* valid but not implemented for this shape    */
  SAS_ERR_WORKSPACE = 6,   /* workspace missing or too small              */
  SAS_ERR_HIP = 7,         /* a HIP launch failed                         */
  SAS_STATUS_INT32 = 0x7FFFFFFF /* not a status: makes every int32 a valid value
                                   of the type (status strings of unknown codes) */
} sas_status;

typedef enum { SAS_F32 = 0, SAS_BF16 = 1 } sas_dtype;

typedef struct {
  int32_t batch, hq, hkv, hks; /* hks <= 0 means hks = hkv                      */
  int32_t tq, tk;              /* training / prefill: tq == tk; decode: tq == 1 */
  int32_t d, ds, block;        /* head dim, selector dim, block size             */
  float sm_scale;              /* <= 0 means 1/sqrt(d)                           */
  float sel_scale;             /* <= 0 means 1/sqrt(ds)                          */
  int32_t dtype, sel_dtype;    /* sas_dtype                                      */
} sas_shape;

/* Selector scores and gate normaliser (training forward, step 1).
 * Computes lam[t] (gate_lse, required) and, if gate_bias != NULL, the full
 * log-gate matrix beta [batch,hq,tq,nb]: z - lam for j < c(t), 0 at j = c(t),
 * -inf for j > c(t).  Source: both abstracts (normalised softmax gates over
 * historical context, current block always retained). */
sas_status sas_gate_scores(const sas_shape* shape, const void* qs, const void* ks,
                           float* gate_lse, float* gate_bias, void* stream);

/* Dense-active gated attention forward (training, every block attended, each
 * historical block with its log-gate).  Inputs q, k, v, qs, ks and gate_lse
 * (from sas_gate_scores); outputs o and lse[t] = log sum_u exp logit[t,u]
 * (kept for the backward).  Source: NeurIPS abstract (gate in log form inside
 * the softmax, all units active in training, FlashAttention-style kernel). */
sas_status sas_attn_fwd(const sas_shape* shape, const void* q, const void* k, const void* v,
                        const void* qs, const void* ks, const float* gate_lse, void* o,
                        float* lse, void* stream);

/* Backward of sas_attn_fwd given dout.  Outputs dq, dk, dv (dk, dv summed
 * over the query heads of each kv head), dqs, dks (summed over the heads
 * sharing a selector head) and dz = dL/dz [batch,hq,tq,nb] (0 for j >= c(t)),
 * the gradient reaching the selector scores.  dz may be NULL (it then lives in
 * the workspace).  The workspace also holds D = <dO, O> per row, an fp32 dks
 * accumulator and, at d = 128, per-row logit offsets for every (row, gate
 * unit): batch * hq * (nb + 1) * ceil32(tq) floats (units under 16 tokens:
 * four values per row, the per-key selector rows and no dz).  Source: blog, "The Logit
 * Injection Mechanism" (gradients reach the selector through the softmax),
 * NeurIPS abstract. */
sas_status sas_attn_bwd(const sas_shape* shape, const void* q, const void* k, const void* v,
                        const void* o, const void* dout, const float* lse, const void* qs,
                        const void* ks, const float* gate_lse, void* dq, void* dk, void* dv,
                        void* dqs, void* dks, float* dz, void* ws, size_t* ws_bytes,
                        void* stream);

/* Hard Top-K of the historical blocks of every query row (inference budget):
 * the min(topk, c(t)) blocks with the largest z, ordered by z descending and
 * block index ascending on ties; idx pads with -1 and bias with -inf.
 * bias = z - lam (renorm == 0, the training log-gate of the block) or
 * z - log sum_{selected} exp z (renorm == 1).  1 <= topk.  topk <= 16
 * takes kernels without LDS (any nb); larger topk needs 4 (nb + 256 +
 * 2 next_pow2(topk)) bytes of LDS per row (topk <= 1024), at most 64 KiB,
 * unless there are at least 16384 rows and topk <= 32 (a kernel without
 * LDS); SAS_ERR_UNSUPPORTED otherwise.
 * Source: both abstracts (selector + hard Top-K; budget = attended units per
 * query); the budget counts historical blocks, the current block is extra. */
sas_status sas_topk_blocks(const sas_shape* shape, int32_t topk, int32_t renorm, const void* qs,
                           const void* ks, int32_t* idx, float* bias, void* stream);

/* Hard Top-K with a budget proportional to each row's history: row t keeps
 * n_t = min(kmax, c(t), ceil(frac_num * c(t) / frac_den)) blocks, the
 * fraction given as an exact ratio and the ceiling taken in integer
 * arithmetic (1/4 keeps a quarter of the history); frac_num <= 0 means no
 * fraction (n_t = min(kmax, c(t)), the fixed budget of sas_topk_blocks, any
 * kmax).  Order, padding (idx -1, bias -inf in slots n_t .. kmax-1) and the
 * two bias modes are those of sas_topk_blocks.  idx, bias: [batch, hq, tq,
 * kmax].  1 <= kmax <= 1024 and frac_den >= 1 (SAS_ERR_SHAPE otherwise).
 * Needs 4 (nb + 256 + 2 * next_pow2(kmax)) bytes of LDS per row, at most
 * 64 KiB (SAS_ERR_UNSUPPORTED beyond).  Source: blog, "Implementation and
 * Efficiency" (attention restricted to the top 25% of the context at 32k);
 * both abstracts (hard Top-K under an attention budget). */
sas_status sas_topk_blocks_budget(const sas_shape* shape, int32_t kmax, int32_t frac_num,
                                  int32_t frac_den, int32_t renorm, const void* qs,
                                  const void* ks, int32_t* idx, float* bias, void* stream);

/* Top-K sparse attention forward (prefill: tq == tk; decode: tq == 1; any
 * 1 <= tq <= tk): every row attends its current block (causal, bias 0) plus
 * the blocks in idx with the matching bias.  idx entries must be -1 or
 * distinct blocks j < c(t); other entries are skipped (never read out of
 * bounds).  lse may be NULL.  Source: NeurIPS abstract (a small set of context
 * units per query under a fixed budget); blog, "Implementation and
 * Efficiency" (only part of the blocks is computed). */
sas_status sas_sparse_fwd(const sas_shape* shape, int32_t topk, const void* q, const void* k,
                          const void* v, const int32_t* idx, const float* bias, void* o,
                          float* lse, void* ws, size_t* ws_bytes, void* stream);

/* Same as sas_attn_bwd, and records caller-owned hipEvent_t handles on
 * `stream` at stage boundaries, for timing single kernels:
 *   events[0] after the query-stationary kernel (dq, dz, dqs),
 *   events[1] after the key-stationary kernel (dk, dv),
 *   events[2] after the dks reduction.
 * n_events may be 0..3; NULL entries are skipped.  Used by the benchmark. */
sas_status sas_attn_bwd_ev(const sas_shape* shape, const void* q, const void* k, const void* v,
                           const void* o, const void* dout, const float* lse, const void* qs,
                           const void* ks, const float* gate_lse, void* dq, void* dk, void* dv,
                           void* dqs, void* dks, float* dz, void* ws, size_t* ws_bytes,
                           void* const* events, int32_t n_events, void* stream);

/* Same as sas_sparse_fwd, and records events[0] (if n_events >= 1 and non-NULL)
 * after the partial kernel, before the merge.  Used by the benchmark. */
sas_status sas_sparse_fwd_ev(const sas_shape* shape, int32_t topk, const void* q, const void* k,
                             const void* v, const int32_t* idx, const float* bias, void* o,
                             float* lse, void* ws, size_t* ws_bytes, void* const* events,
                             int32_t n_events, void* stream);

/* Same as sas_sparse_fwd, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the workspace is a fixed array of sas_noalloc_scratch_bytes()
 * (256 MiB) that the library holds in each GPU's memory from the first call
 * on that GPU until the process ends; the call itself allocates nothing.
 * Shapes whose workspace (the size query of sas_sparse_fwd) exceeds it return
 * SAS_ERR_WORKSPACE before anything is enqueued; tq == 1 needs none.  Every
 * call on one GPU shares that array: calls that overlap in time on one GPU
 * (two streams, or two threads) race and must be serialised by the caller.
 * The call clears the scratch it needs itself. */
sas_status sas_sparse_fwd_noalloc(const sas_shape* shape, int32_t topk, const void* q,
                                  const void* k, const void* v, const int32_t* idx,
                                  const float* bias, void* o, float* lse, void* stream);

/* Bytes of the fixed workspace of sas_sparse_fwd_noalloc. */
size_t sas_noalloc_scratch_bytes(void);

/* ---------------------------------------------------------------------------
 * Dynamic-threshold selection.  Instead of a fixed budget, row t keeps every
 * historical block whose normalised gate g = exp(z - lam) is at least theta
 * (z - lam >= log theta, evaluated in float32; theta <= 0 keeps every
 * historical block, theta > 1 none).  The count varies per row, so the
 * selection is CSR over the rows r = (b * hq + h) * tq + i:
 *   row_ptr [batch*hq*tq + 1] int64, row_ptr[0] = 0, row_ptr[rows] = nnz;
 *   col, bias [nnz]: row r's kept blocks in ascending order in
 *   row_ptr[r] .. row_ptr[r+1]-1, bias as in sas_topk_blocks (renorm 0:
 *   z - lam = log g; renorm 1: z - log sum_{kept} exp z).
 * Source: blog, "Implementation and Efficiency" (attention only for the
 * blocks whose score clears a dynamic threshold); the pages do not say what
 * the threshold is compared with: here the normalised gate of the NeurIPS
 * abstract's softmax gating. */

/* Pass 1: counts and their scan into row_ptr (device).  The caller reads
 * nnz = row_ptr[rows] after the stream reaches it and sizes col / bias.
 * theta must not be NaN.  Workspace by size query (8 bytes per 4096 rows). */
sas_status sas_threshold_count(const sas_shape* shape, float theta, const void* qs,
                               const void* ks, int64_t* row_ptr, void* ws, size_t* ws_bytes,
                               void* stream);

/* Pass 2: the kept blocks and their bias.  row_ptr from pass 1 with the same
 * shape, theta, qs and ks (the same kernel evaluates the predicate, so the
 * counts match); nnz is the capacity of col / bias: entries at positions
 * >= nnz are never written, and nnz == 0 writes nothing.  With
 * nnz = row_ptr[rows] (read back after pass 1) the selection is written
 * whole.  A caller that cannot read it back in between passes an upper
 * bound instead and enqueues pass 1, pass 2 and sas_sparse_fwd_csr with the
 * same nnz one after the other: positions from row_ptr[rows] to nnz - 1
 * belong to no row and are skipped by the forward, and the result is exact
 * iff row_ptr[rows] <= nnz, which the caller checks after its next
 * synchronisation (rows past the capacity lose their last blocks). */
sas_status sas_threshold_fill(const sas_shape* shape, float theta, int32_t renorm, const void* qs,
                              const void* ks, const int64_t* row_ptr, int64_t nnz, int32_t* col,
                              float* bias, void* stream);

/* Sparse forward over a CSR selection (any 1 <= tq <= tk, dtype SAS_BF16):
 * row r attends its current block (causal, bias 0) plus the blocks
 * col[row_ptr[r] .. row_ptr[r+1]-1] with their bias.  Entries that are not
 * historical blocks of the row, and positions outside 0 .. nnz-1, are
 * skipped; a block listed twice in a row counts twice.  Semantics otherwise
 * those of sas_sparse_fwd.  Needs nb <= 8192 and nnz plus about batch * hkv
 * * tk * hq / hkv current-block slots below 2^31 (SAS_ERR_UNSUPPORTED).
 * lse may be NULL.  Workspace by size query (grows with nnz). */
sas_status sas_sparse_fwd_csr(const sas_shape* shape, int64_t nnz, const int64_t* row_ptr,
                              const int32_t* col, const float* bias, const void* q, const void* k,
                              const void* v, void* o, float* lse, void* ws, size_t* ws_bytes,
                              void* stream);

/* Same as sas_sparse_fwd_csr, and records events[0] after the partial kernel. */
sas_status sas_sparse_fwd_csr_ev(const sas_shape* shape, int64_t nnz, const int64_t* row_ptr,
                                 const int32_t* col, const float* bias, const void* q,
                                 const void* k, const void* v, void* o, float* lse, void* ws,
                                 size_t* ws_bytes, void* const* events, int32_t n_events,
                                 void* stream);

/* ---------------------------------------------------------------------------
 * Decode over a paged cache (serving).  A page holds one 64-key block of one
 * sequence for every kv head; sequences have their own lengths and a block
 * table maps their blocks to pages, so caches grow a block at a time without
 * moving data.  Layouts (device buffers, caller-owned):
 *   k_pool, v_pool [pages, hkv, 64, d]   (dtype; one head's block = 64 x d)
 *   ks_pool        [pages, hks, ds]      (sel_dtype; the selector key of the
 *                                         block stored on the page)
 *   block_table    [batch, max_blocks]   int32 page ids
 *   seq_len        [batch]               int32 cached tokens per sequence,
 *                                         the current query's token included
 *   q [batch, hq, d], qs [batch, hq, ds], o [batch, hq, d], lse [batch, hq],
 *   idx, bias [batch, hq, topk]
 * Sequence b's query sits at t = seq_len[b] - 1 (block c(t) = t / 64) and
 * attends its current block (causal, bias 0) plus the selected historical
 * blocks, exactly as sas_sparse_fwd at tq == 1 with the sequence's blocks
 * laid out contiguously.  Device-side contents are not checked on the host:
 * a sequence with seq_len outside 1 .. max_blocks * 64 has no keys (o = 0,
 * lse = -inf, no blocks selected); a block whose page id is outside
 * 0 .. pages-1 is never read (it scores -inf in the selection and is skipped
 * in the attention).  Supported: block == 64, d in {64, 128},
 * ds in {16, 32, 64}, hq % hkv == 0, hq % hks == 0, dtype == sel_dtype.
 * Source: the method's inference mode (both abstracts: a small set of
 * context units per query under a fixed budget) applied to the usual
 * block-paged serving cache; the pages leave the cache layout open. */
typedef struct {
  int32_t batch, hq, hkv, hks; /* hks <= 0 means hks = hkv                 */
  int32_t d, ds, block;        /* block must be 64 (the page size)          */
  int32_t max_blocks;          /* columns of block_table                    */
  int32_t pages;               /* pages in the pools                        */
  float sm_scale;              /* <= 0 means 1/sqrt(d)                      */
  float sel_scale;             /* <= 0 means 1/sqrt(ds)                     */
  int32_t dtype, sel_dtype;    /* sas_dtype                                 */
} sas_paged_shape;

/* Appends one token per sequence: the rows k_new, v_new [batch, hkv, d] go to
 * position pos[b] of sequence b (page block_table[b, pos[b] / 64], row
 * pos[b] % 64).  When that token completes its block (pos[b] % 64 == 63) and
 * ks_new [batch, hks, ds] is not NULL, ks_new[b] is stored as the block's
 * selector key on the same page: the selector scores a block once it is
 * complete, and only complete blocks are ever historical.  ks_pool is
 * required when ks_new is given.  Sequences with pos outside
 * 0 .. max_blocks*64-1 or an out-of-range page are skipped.  Two sequences
 * must not write the same page row in one call. */
sas_status sas_paged_append(const sas_paged_shape* shape, const int32_t* pos,
                            const int32_t* block_table, const void* k_new, const void* v_new,
                            const void* ks_new, void* k_pool, void* v_pool, void* ks_pool,
                            void* stream);

/* Hard Top-K of the historical blocks of each sequence's query (semantics,
 * order, padding and renorm as sas_topk_blocks).  topk <= 16: any
 * max_blocks; larger topk needs 4 (max_blocks + topk) bytes of LDS per row,
 * at most 64 KiB (SAS_ERR_UNSUPPORTED beyond). */
sas_status sas_paged_topk(const sas_paged_shape* shape, int32_t topk, int32_t renorm,
                          const int32_t* seq_len, const int32_t* block_table, const void* qs,
                          const void* ks_pool, int32_t* idx, float* bias, void* stream);

/* Top-K sparse decode over the paged pools (semantics of sas_sparse_fwd at
 * tq == 1 per sequence).  lse may be NULL.  Workspace by size query. */
sas_status sas_paged_decode(const sas_paged_shape* shape, int32_t topk, const int32_t* seq_len,
                            const int32_t* block_table, const void* q, const void* k_pool,
                            const void* v_pool, const int32_t* idx, const float* bias, void* o,
                            float* lse, void* ws, size_t* ws_bytes, void* stream);

/* Selection and decode in one call: sas_topk_blocks followed by
 * sas_sparse_fwd (identical selection, padding, bias modes and outputs),
 * with one workgroup per query row choosing its blocks and attending them
 * in the same launch (no round trip of the selection through global memory,
 * one launch instead of two).  Meant for decode and other calls with few
 * rows (one workgroup per row, any tq).  1 <= topk <= 16 (SAS_ERR_SHAPE
 * below, SAS_ERR_UNSUPPORTED above); idx, bias [batch, hq, tq, topk] receive
 * the selection when not NULL; lse may be NULL.  No workspace.  Source: both
 * abstracts (a small set of context units per query at inference). */
sas_status sas_topk_decode(const sas_shape* shape, int32_t topk, int32_t renorm, const void* q,
                           const void* k, const void* v, const void* qs, const void* ks,
                           int32_t* idx, float* bias, void* o, float* lse, void* stream);

/* The same over the paged pools: sas_paged_topk followed by sas_paged_decode
 * in one launch; arguments as those two calls take them (idx, bias [batch,
 * hq, topk] may be NULL, lse may be NULL), 1 <= topk <= 16. */
sas_status sas_paged_topk_decode(const sas_paged_shape* shape, int32_t topk, int32_t renorm,
                                 const int32_t* seq_len, const int32_t* block_table,
                                 const void* q, const void* k_pool, const void* v_pool,
                                 const void* qs, const void* ks_pool, int32_t* idx, float* bias,
                                 void* o, float* lse, void* stream);

/* Static text for a status code. */
const char* sas_status_string(sas_status status);

/* Last HIP error code seen by this thread's most recent SAS_ERR_HIP (0 if none). */
int32_t sas_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SAS_H */
