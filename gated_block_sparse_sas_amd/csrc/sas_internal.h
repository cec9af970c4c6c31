// sas_internal.h -- launchers shared between the C ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>

#include "sas_device.h"

namespace sas {

// Optional caller-owned events recorded between the kernels of one call.
struct StageEvents {
  void* const* ev;
  int n;
  void record(int i, hipStream_t st) const {
    if (ev && i < n && ev[i]) (void)hipEventRecord((hipEvent_t)ev[i], st);
  }
};

// Step 1: gate normaliser lam (and optional full log-gate matrix).
hipError_t launch_gate(const void* qs, const void* ks, float* lam, float* beta, const Dims& D,
                       bool sel_bf16, hipStream_t st);

// Step 2: dense-active gated forward.
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, const void* qs,
                           const void* ks, const float* lam, void* o, float* lse, const Dims& D,
                           hipStream_t st);
hipError_t launch_fwd_given_bias(const void* q, const void* k, const void* v, const float* bt,
                                 void* o, float* lse, const Dims& D, hipStream_t st);
hipError_t launch_fwd_f32(const void* q, const void* k, const void* v, const void* qs,
                          const void* ks, const float* lam, void* o, float* lse, const Dims& D,
                          hipStream_t st);

// Steps 3-4: backward.  Workspace layout is decided by bwd_workspace().
struct BwdWs {
  size_t total;
  size_t off_delta;  // float [rows]          D = <dO, O>
  size_t off_dz;     // float [rows, nb]      only when the caller passes no dz
  size_t off_dks;    // float [b, hks, nb, ds] fp32 accumulator of dks
  size_t off_rows;   // d = 128: float [b, hq, nb + 1, tqp] per-row data of the dK/dV kernel
                     // (units under 16 tokens: [b, hq, 4, tqp])
  size_t off_ksx;    // units of 2 .. 8 tokens: bf16 [b, hks, tk, ds] per-key selector rows
  int tqp;           // tq rounded up to 32
};
BwdWs bwd_workspace(const Dims& D, bool need_dz);
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, const void* qs, const void* ks,
                           const float* lam, void* dq, void* dk, void* dv, void* dqs, void* dks,
                           float* dz, char* ws, const BwdWs& W, const Dims& D,
                           const StageEvents& E, hipStream_t st);
hipError_t launch_bwd_f32(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, const void* qs, const void* ks,
                          const float* lam, void* dq, void* dk, void* dv, void* dqs, void* dks,
                          float* dz, char* ws, const BwdWs& W, const Dims& D,
                          const StageEvents& E, hipStream_t st);

// Step 5: top-K blocks.
bool topk_supported(const Dims& D, int K);
bool topk_budget_supported(const Dims& D, int kmax);
hipError_t launch_topk_budget(const void* qs, const void* ks, int kmax, int fnum, int fden,
                              int renorm, int* idx, float* bias, const Dims& D, bool sel_bf16,
                              hipStream_t st);
hipError_t launch_topk(const void* qs, const void* ks, int K, int renorm, int* idx, float* bias,
                       const Dims& D, bool sel_bf16, hipStream_t st);

// Steps 6-7: sparse forward.
size_t sparse_workspace(const Dims& D, int K);
hipError_t launch_sparse(const void* q, const void* k, const void* v, const int* idx,
                         const float* bias, void* o, float* lse, char* ws, size_t ws_bytes,
                         int K, const Dims& D, bool bf16_io, const StageEvents& E,
                         hipStream_t st);

// Selection and decode in one launch (K <= 16).
hipError_t launch_topk_decode(const void* q, const void* k, const void* v, const void* qs,
                              const void* ks, int K, int renorm, int* idx, float* bias, void* o,
                              float* lse, const Dims& D, bool bf16_io, hipStream_t st);
hipError_t launch_paged_topk_decode(const void* q, const void* k_pool, const void* v_pool,
                                    const void* qs, const void* ks_pool, const int* table,
                                    const int* lens, int pages, int K, int renorm, int* idx,
                                    float* bias, void* o, float* lse, const Dims& D,
                                    bool bf16_io, hipStream_t st);

// Dynamic-threshold selection (CSR) and the sparse forward over a CSR selection.
size_t threshold_workspace(const Dims& D);
hipError_t launch_threshold(const void* qs, const void* ks, float theta, int renorm, int fill,
                            long long* row_ptr, int* col, float* bias, long long nnz, char* ws,
                            const Dims& D, bool sel_bf16, hipStream_t st);
bool sparse_csr_supported(const Dims& D, long long nnz);
size_t sparse_csr_workspace(const Dims& D, long long nnz);
hipError_t launch_sparse_csr(const void* q, const void* k, const void* v, const long long* row_ptr,
                             const int* col, const float* bias, long long nnz, void* o,
                             float* lse, char* ws, const Dims& D, const StageEvents& E,
                             hipStream_t st);

// Paged decode cache (serving): append, selection and decode over page pools.
// Dims: tq = 1, nb = max_blocks, tk = 64 * max_blocks.
hipError_t launch_paged_append(const int* pos, const int* table, const void* k_new,
                               const void* v_new, const void* ks_new, void* k_pool, void* v_pool,
                               void* ks_pool, const Dims& D, int pages, bool is_bf16,
                               hipStream_t st);
hipError_t launch_paged_topk(const void* qs, const void* ks_pool, const int* table,
                             const int* lens, int pages, int K, int renorm, int* idx, float* bias,
                             const Dims& D, bool sel_bf16, hipStream_t st);
size_t paged_workspace(const Dims& D, int K);
hipError_t launch_paged_decode(const void* q, const void* k_pool, const void* v_pool,
                               const int* table, const int* lens, int pages, const int* idx,
                               const float* bias, void* o, float* lse, char* ws, int K,
                               const Dims& D, bool bf16_io, hipStream_t st);

}  // namespace sas
