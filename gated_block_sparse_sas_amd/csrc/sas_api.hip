// sas_api.hip -- the C ABI of libsas.so: argument checks and dispatch.
//
// Every check runs on the host before anything is enqueued; a failing call
// writes nothing and launches nothing.  Calls never synchronise, allocate or
// keep state.  Entry points and semantics are documented in include/sas.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/sas.h"
#include "sas_internal.h"

namespace {

thread_local int32_t g_last_hip = 0;

sas_status hip_status(hipError_t e) {
  if (e == hipSuccess) return SAS_OK;
  g_last_hip = (int32_t)e;
  return SAS_ERR_HIP;
}

bool aligned(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Resolves and validates a shape.  `need_sel` checks the selector sizes too.
sas_status resolve(const sas_shape* s, sas::Dims* D) {
  if (!s) return SAS_ERR_NULL;
  if ((s->dtype != SAS_F32 && s->dtype != SAS_BF16) ||
      (s->sel_dtype != SAS_F32 && s->sel_dtype != SAS_BF16))
    return SAS_ERR_DTYPE;
  if (s->dtype != s->sel_dtype) return SAS_ERR_DTYPE;
  const int hks = s->hks > 0 ? s->hks : s->hkv;
  if (s->batch < 0 || s->hq < 1 || s->hkv < 1 || hks < 1 || s->tq < 1 || s->tk < 1 ||
      s->d < 1 || s->ds < 1 || s->block < 1)
    return SAS_ERR_SHAPE;
  if (s->tq > s->tk || s->hq % s->hkv != 0 || s->hq % hks != 0) return SAS_ERR_SHAPE;
  if (!(s->sm_scale <= 0.f || isfinite(s->sm_scale)) ||
      !(s->sel_scale <= 0.f || isfinite(s->sel_scale)) || isnan(s->sm_scale) ||
      isnan(s->sel_scale))
    return SAS_ERR_SHAPE;
  // gate blocks of 1, 2, 4, ..., 64 tokens; keys come in 64-key tiles
  if (s->block > sas::kBlock || (s->block & (s->block - 1)) != 0 || s->tk % sas::kBlock != 0)
    return SAS_ERR_UNSUPPORTED;
  if (s->d != 64 && s->d != 128) return SAS_ERR_UNSUPPORTED;
  if (s->ds != 16 && s->ds != 32 && s->ds != 64) return SAS_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)s->batch * s->hq * s->tq;
  const int64_t keys = (int64_t)s->batch * s->hkv * s->tk;
  if (rows >= (int64_t)1 << 31 || keys >= (int64_t)1 << 31) return SAS_ERR_UNSUPPORTED;
  D->batch = s->batch;
  D->hq = s->hq;
  D->hkv = s->hkv;
  D->hks = hks;
  D->tq = s->tq;
  D->tk = s->tk;
  D->d = s->d;
  D->ds = s->ds;
  D->nb = s->tk / s->block;
  D->blk = s->block;
  D->qoff = s->tk - s->tq;
  D->hpg = s->hq / s->hkv;
  D->hps = s->hq / hks;
  D->sm_scale = s->sm_scale > 0.f ? s->sm_scale : 1.0f / sqrtf((float)s->d);
  D->sel_scale = s->sel_scale > 0.f ? s->sel_scale : 1.0f / sqrtf((float)s->ds);
  return SAS_OK;
}

// Paged-cache shape -> Dims with tq = 1, nb = max_blocks, tk = 64 * max_blocks.
sas_status resolve_paged(const sas_paged_shape* s, sas::Dims* D) {
  if (!s) return SAS_ERR_NULL;
  if ((s->dtype != SAS_F32 && s->dtype != SAS_BF16) ||
      (s->sel_dtype != SAS_F32 && s->sel_dtype != SAS_BF16))
    return SAS_ERR_DTYPE;
  if (s->dtype != s->sel_dtype) return SAS_ERR_DTYPE;
  const int hks = s->hks > 0 ? s->hks : s->hkv;
  if (s->batch < 0 || s->hq < 1 || s->hkv < 1 || hks < 1 || s->d < 1 || s->ds < 1 ||
      s->block < 1 || s->max_blocks < 1 || s->pages < 1)
    return SAS_ERR_SHAPE;
  if (s->hq % s->hkv != 0 || s->hq % hks != 0) return SAS_ERR_SHAPE;
  if (isnan(s->sm_scale) || isnan(s->sel_scale) ||
      !(s->sm_scale <= 0.f || isfinite(s->sm_scale)) ||
      !(s->sel_scale <= 0.f || isfinite(s->sel_scale)))
    return SAS_ERR_SHAPE;
  if (s->block != sas::kBlock) return SAS_ERR_UNSUPPORTED;
  if (s->d != 64 && s->d != 128) return SAS_ERR_UNSUPPORTED;
  if (s->ds != 16 && s->ds != 32 && s->ds != 64) return SAS_ERR_UNSUPPORTED;
  if ((int64_t)s->max_blocks * sas::kBlock >= (int64_t)1 << 31 ||
      (int64_t)s->batch * s->hq >= (int64_t)1 << 31)
    return SAS_ERR_UNSUPPORTED;
  D->batch = s->batch;
  D->hq = s->hq;
  D->hkv = s->hkv;
  D->hks = hks;
  D->tq = 1;
  D->tk = s->max_blocks * sas::kBlock;
  D->d = s->d;
  D->ds = s->ds;
  D->nb = s->max_blocks;
  D->blk = sas::kBlock;
  D->qoff = D->tk - 1;
  D->hpg = s->hq / s->hkv;
  D->hps = s->hq / hks;
  D->sm_scale = s->sm_scale > 0.f ? s->sm_scale : 1.0f / sqrtf((float)s->d);
  D->sel_scale = s->sel_scale > 0.f ? s->sel_scale : 1.0f / sqrtf((float)s->ds);
  return SAS_OK;
}

sas_status check_ptrs(std::initializer_list<const void*> req) {
  for (const void* p : req)
    if (!p) return SAS_ERR_NULL;
  for (const void* p : req)
    if (!aligned(p)) return SAS_ERR_ALIGN;
  return SAS_OK;
}

sas_status check_opt(std::initializer_list<const void*> opt) {
  for (const void* p : opt)
    if (p && !aligned(p)) return SAS_ERR_ALIGN;
  return SAS_OK;
}

}  // namespace

extern "C" {

const char* sas_status_string(sas_status st) {
  switch (st) {
    case SAS_OK: return "ok";
    case SAS_ERR_NULL: return "required pointer is NULL";
    case SAS_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case SAS_ERR_DTYPE: return "unknown or mismatched dtype";
    case SAS_ERR_ALIGN: return "pointer not 16-byte aligned";
    case SAS_ERR_UNSUPPORTED: return "valid shape not supported by this build";
    case SAS_ERR_WORKSPACE: return "workspace missing or too small";
    case SAS_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t sas_last_hip_error(void) { return g_last_hip; }

sas_status sas_gate_scores(const sas_shape* shape, const void* qs, const void* ks,
                           float* gate_lse, float* gate_bias, void* stream) {
  sas::Dims D;
  sas_status r = resolve(shape, &D);
  if (r != SAS_OK) return r;
  if ((r = check_ptrs({qs, ks, gate_lse})) != SAS_OK) return r;
  if ((r = check_opt({gate_bias})) != SAS_OK) return r;
  if (D.batch == 0) return SAS_OK;
  return hip_status(sas::launch_gate(qs, ks, gate_lse, gate_bias, D,
                                     shape->sel_dtype == SAS_BF16, (hipStream_t)stream));
}

sas_status sas_attn_fwd(const sas_shape* shape, const void* q, const void* k, const void* v,
                        const void* qs, const void* ks, const float* gate_lse, void* o,
                        float* lse, void* stream) {
  sas::Dims D;
  sas_status r = resolve(shape, &D);
  if (r != SAS_OK) return r;
  if ((r = check_ptrs({q, k, v, qs, ks, gate_lse, o, lse})) != SAS_OK) return r;
  if (shape->dtype == SAS_F32 && D.d != 64) return SAS_ERR_UNSUPPORTED;
  if (D.batch == 0) return SAS_OK;
  hipStream_t st = (hipStream_t)stream;
  if (shape->dtype == SAS_BF16)
    return hip_status(sas::launch_fwd_bf16(q, k, v, qs, ks, gate_lse, o, lse, D, st));
  return hip_status(sas::launch_fwd_f32(q, k, v, qs, ks, gate_lse, o, lse, D, st));
}

static sas_status attn_bwd_impl(const sas_shape* shape, const void* q, const void* k,
                                const void* v, const void* o, const void* dout, const float* lse,
                                const void* qs, const void* ks, const float* gate_lse, void* dq,
                                void* dk, void* dv, void* dqs, void* dks, float* dz, void* ws,
                                size_t* ws_bytes, const sas::StageEvents& E, void* stream) {
  sas::Dims D;
  sas_status r = resolve(shape, &D);
  if (r != SAS_OK) return r;
  if (!ws_bytes) return SAS_ERR_NULL;
  if (shape->dtype == SAS_F32 && D.d != 64) return SAS_ERR_UNSUPPORTED;
  // bf16: units of 16, 32, 64 tokens at d = 128 (and of 1 .. 8 tokens with
  // ds = 32), 64 at d = 64
  if (shape->dtype == SAS_BF16 &&
      (D.d == 128 ? D.blk < 16 && D.ds != 32 : D.blk != sas::kBlock))
    return SAS_ERR_UNSUPPORTED;
  const sas::BwdWs W = sas::bwd_workspace(D, dz == nullptr);
  if (!ws) {
    *ws_bytes = W.total;
    return SAS_OK;
  }
  if ((r = check_ptrs({q, k, v, o, dout, lse, qs, ks, gate_lse, dq, dk, dv, dqs, dks, ws})) !=
      SAS_OK)
    return r;
  if ((r = check_opt({dz})) != SAS_OK) return r;
  if (*ws_bytes < W.total) return SAS_ERR_WORKSPACE;
  if (D.batch == 0) return SAS_OK;
  hipStream_t st = (hipStream_t)stream;
  if (shape->dtype == SAS_BF16)
    return hip_status(sas::launch_bwd_bf16(q, k, v, o, dout, lse, qs, ks, gate_lse, dq, dk, dv,
                                           dqs, dks, dz, (char*)ws, W, D, E, st));
  return hip_status(sas::launch_bwd_f32(q, k, v, o, dout, lse, qs, ks, gate_lse, dq, dk, dv, dqs,
                                        dks, dz, (char*)ws, W, D, E, st));
}

sas_status sas_attn_bwd(const sas_shape* shape, const void* q, const void* k, const void* v,
                        const void* o, const void* dout, const float* lse, const void* qs,
                        const void* ks, const float* gate_lse, void* dq, void* dk, void* dv,
                        void* dqs, void* dks, float* dz, void* ws, size_t* ws_bytes,
                        void* stream) {
  return attn_bwd_impl(shape, q, k, v, o, dout, lse, qs, ks, gate_lse, dq, dk, dv, dqs, dks, dz,
                       ws, ws_bytes, sas::StageEvents{nullptr, 0}, stream);
}

sas_status sas_attn_bwd_ev(const sas_shape* shape, const void* q, const void* k, const void* v,
                           const void* o, const void* dout, const float* lse, const void* qs,
                           const void* ks, const float* gate_lse, void* dq, void* dk, void* dv,
                           void* dqs, void* dks, float* dz, void* ws, size_t* ws_bytes,
                           void* const* events, int32_t n_events, void* stream) {
  if (n_events < 0 || n_events > 3) return SAS_ERR_SHAPE;
  return attn_bwd_impl(shape, q, k, v, o, dout, lse, qs, ks, gate_lse, dq, dk, dv, dqs, dks, dz,
                       ws, ws_bytes, sas::StageEvents{events, n_events}, stream);
}

sas_status sas_topk_blocks(const sas_shape* shape, int32_t topk, int32_t renorm, const void* qs,
                           const void* ks, int32_t* idx, float* bias, void* stream) {
  sas::Dims D;
  sas_status r = resolve(shape, &D);
  if (r != SAS_OK) return r;
  if (topk < 1 || (renorm != 0 && renorm != 1)) return SAS_ERR_SHAPE;
  if ((r = check_ptrs({qs, ks, idx, bias})) != SAS_OK) return r;
  if (!sas::topk_supported(D, topk)) return SAS_ERR_UNSUPPORTED;
  if ((int64_t)D.batch * D.hq * D.tq * topk >= (int64_t)1 << 31) return SAS_ERR_UNSUPPORTED;
  if (D.batch == 0) return SAS_OK;
  return hip_status(sas::launch_topk(qs, ks, topk, renorm, idx, bias, D,
                                     shape->sel_dtype == SAS_BF16, (hipStream_t)stream));
}

sas_status sas_topk_blocks_budget(const sas_shape* shape, int32_t kmax, int32_t frac_num,
                                  int32_t frac_den, int32_t renorm, const void* qs,
                                  const void* ks, int32_t* idx, float* bias, void* stream) {
  sas::Dims D;
  sas_status r = resolve(shape, &D);
  if (r != SAS_OK) return r;
  if (kmax < 1 || (renorm != 0 && renorm != 1) || frac_den < 1) return SAS_ERR_SHAPE;
  if ((r = check_ptrs({qs, ks, idx, bias})) != SAS_OK) return r;
  if (!sas::topk_budget_supported(D, kmax)) return SAS_ERR_UNSUPPORTED;
  if ((int64_t)D.batch * D.hq * D.tq * kmax >= (int64_t)1 << 31) return SAS_ERR_UNSUPPORTED;
  if (D.batch == 0) return SAS_OK;
  return hip_status(sas::launch_topk_budget(qs, ks, kmax, frac_num, frac_den, renorm, idx, bias,
                                            D, shape->sel_dtype == SAS_BF16,
                                            (hipStream_t)stream));
}

// Checks shared by the sparse forward entry points; *need = workspace bytes.
static sas_status sparse_fwd_check(const sas_shape* shape, int32_t topk, sas::Dims* D,
                                   size_t* need) {
  sas_status r = resolve(shape, D);
  if (r != SAS_OK) return r;
  if (topk < 1) return SAS_ERR_SHAPE;
  if (shape->dtype == SAS_F32 && D->d != 64) return SAS_ERR_UNSUPPORTED;
  if ((int64_t)D->batch * D->hq * D->tq * (topk + 1) >= (int64_t)1 << 31)
    return SAS_ERR_UNSUPPORTED;
  *need = sas::sparse_workspace(*D, topk);
  return SAS_OK;
}

static sas_status sparse_fwd_impl(const sas_shape* shape, int32_t topk, const void* q,
                                  const void* k, const void* v, const int32_t* idx,
                                  const float* bias, void* o, float* lse, void* ws,
                                  size_t* ws_bytes, const sas::StageEvents& E, void* stream) {
  sas::Dims D;
  size_t need = 0;
  sas_status r = sparse_fwd_check(shape, topk, &D, &need);
  if (r != SAS_OK) return r;
  if (!ws_bytes) return SAS_ERR_NULL;
  if (!ws) {
    *ws_bytes = need;
    return SAS_OK;
  }
  if ((r = check_ptrs({q, k, v, idx, bias, o, ws})) != SAS_OK) return r;
  if ((r = check_opt({lse})) != SAS_OK) return r;
  if (*ws_bytes < need) return SAS_ERR_WORKSPACE;
  if (D.batch == 0) return SAS_OK;
  return hip_status(sas::launch_sparse(q, k, v, idx, bias, o, lse, (char*)ws, *ws_bytes, topk,
                                       D, shape->dtype == SAS_BF16, E, (hipStream_t)stream));
}

sas_status sas_sparse_fwd(const sas_shape* shape, int32_t topk, const void* q, const void* k,
                          const void* v, const int32_t* idx, const float* bias, void* o,
                          float* lse, void* ws, size_t* ws_bytes, void* stream) {
  return sparse_fwd_impl(shape, topk, q, k, v, idx, bias, o, lse, ws, ws_bytes,
                         sas::StageEvents{nullptr, 0}, stream);
}

sas_status sas_sparse_fwd_ev(const sas_shape* shape, int32_t topk, const void* q, const void* k,
                             const void* v, const int32_t* idx, const float* bias, void* o,
                             float* lse, void* ws, size_t* ws_bytes, void* const* events,
                             int32_t n_events, void* stream) {
  if (n_events < 0 || n_events > 1) return SAS_ERR_SHAPE;
  return sparse_fwd_impl(shape, topk, q, k, v, idx, bias, o, lse, ws, ws_bytes,
                         sas::StageEvents{events, n_events}, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Scratch of sas_sparse_fwd_noalloc: a fixed array in device memory, one per
// GPU (each GPU's copy of the code object holds its own), so the call needs
// no allocation.  Host code never passes `scratch` itself to a kernel (on the
// host it only names the symbol): the device address of each GPU's copy is
// looked up once per device, with that device current, and kept.
constexpr size_t kNoAllocScratchBytes = (size_t)256 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current GPU's scratch array.
hipError_t scratch_on_current_device(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  ScratchSlot& s = g_scratch[dev];
  std::call_once(s.once, [&s] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
  if (s.err != hipSuccess) return s.err;
  if (!s.ptr) return hipErrorInvalidSymbol;
  *out = (char*)s.ptr;
  return hipSuccess;
}
}  // namespace

extern "C" {

size_t sas_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

sas_status sas_sparse_fwd_noalloc(const sas_shape* shape, int32_t topk, const void* q,
                                  const void* k, const void* v, const int32_t* idx,
                                  const float* bias, void* o, float* lse, void* stream) {
  sas::Dims D;
  size_t need = 0;
  sas_status r = sparse_fwd_check(shape, topk, &D, &need);
  if (r != SAS_OK) return r;
  if ((r = check_ptrs({q, k, v, idx, bias, o})) != SAS_OK) return r;
  if ((r = check_opt({lse})) != SAS_OK) return r;
  if (need > kNoAllocScratchBytes) return SAS_ERR_WORKSPACE;
  if (D.batch == 0) return SAS_OK;
  char* ws = nullptr;
  hipError_t e = scratch_on_current_device(&ws);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(sas::launch_sparse(q, k, v, idx, bias, o, lse, ws, kNoAllocScratchBytes,
                                       topk, D, shape->dtype == SAS_BF16,
                                       sas::StageEvents{nullptr, 0}, (hipStream_t)stream));
}

sas_status sas_threshold_count(const sas_shape* shape, float theta, const void* qs,
                               const void* ks, int64_t* row_ptr, void* ws, size_t* ws_bytes,
                               void* stream) {
  sas::Dims D;
  sas_status r = resolve(shape, &D);
  if (r != SAS_OK) return r;
  if (theta != theta) return SAS_ERR_SHAPE;
  if (!ws_bytes) return SAS_ERR_NULL;
  if (D.hq > 65535 || D.batch > 65535) return SAS_ERR_UNSUPPORTED;  // grid y / z
  const size_t need = sas::threshold_workspace(D);
  if (!ws) {
    *ws_bytes = need;
    return SAS_OK;
  }
  if ((r = check_ptrs({qs, ks, row_ptr, ws})) != SAS_OK) return r;
  if (*ws_bytes < need) return SAS_ERR_WORKSPACE;
  if (D.batch == 0) return SAS_OK;
  return hip_status(sas::launch_threshold(qs, ks, theta, 0, 0, (long long*)row_ptr, nullptr,
                                          nullptr, 0, (char*)ws, D, shape->sel_dtype == SAS_BF16,
                                          (hipStream_t)stream));
}

sas_status sas_threshold_fill(const sas_shape* shape, float theta, int32_t renorm, const void* qs,
                              const void* ks, const int64_t* row_ptr, int64_t nnz, int32_t* col,
                              float* bias, void* stream) {
  sas::Dims D;
  sas_status r = resolve(shape, &D);
  if (r != SAS_OK) return r;
  if (theta != theta || nnz < 0 || (renorm != 0 && renorm != 1)) return SAS_ERR_SHAPE;
  if (D.hq > 65535 || D.batch > 65535) return SAS_ERR_UNSUPPORTED;  // grid y / z
  if ((r = check_ptrs({qs, ks, row_ptr})) != SAS_OK) return r;
  if (nnz > 0 && (r = check_ptrs({col, bias})) != SAS_OK) return r;
  if (D.batch == 0 || nnz == 0) return SAS_OK;
  return hip_status(sas::launch_threshold(qs, ks, theta, renorm, 1, (long long*)row_ptr, col,
                                          bias, nnz, nullptr, D, shape->sel_dtype == SAS_BF16,
                                          (hipStream_t)stream));
}

static sas_status sparse_csr_impl(const sas_shape* shape, int64_t nnz, const int64_t* row_ptr,
                                  const int32_t* col, const float* bias, const void* q,
                                  const void* k, const void* v, void* o, float* lse, void* ws,
                                  size_t* ws_bytes, const sas::StageEvents& E, void* stream) {
  sas::Dims D;
  sas_status r = resolve(shape, &D);
  if (r != SAS_OK) return r;
  if (nnz < 0) return SAS_ERR_SHAPE;
  if (!ws_bytes) return SAS_ERR_NULL;
  if (shape->dtype != SAS_BF16) return SAS_ERR_UNSUPPORTED;
  if (!sas::sparse_csr_supported(D, nnz)) return SAS_ERR_UNSUPPORTED;
  const size_t need = sas::sparse_csr_workspace(D, nnz);
  if (!ws) {
    *ws_bytes = need;
    return SAS_OK;
  }
  if ((r = check_ptrs({row_ptr, q, k, v, o, ws})) != SAS_OK) return r;
  if (nnz > 0 && (r = check_ptrs({col, bias})) != SAS_OK) return r;
  if ((r = check_opt({lse})) != SAS_OK) return r;
  if (*ws_bytes < need) return SAS_ERR_WORKSPACE;
  if (D.batch == 0) return SAS_OK;
  return hip_status(sas::launch_sparse_csr(q, k, v, (const long long*)row_ptr, col, bias, nnz, o,
                                           lse, (char*)ws, D, E, (hipStream_t)stream));
}

sas_status sas_sparse_fwd_csr(const sas_shape* shape, int64_t nnz, const int64_t* row_ptr,
                              const int32_t* col, const float* bias, const void* q, const void* k,
                              const void* v, void* o, float* lse, void* ws, size_t* ws_bytes,
                              void* stream) {
  return sparse_csr_impl(shape, nnz, row_ptr, col, bias, q, k, v, o, lse, ws, ws_bytes,
                         sas::StageEvents{nullptr, 0}, stream);
}

sas_status sas_sparse_fwd_csr_ev(const sas_shape* shape, int64_t nnz, const int64_t* row_ptr,
                                 const int32_t* col, const float* bias, const void* q,
                                 const void* k, const void* v, void* o, float* lse, void* ws,
                                 size_t* ws_bytes, void* const* events, int32_t n_events,
                                 void* stream) {
  if (n_events < 0 || n_events > 1) return SAS_ERR_SHAPE;
  return sparse_csr_impl(shape, nnz, row_ptr, col, bias, q, k, v, o, lse, ws, ws_bytes,
                         sas::StageEvents{events, n_events}, stream);
}

sas_status sas_paged_append(const sas_paged_shape* shape, const int32_t* pos,
                            const int32_t* block_table, const void* k_new, const void* v_new,
                            const void* ks_new, void* k_pool, void* v_pool, void* ks_pool,
                            void* stream) {
  sas::Dims D;
  sas_status r = resolve_paged(shape, &D);
  if (r != SAS_OK) return r;
  if ((r = check_ptrs({pos, block_table, k_new, v_new, k_pool, v_pool})) != SAS_OK) return r;
  if (ks_new && !ks_pool) return SAS_ERR_NULL;
  if ((r = check_opt({ks_new, ks_pool})) != SAS_OK) return r;
  if (D.batch == 0) return SAS_OK;
  return hip_status(sas::launch_paged_append(pos, block_table, k_new, v_new, ks_new, k_pool,
                                             v_pool, ks_pool, D, shape->pages,
                                             shape->dtype == SAS_BF16, (hipStream_t)stream));
}

sas_status sas_paged_topk(const sas_paged_shape* shape, int32_t topk, int32_t renorm,
                          const int32_t* seq_len, const int32_t* block_table, const void* qs,
                          const void* ks_pool, int32_t* idx, float* bias, void* stream) {
  sas::Dims D;
  sas_status r = resolve_paged(shape, &D);
  if (r != SAS_OK) return r;
  if (topk < 1 || (renorm != 0 && renorm != 1)) return SAS_ERR_SHAPE;
  if ((r = check_ptrs({seq_len, block_table, qs, ks_pool, idx, bias})) != SAS_OK) return r;
  if (topk > 16 && (size_t)(D.nb + topk) * sizeof(float) > 65536) return SAS_ERR_UNSUPPORTED;
  if ((int64_t)D.batch * D.hq * topk >= (int64_t)1 << 31) return SAS_ERR_UNSUPPORTED;
  if (D.batch == 0) return SAS_OK;
  return hip_status(sas::launch_paged_topk(qs, ks_pool, block_table, seq_len, shape->pages, topk,
                                           renorm, idx, bias, D, shape->sel_dtype == SAS_BF16,
                                           (hipStream_t)stream));
}

sas_status sas_paged_decode(const sas_paged_shape* shape, int32_t topk, const int32_t* seq_len,
                            const int32_t* block_table, const void* q, const void* k_pool,
                            const void* v_pool, const int32_t* idx, const float* bias, void* o,
                            float* lse, void* ws, size_t* ws_bytes, void* stream) {
  sas::Dims D;
  sas_status r = resolve_paged(shape, &D);
  if (r != SAS_OK) return r;
  if (topk < 1) return SAS_ERR_SHAPE;
  if (!ws_bytes) return SAS_ERR_NULL;
  if ((int64_t)D.batch * D.hq * (topk + 1) >= (int64_t)1 << 31) return SAS_ERR_UNSUPPORTED;
  const size_t need = sas::paged_workspace(D, topk);
  if (!ws) {
    *ws_bytes = need;
    return SAS_OK;
  }
  if ((r = check_ptrs({seq_len, block_table, q, k_pool, v_pool, idx, bias, o, ws})) != SAS_OK)
    return r;
  if ((r = check_opt({lse})) != SAS_OK) return r;
  if (*ws_bytes < need) return SAS_ERR_WORKSPACE;
  if (D.batch == 0) return SAS_OK;
  return hip_status(sas::launch_paged_decode(q, k_pool, v_pool, block_table, seq_len,
                                             shape->pages, idx, bias, o, lse, (char*)ws, topk, D,
                                             shape->dtype == SAS_BF16, (hipStream_t)stream));
}

sas_status sas_topk_decode(const sas_shape* shape, int32_t topk, int32_t renorm, const void* q,
                           const void* k, const void* v, const void* qs, const void* ks,
                           int32_t* idx, float* bias, void* o, float* lse, void* stream) {
  sas::Dims D;
  sas_status r = resolve(shape, &D);
  if (r != SAS_OK) return r;
  if (topk < 1 || (renorm != 0 && renorm != 1)) return SAS_ERR_SHAPE;
  if ((r = check_ptrs({q, k, v, qs, ks, o})) != SAS_OK) return r;
  if ((r = check_opt({idx, bias, lse})) != SAS_OK) return r;
  if (topk > 16) return SAS_ERR_UNSUPPORTED;
  if (shape->dtype == SAS_F32 && D.d != 64) return SAS_ERR_UNSUPPORTED;
  if ((int64_t)D.batch * D.hq * D.tq * (topk + 1) >= (int64_t)1 << 31) return SAS_ERR_UNSUPPORTED;
  if (D.batch == 0) return SAS_OK;
  return hip_status(sas::launch_topk_decode(q, k, v, qs, ks, topk, renorm, idx, bias, o, lse, D,
                                            shape->dtype == SAS_BF16, (hipStream_t)stream));
}

sas_status sas_paged_topk_decode(const sas_paged_shape* shape, int32_t topk, int32_t renorm,
                                 const int32_t* seq_len, const int32_t* block_table,
                                 const void* q, const void* k_pool, const void* v_pool,
                                 const void* qs, const void* ks_pool, int32_t* idx, float* bias,
                                 void* o, float* lse, void* stream) {
  sas::Dims D;
  sas_status r = resolve_paged(shape, &D);
  if (r != SAS_OK) return r;
  if (topk < 1 || (renorm != 0 && renorm != 1)) return SAS_ERR_SHAPE;
  if ((r = check_ptrs({seq_len, block_table, q, k_pool, v_pool, qs, ks_pool, o})) != SAS_OK)
    return r;
  if ((r = check_opt({idx, bias, lse})) != SAS_OK) return r;
  if (topk > 16) return SAS_ERR_UNSUPPORTED;
  if (shape->dtype == SAS_F32 && D.d != 64) return SAS_ERR_UNSUPPORTED;
  if ((int64_t)D.batch * D.hq * (topk + 1) >= (int64_t)1 << 31) return SAS_ERR_UNSUPPORTED;
  if (D.batch == 0) return SAS_OK;
  return hip_status(sas::launch_paged_topk_decode(
      q, k_pool, v_pool, qs, ks_pool, block_table, seq_len, shape->pages, topk, renorm, idx, bias,
      o, lse, D, shape->dtype == SAS_BF16, (hipStream_t)stream));
}

}  // extern "C"
