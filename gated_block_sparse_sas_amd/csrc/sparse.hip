// sparse.hip -- top-K block-sparse attention forward (inference).
//
// Each query row t attends its current block (keys c(t)*64 .. t, bias 0) and
// the historical blocks listed in idx[t, :] with bias[t, :] on every logit of
// the block.  SAS abstracts (NeurIPS poster page, Hugging Face page): at
// inference each query attends a small set of context units chosen by hard
// Top-K under a fixed budget; blog "SAS Learns Token Importance for Sparse
// Attention", "Implementation and Efficiency": attention is computed only for
// part of the blocks.
//
// Pair path (decode and any shape): one wavefront per (row, slot), slot K
// being the current block.  A lane owns one key of the block (its q.k dot
// product over d), the wave reduces max / sum, and the lane then owns d/64
// output columns for P V.  The partial (log-sum-exp, normalised output) goes
// to the workspace; a combine pass merges the K+1 partials of each row by
// their log-sum-exp.  Entries of idx that are not blocks before c(t) are
// skipped, so no out-of-range block is ever read.
#include "sas_device.h"
#include "sas_internal.h"

namespace sas {

static size_t align256s(size_t x) { return (x + 255) & ~(size_t)255; }

template <int HD, typename T>
__global__ __launch_bounds__(64) void sparse_pair_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int* __restrict__ idx, const float* __restrict__ bias, float* __restrict__ plse,
    T* __restrict__ po, Dims D, int K) {
  __shared__ float qsh[HD];
  __shared__ float ps[64];
  const int lane = threadIdx.x;
  const size_t pair = blockIdx.x + (size_t)gridDim.x * blockIdx.y;
  const size_t nrows = (size_t)D.batch * D.hq * D.tq;
  if (pair >= nrows * (K + 1)) return;
  const size_t row = pair / (K + 1);
  const int slot = (int)(pair % (K + 1));
  const int i = (int)(row % D.tq);
  const int h = (int)((row / D.tq) % D.hq);
  const int b = (int)(row / ((size_t)D.tq * D.hq));
  const int t = D.qoff + i, c = t / kBlock;
  const int g = h / D.hpg;
  int j;
  float add;
  if (slot < K) {
    j = idx[row * K + slot];
    add = bias[row * K + slot];
    if (j < 0 || j >= c) {
      if (lane == 0) plse[pair] = -INFINITY;
      return;
    }
  } else {
    j = c;
    add = 0.f;
  }
  for (int e = lane; e < HD; e += 64) qsh[e] = to_f32(q[row * HD + e]);
  __syncthreads();
  const size_t kvbase = ((size_t)b * D.hkv + g) * D.tk;
  const int key = j * kBlock + lane;
  const T* kr = k + (kvbase + key) * HD;
  float s = 0.f;
#pragma unroll 16
  for (int e = 0; e < HD; ++e) s = fmaf(qsh[e], to_f32(kr[e]), s);
  s = s * D.sm_scale + add;
  if (key > t) s = -INFINITY;
  const float m = wave_max(s);
  const float p = (m == -INFINITY) ? 0.f : exp2f((s - m) * kLog2e);
  const float l = wave_sum(p);
  ps[lane] = p;
  __syncthreads();
  constexpr int DPL = HD / 64;  // output columns per lane
  float acc[DPL];
#pragma unroll
  for (int x = 0; x < DPL; ++x) acc[x] = 0.f;
  const T* vb = v + (kvbase + (size_t)j * kBlock) * HD;
#pragma unroll 8
  for (int u = 0; u < kBlock; ++u) {
    const float pu = ps[u];
#pragma unroll
    for (int x = 0; x < DPL; ++x) acc[x] = fmaf(pu, to_f32(vb[(size_t)u * HD + lane * DPL + x]), acc[x]);
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int x = 0; x < DPL; ++x) po[pair * HD + lane * DPL + x] = from_f32<T>(acc[x] * inv);
  if (lane == 0) plse[pair] = (l > 0.f) ? m + logf(l) : -INFINITY;
}

// Merge the K+1 partials of each row: L = log sum_k exp(lse_k),
// O = sum_k exp(lse_k - L) O_k.  One wavefront per row.
template <int HD, typename T>
__global__ __launch_bounds__(256) void sparse_combine_kernel(const float* __restrict__ plse,
                                                             const T* __restrict__ po,
                                                             T* __restrict__ o,
                                                             float* __restrict__ lse, Dims D,
                                                             int K) {
  const int lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const size_t nrows = (size_t)D.batch * D.hq * D.tq;
  if (row >= nrows) return;
  const int np = K + 1;
  const float* pl = plse + row * np;
  float m = -INFINITY;
  for (int x = lane; x < np; x += 64) m = fmaxf(m, pl[x]);
  m = wave_max(m);
  float s = 0.f;
  for (int x = lane; x < np; x += 64) s += exp2f((pl[x] - m) * kLog2e);
  s = wave_sum(s);
  const float L = m + logf(s);
  constexpr int DPL = HD / 64;
  float acc[DPL];
#pragma unroll
  for (int x = 0; x < DPL; ++x) acc[x] = 0.f;
  for (int p = 0; p < np; ++p) {
    const float lp = pl[p];
    if (lp == -INFINITY) continue;
    const float w = exp2f((lp - L) * kLog2e);
    const T* src = po + (row * np + p) * HD + lane * DPL;
#pragma unroll
    for (int x = 0; x < DPL; ++x) acc[x] = fmaf(w, to_f32(src[x]), acc[x]);
  }
#pragma unroll
  for (int x = 0; x < DPL; ++x) o[row * HD + lane * DPL + x] = from_f32<T>(acc[x]);
  if (lse && lane == 0) lse[row] = L;
}

size_t sparse_workspace(const Dims& D, int K) {
  const size_t pairs = (size_t)D.batch * D.hq * D.tq * (K + 1);
  const size_t esz = 4;  // partial outputs are stored in the io dtype (<= 4 bytes)
  return align256s(pairs * sizeof(float)) + align256s(pairs * D.d * esz);
}

template <int HD, typename T>
static hipError_t launch_sparse_t(const void* q, const void* k, const void* v, const int* idx,
                                  const float* bias, void* o, float* lse, char* ws, int K,
                                  const Dims& D, const StageEvents& E, hipStream_t st) {
  const size_t rows = (size_t)D.batch * D.hq * D.tq;
  const size_t pairs = rows * (K + 1);
  float* plse = (float*)ws;
  T* po = (T*)(ws + align256s(pairs * sizeof(float)));
  const unsigned gx = pairs < 65536 ? (unsigned)pairs : 65536u;
  const unsigned gy = (unsigned)((pairs + gx - 1) / gx);
  hipLaunchKernelGGL((sparse_pair_kernel<HD, T>), dim3(gx, gy), dim3(64), 0, st, (const T*)q,
                     (const T*)k, (const T*)v, idx, bias, plse, po, D, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  E.record(0, st);
  hipLaunchKernelGGL((sparse_combine_kernel<HD, T>), dim3((unsigned)((rows + 3) / 4)), dim3(256),
                     0, st, (const float*)plse, (const T*)po, (T*)o, lse, D, K);
  return hipGetLastError();
}

hipError_t launch_sparse(const void* q, const void* k, const void* v, const int* idx,
                         const float* bias, void* o, float* lse, char* ws, size_t ws_bytes,
                         int K, const Dims& D, bool bf16_io, const StageEvents& E,
                         hipStream_t st) {
  (void)ws_bytes;
  if (D.d == 128)
    return bf16_io ? launch_sparse_t<128, bf16>(q, k, v, idx, bias, o, lse, ws, K, D, E, st)
                   : launch_sparse_t<128, float>(q, k, v, idx, bias, o, lse, ws, K, D, E, st);
  if (D.d == 64)
    return bf16_io ? launch_sparse_t<64, bf16>(q, k, v, idx, bias, o, lse, ws, K, D, E, st)
                   : launch_sparse_t<64, float>(q, k, v, idx, bias, o, lse, ws, K, D, E, st);
  return hipErrorInvalidValue;
}

}  // namespace sas
