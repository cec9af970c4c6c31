// topk.hip -- hard Top-K of the historical blocks of each query row.
//
// SAS abstracts (NeurIPS poster page, Hugging Face page): at inference a
// selector scores the context units and a hard Top-K under a fixed attention
// budget picks the ones each query attends.  Here K counts historical blocks;
// the order is score descending, block index ascending on ties; rows with
// c(t) < K keep all their c(t) blocks and pad with -1 / -inf.  The bias of a
// kept block is its training log-gate z - lam (renorm = 0) or the gate
// renormalised over the kept set (renorm = 1).
//
// One wavefront per query row.  The row's scores are computed once into LDS
// (lane j % 64 owns block j), lam comes from a wave max + sum, then K rounds
// each pick the best remaining block with a 64-lane argmax on (z, -j): round
// r takes the best candidate strictly after round r-1's winner in that total
// order, so no "already taken" set is needed.  Scores use the same fp32 dot
// product routine as the gate kernel.
#include "sas_device.h"
#include "sas_internal.h"

namespace sas {

__device__ __forceinline__ bool better(float za, int ja, float zb, int jb) {
  return za > zb || (za == zb && ja < jb);
}

template <int DS, typename ST>
__global__ __launch_bounds__(256) void topk_wave_kernel(const ST* __restrict__ qs,
                                                        const ST* __restrict__ ks, int K,
                                                        int renorm, int* __restrict__ idx,
                                                        float* __restrict__ bias, Dims D,
                                                        int wpg) {
  extern __shared__ float smem[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t nrows = (size_t)D.batch * D.hq * D.tq;
  const size_t row = (size_t)blockIdx.x * wpg + wave;
  const bool active = row < nrows;
  float* zc = smem + (size_t)wave * (D.nb + K);  // scores of this row's blocks
  float* zw = zc + D.nb;                          // winners' scores in order
  int n = 0;
  float lam = -INFINITY;
  if (active) {
    const int i = (int)(row % D.tq);
    const int h = (int)((row / D.tq) % D.hq);
    const int b = (int)(row / ((size_t)D.tq * D.hq));
    const int c = (D.qoff + i) / kBlock;
    float qsv[DS];
#pragma unroll
    for (int e = 0; e < DS; ++e) qsv[e] = to_f32(qs[row * DS + e]);
    const ST* ksb = ks + ((size_t)b * D.hks + h / D.hps) * (size_t)D.nb * DS;
    float m = -INFINITY;
    for (int j = lane; j < c; j += 64) {
      const float z = D.sel_scale * sel_dot<DS>(qsv, ksb + (size_t)j * DS);
      zc[j] = z;
      m = fmaxf(m, z);
    }
    m = wave_max(m);
    float s = 0.f;
    if (m != -INFINITY)
      for (int j = lane; j < c; j += 64) s += exp2f((zc[j] - m) * kLog2e);
    s = wave_sum(s);
    lam = c == 0 ? -INFINITY : m + log2f(s) * kLn2;
    n = c < K ? c : K;
    float pz = INFINITY;
    int pj = -1;
    for (int r = 0; r < n; ++r) {
      float bz = -INFINITY;
      int bj = 0x7fffffff;
      for (int j = lane; j < c; j += 64) {
        const float zj = zc[j];
        const bool elig = zj < pz || (zj == pz && j > pj);
        if (elig && better(zj, j, bz, bj)) {
          bz = zj;
          bj = j;
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float oz = __shfl_xor(bz, o);
        const int oj = __shfl_xor(bj, o);
        if (better(oz, oj, bz, bj)) {
          bz = oz;
          bj = oj;
        }
      }
      if (bj == 0x7fffffff) {  // nothing comparable left (non-finite scores)
        n = r;
        break;
      }
      pz = bz;
      pj = bj;
      if (lane == 0) {
        idx[row * K + r] = bj;
        zw[r] = bz;
      }
    }
  }
  __syncthreads();
  if (!active) return;
  float norm = lam;
  if (renorm) {
    float m = -INFINITY;
    for (int r = lane; r < n; r += 64) m = fmaxf(m, zw[r]);
    m = wave_max(m);
    float s = 0.f;
    for (int r = lane; r < n; r += 64) s += exp2f((zw[r] - m) * kLog2e);
    s = wave_sum(s);
    norm = n == 0 ? -INFINITY : m + log2f(s) * kLn2;
  }
  for (int r = lane; r < K; r += 64) {
    if (r < n) {
      bias[row * K + r] = zw[r] - norm;
    } else {
      idx[row * K + r] = -1;
      bias[row * K + r] = -INFINITY;
    }
  }
}

template <int DS, typename ST>
static hipError_t launch_topk_t(const void* qs, const void* ks, int K, int renorm, int* idx,
                                float* bias, const Dims& D, hipStream_t st) {
  const size_t per = (size_t)(D.nb + K) * sizeof(float);
  int wpg = 4;
  while (wpg > 1 && per * wpg > 65536) wpg >>= 1;
  if (per * wpg > 65536) return hipErrorInvalidValue;
  const size_t nrows = (size_t)D.batch * D.hq * D.tq;
  const unsigned grid = (unsigned)((nrows + wpg - 1) / wpg);
  hipLaunchKernelGGL((topk_wave_kernel<DS, ST>), dim3(grid), dim3(64 * wpg), per * wpg, st,
                     (const ST*)qs, (const ST*)ks, K, renorm, idx, bias, D, wpg);
  return hipGetLastError();
}

bool topk_supported(const Dims& D, int K) {
  return (size_t)(D.nb + K) * sizeof(float) <= 65536;
}

hipError_t launch_topk(const void* qs, const void* ks, int K, int renorm, int* idx, float* bias,
                       const Dims& D, bool sel_bf16, hipStream_t st) {
#define SAS_TOPK_CASE(DSV)                                                              \
  case DSV:                                                                             \
    return sel_bf16 ? launch_topk_t<DSV, bf16>(qs, ks, K, renorm, idx, bias, D, st)     \
                    : launch_topk_t<DSV, float>(qs, ks, K, renorm, idx, bias, D, st);
  switch (D.ds) {
    SAS_TOPK_CASE(16)
    SAS_TOPK_CASE(32)
    SAS_TOPK_CASE(64)
  }
#undef SAS_TOPK_CASE
  return hipErrorInvalidValue;
}

}  // namespace sas
