// attn_f32.hip -- fp32 path of the dense-active gated attention (d = 64).
//
// Same mathematics as attn_fwd.hip / attn_bwd.hip (SAS abstracts: log gate
// inside the softmax, all blocks active, current block with zero bias), in
// plain fp32 vector arithmetic for fp32 inputs: one lane per query row
// (forward, dQ/dz/dqs) or per key (dK/dV), K/V or Q/dO tiles staged in LDS and
// read as wave-wide broadcasts.  Inputs of this path are small (the fp32
// workload is T = 512); the bf16 MFMA kernels are the throughput path.
#include "sas_device.h"
#include "sas_internal.h"

#include <algorithm>

namespace sas {

template <int DS>
__device__ __forceinline__ float dot_sel(const float* a, const float* b) {
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < DS; ++e) acc = fmaf(a[e], b[e], acc);
  return acc;
}

// Forward: 64 query rows per workgroup (one wave), one row per lane.
template <int HD, int DS>
__global__ __launch_bounds__(64) void fwd_f32_kernel(const float* __restrict__ q,
                                                     const float* __restrict__ k,
                                                     const float* __restrict__ v,
                                                     const float* __restrict__ qs,
                                                     const float* __restrict__ ks,
                                                     const float* __restrict__ lam,
                                                     float* __restrict__ o,
                                                     float* __restrict__ lse, Dims D) {
  __shared__ float Kt[64][HD + 1];
  __shared__ float Vt[64][HD + 1];
  const int lane = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int i = blockIdx.x * 64 + lane;
  const int ic = min(i, D.tq - 1);
  const int t = D.qoff + ic, c = t / kBlock;
  const int c_end = (D.qoff + min(blockIdx.x * 64 + 63, D.tq - 1)) / kBlock;
  const int g = h / D.hpg, sh = h / D.hps;
  const size_t row = ((size_t)b * D.hq + h) * D.tq + ic;
  float qr[HD], acc[HD], qsv[DS];
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    qr[e] = q[row * HD + e];
    acc[e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < DS; ++e) qsv[e] = qs[row * DS + e];
  const float lam_t = c > 0 ? lam[row] : 0.f;
  const size_t kvb = ((size_t)b * D.hkv + g) * D.tk;
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j <= c_end; ++j) {
    __syncthreads();
    for (int x = lane; x < 64 * HD; x += 64) {
      const int r = x / HD, e = x % HD;
      Kt[r][e] = k[(kvb + j * kBlock + r) * HD + e];
      Vt[r][e] = v[(kvb + j * kBlock + r) * HD + e];
    }
    __syncthreads();
    if (j > c) continue;
    const float bias =
        j < c ? D.sel_scale * dot_sel<DS>(qsv, ks + (((size_t)b * D.hks + sh) * D.nb + j) * DS) -
                    lam_t
              : 0.f;
    float s[64];
    float mx = -INFINITY;
    for (int u = 0; u < 64; ++u) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < HD; ++e) a = fmaf(qr[e], Kt[u][e], a);
      a = a * D.sm_scale + bias;
      if (j * kBlock + u > t) a = -INFINITY;
      s[u] = a;
      mx = fmaxf(mx, a);
    }
    const float mn = fmaxf(m, mx);
    const float alpha = expf(m - mn);
#pragma unroll
    for (int e = 0; e < HD; ++e) acc[e] *= alpha;
    l *= alpha;
    for (int u = 0; u < 64; ++u) {
      const float p = expf(s[u] - mn);
      l += p;
#pragma unroll
      for (int e = 0; e < HD; ++e) acc[e] = fmaf(p, Vt[u][e], acc[e]);
    }
    m = mn;
  }
  if (i < D.tq) {
#pragma unroll
    for (int e = 0; e < HD; ++e) o[row * HD + e] = acc[e] / l;
    lse[row] = m + logf(l);
  }
}

// dQ, D, dz, dqs: one query row per lane; key tiles from the diagonal down so
// that sum_j dbeta (= minus the current block's row sum of dS) is known first.
template <int HD, int DS>
__global__ __launch_bounds__(64) void bwd_dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ o, const float* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ qs, const float* __restrict__ ks, const float* __restrict__ lam,
    float* __restrict__ dq, float* __restrict__ dqs, float* __restrict__ dz,
    float* __restrict__ delta, Dims D) {
  __shared__ float Kt[64][HD + 1];
  __shared__ float Vt[64][HD + 1];
  const int lane = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int i = blockIdx.x * 64 + lane;
  const bool valid = i < D.tq;
  const int ic = min(i, D.tq - 1);
  const int t = D.qoff + ic, c = t / kBlock;
  const int c_end = (D.qoff + min(blockIdx.x * 64 + 63, D.tq - 1)) / kBlock;
  const int g = h / D.hpg, sh = h / D.hps;
  const size_t row = ((size_t)b * D.hq + h) * D.tq + ic;
  float qr[HD], dor[HD], acc[HD], qsv[DS], dqsa[DS];
  float dl = 0.f;
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    qr[e] = q[row * HD + e];
    dor[e] = dout[row * HD + e];
    dl = fmaf(dor[e], o[row * HD + e], dl);
    acc[e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < DS; ++e) {
    qsv[e] = qs[row * DS + e];
    dqsa[e] = 0.f;
  }
  if (valid) {
    delta[row] = dl;
    for (int j = c; j < D.nb; ++j) dz[row * D.nb + j] = 0.f;
  }
  const float lam_t = c > 0 ? lam[row] : 0.f;
  const float L = lse[row];
  const size_t kvb = ((size_t)b * D.hkv + g) * D.tk;
  const float* ksb = ks + ((size_t)b * D.hks + sh) * (size_t)D.nb * DS;
  float sdb = 0.f;
  for (int j = c_end; j >= 0; --j) {
    __syncthreads();
    for (int x = lane; x < 64 * HD; x += 64) {
      const int r = x / HD, e = x % HD;
      Kt[r][e] = k[(kvb + j * kBlock + r) * HD + e];
      Vt[r][e] = v[(kvb + j * kBlock + r) * HD + e];
    }
    __syncthreads();
    if (j > c) continue;
    const float bias = j < c ? D.sel_scale * dot_sel<DS>(qsv, ksb + (size_t)j * DS) - lam_t : 0.f;
    float dsum = 0.f;
    for (int u = 0; u < 64; ++u) {
      if (j * kBlock + u > t) break;
      float a = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < HD; ++e) {
        a = fmaf(qr[e], Kt[u][e], a);
        dp = fmaf(dor[e], Vt[u][e], dp);
      }
      const float p = expf(a * D.sm_scale + bias - L);
      const float ds = p * (dp - dl);
      dsum += ds;
#pragma unroll
      for (int e = 0; e < HD; ++e) acc[e] = fmaf(ds, Kt[u][e], acc[e]);
    }
    if (j == c) {
      sdb = -dsum;
    } else {
      const float dzv = dsum - expf(bias) * sdb;
      if (valid) dz[row * D.nb + j] = dzv;
      const float* kr = ksb + (size_t)j * DS;
#pragma unroll
      for (int e = 0; e < DS; ++e) dqsa[e] = fmaf(dzv, kr[e], dqsa[e]);
    }
  }
  if (valid) {
#pragma unroll
    for (int e = 0; e < HD; ++e) dq[row * HD + e] = acc[e] * D.sm_scale;
#pragma unroll
    for (int e = 0; e < DS; ++e) dqs[row * DS + e] = dqsa[e] * D.sel_scale;
  }
}

// dK, dV: one key per lane (64 keys = one block per workgroup); loops over the
// query heads of the group and 64-row query tiles at or after the block.
template <int HD, int DS>
__global__ __launch_bounds__(64) void bwd_dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, const float* __restrict__ qs, const float* __restrict__ ks,
    const float* __restrict__ lam, float* __restrict__ dk, float* __restrict__ dv, Dims D) {
  __shared__ float Qt[64][HD + 1];
  __shared__ float Ot[64][HD + 1];
  __shared__ float offs[64], Ls[64], Ds[64];
  const int lane = threadIdx.x;
  const int jb = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int u = jb * kBlock + lane;
  const size_t kvrow = ((size_t)b * D.hkv + g) * D.tk + u;
  float kr[HD], vr[HD], dka[HD], dva[HD];
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    kr[e] = k[kvrow * HD + e];
    vr[e] = v[kvrow * HD + e];
    dka[e] = 0.f;
    dva[e] = 0.f;
  }
  const int i_first = max(0, jb * kBlock - D.qoff);
  for (int hl = 0; hl < D.hpg; ++hl) {
    const int h = g * D.hpg + hl;
    const size_t base = ((size_t)b * D.hq + h) * D.tq;
    for (int i0 = (i_first / 64) * 64; i0 < D.tq; i0 += 64) {
      __syncthreads();
      for (int x = lane; x < 64 * HD; x += 64) {
        const int r = x / HD, e = x % HD;
        const int i = i0 + r;
        Qt[r][e] = i < D.tq ? q[(base + i) * HD + e] : 0.f;
        Ot[r][e] = i < D.tq ? dout[(base + i) * HD + e] : 0.f;
      }
      {
        const int i = i0 + lane;
        float off = -INFINITY, Lv = 0.f, Dv = 0.f;
        if (i < D.tq) {
          const size_t rw = base + i;
          const int t = D.qoff + i, c = t / kBlock;
          Lv = lse[rw];
          Dv = delta[rw];
          if (jb == c) {
            off = 0.f;
          } else if (jb < c) {
            off = D.sel_scale *
                      dot_sel<DS>(qs + rw * DS, ks + (((size_t)b * D.hks + h / D.hps) * D.nb + jb) * DS) -
                  lam[rw];
          }
        }
        offs[lane] = off;
        Ls[lane] = Lv;
        Ds[lane] = Dv;
      }
      __syncthreads();
      for (int r = 0; r < 64; ++r) {
        const int t = D.qoff + i0 + r;
        if (offs[r] == -INFINITY || u > t) continue;
        float a = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < HD; ++e) {
          a = fmaf(Qt[r][e], kr[e], a);
          dp = fmaf(Ot[r][e], vr[e], dp);
        }
        const float p = expf(a * D.sm_scale + offs[r] - Ls[r]);
        const float ds = p * (dp - Ds[r]);
#pragma unroll
        for (int e = 0; e < HD; ++e) {
          dka[e] = fmaf(ds, Qt[r][e], dka[e]);
          dva[e] = fmaf(p, Ot[r][e], dva[e]);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    dk[kvrow * HD + e] = dka[e] * D.sm_scale;
    dv[kvrow * HD + e] = dva[e];
  }
}

template <int DS>
static hipError_t fwd_f32_t(const void* q, const void* k, const void* v, const void* qs,
                            const void* ks, const float* lam, void* o, float* lse, const Dims& D,
                            hipStream_t st) {
  dim3 grid((D.tq + 63) / 64, D.hq, D.batch);
  hipLaunchKernelGGL((fwd_f32_kernel<64, DS>), grid, dim3(64), 0, st, (const float*)q,
                     (const float*)k, (const float*)v, (const float*)qs, (const float*)ks, lam,
                     (float*)o, lse, D);
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const void* q, const void* k, const void* v, const void* qs,
                          const void* ks, const float* lam, void* o, float* lse, const Dims& D,
                          hipStream_t st) {
  if (D.d != 64) return hipErrorInvalidValue;
  switch (D.ds) {
    case 16: return fwd_f32_t<16>(q, k, v, qs, ks, lam, o, lse, D, st);
    case 32: return fwd_f32_t<32>(q, k, v, qs, ks, lam, o, lse, D, st);
    case 64: return fwd_f32_t<64>(q, k, v, qs, ks, lam, o, lse, D, st);
  }
  return hipErrorInvalidValue;
}

template <typename ST>
hipError_t launch_dks(const float* dz, const void* qs, float* acc, void* dks, const Dims& D,
                      hipStream_t st);

template <int DS>
static hipError_t bwd_f32_t(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, const void* qs, const void* ks,
                            const float* lam, void* dq, void* dk, void* dv, void* dqs, void* dks,
                            float* dz, char* ws, const BwdWs& W, const Dims& D,
                            const StageEvents& E, hipStream_t st) {
  float* delta = (float*)(ws + W.off_delta);
  float* dzp = dz ? dz : (float*)(ws + W.off_dz);
  float* acc = (float*)(ws + W.off_dks);
  dim3 g1((D.tq + 63) / 64, D.hq, D.batch);
  hipLaunchKernelGGL((bwd_dq_f32_kernel<64, DS>), g1, dim3(64), 0, st, (const float*)q,
                     (const float*)k, (const float*)v, (const float*)o, (const float*)dout, lse,
                     (const float*)qs, (const float*)ks, lam, (float*)dq, (float*)dqs, dzp, delta,
                     D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  E.record(0, st);
  dim3 g2(D.nb, D.hkv, D.batch);
  hipLaunchKernelGGL((bwd_dkdv_f32_kernel<64, DS>), g2, dim3(64), 0, st, (const float*)q,
                     (const float*)k, (const float*)v, (const float*)dout, lse,
                     (const float*)delta, (const float*)qs, (const float*)ks, lam, (float*)dk,
                     (float*)dv, D);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  E.record(1, st);
  e = launch_dks<float>(dzp, qs, acc, dks, D, st);
  E.record(2, st);
  return e;
}

hipError_t launch_bwd_f32(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, const void* qs, const void* ks,
                          const float* lam, void* dq, void* dk, void* dv, void* dqs, void* dks,
                          float* dz, char* ws, const BwdWs& W, const Dims& D,
                          const StageEvents& E, hipStream_t st) {
  if (D.d != 64) return hipErrorInvalidValue;
  switch (D.ds) {
    case 16:
      return bwd_f32_t<16>(q, k, v, o, dout, lse, qs, ks, lam, dq, dk, dv, dqs, dks, dz, ws, W, D, E, st);
    case 32:
      return bwd_f32_t<32>(q, k, v, o, dout, lse, qs, ks, lam, dq, dk, dv, dqs, dks, dz, ws, W, D, E, st);
    case 64:
      return bwd_f32_t<64>(q, k, v, o, dout, lse, qs, ks, lam, dq, dk, dv, dqs, dks, dz, ws, W, D, E, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace sas
