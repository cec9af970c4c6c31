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

// Keys come in 64-key tiles; a tile holds 64 / B gate blocks of B keys
// (B = D.blk, 1 .. 64).  Key u belongs to block u / B; a query row t has
// c(t) = t / B historical blocks, its own block c(t) has bias 0.

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
  const int B = D.blk;
  const int t = D.qoff + ic, c = t / B;
  const int jt_end = (D.qoff + min(blockIdx.x * 64 + 63, D.tq - 1)) / kBlock;
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
  const float* ksb = ks + ((size_t)b * D.hks + sh) * (size_t)D.nb * DS;
  float m = -INFINITY, l = 0.f;
  for (int jt = 0; jt <= jt_end; ++jt) {
    __syncthreads();
    for (int x = lane; x < 64 * HD; x += 64) {
      const int r = x / HD, e = x % HD;
      Kt[r][e] = k[(kvb + jt * kBlock + r) * HD + e];
      Vt[r][e] = v[(kvb + jt * kBlock + r) * HD + e];
    }
    __syncthreads();
    if (jt * kBlock > t) continue;
    float s[64];
    float mx = -INFINITY;
    int pb = -1;
    float bias = 0.f;
    for (int u = 0; u < 64; ++u) {
      const int key = jt * kBlock + u, bu = key / B;
      if (bu != pb) {  // uniform: a new gate block starts at this key
        pb = bu;
        bias = bu < c ? D.sel_scale * dot_sel<DS>(qsv, ksb + (size_t)bu * DS) - lam_t : 0.f;
      }
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < HD; ++e) a = fmaf(qr[e], Kt[u][e], a);
      a = a * D.sm_scale + bias;
      if (key > t) a = -INFINITY;
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

// dQ, D, dz, dqs: one query row per lane; key tiles from the diagonal down.
// In the diagonal tile the current block's row sum of dS is taken first:
// sum_j dbeta_j over the historical blocks is its negative (every row of dS
// sums to zero), and dz_j = dbeta_j - g_j sum_j' dbeta_j' needs it.
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
  const int B = D.blk;
  const int t = D.qoff + ic, c = t / B, jt_t = t / kBlock;
  const int jt_end = (D.qoff + min(blockIdx.x * 64 + 63, D.tq - 1)) / kBlock;
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
  auto gate_bias = [&](int bu) __attribute__((always_inline)) {
    return bu < c ? D.sel_scale * dot_sel<DS>(qsv, ksb + (size_t)bu * DS) - lam_t : 0.f;
  };
  auto flush = [&](int bu, float bias, float dsum) __attribute__((always_inline)) {
    if (bu >= c) return;  // the current block has no selector score
    const float dzv = dsum - expf(bias) * sdb;
    if (valid) dz[row * D.nb + bu] = dzv;
    const float* kr = ksb + (size_t)bu * DS;
#pragma unroll
    for (int e = 0; e < DS; ++e) dqsa[e] = fmaf(dzv, kr[e], dqsa[e]);
  };
  for (int jt = jt_end; jt >= 0; --jt) {
    __syncthreads();
    for (int x = lane; x < 64 * HD; x += 64) {
      const int r = x / HD, e = x % HD;
      Kt[r][e] = k[(kvb + jt * kBlock + r) * HD + e];
      Vt[r][e] = v[(kvb + jt * kBlock + r) * HD + e];
    }
    __syncthreads();
    if (jt > jt_t) continue;
    if (jt == jt_t) {
      float dcur = 0.f;
      for (int key = c * B; key <= t; ++key) {
        const int u = key - jt * kBlock;
        float a = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < HD; ++e) {
          a = fmaf(qr[e], Kt[u][e], a);
          dp = fmaf(dor[e], Vt[u][e], dp);
        }
        dcur += expf(a * D.sm_scale - L) * (dp - dl);
      }
      sdb = -dcur;
    }
    int pb = (jt * kBlock) / B;
    float bias = gate_bias(pb), dsum = 0.f;
    for (int u = 0; u < 64; ++u) {
      const int key = jt * kBlock + u;
      if (key > t) break;
      const int bu = key / B;
      if (bu != pb) {
        flush(pb, bias, dsum);
        pb = bu;
        bias = gate_bias(bu);
        dsum = 0.f;
      }
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
    flush(pb, bias, dsum);
  }
  if (valid) {
#pragma unroll
    for (int e = 0; e < HD; ++e) dq[row * HD + e] = acc[e] * D.sm_scale;
#pragma unroll
    for (int e = 0; e < DS; ++e) dqs[row * DS + e] = dqsa[e] * D.sel_scale;
  }
}

// dK, dV: one key per lane (a 64-key tile per workgroup); loops over the
// query heads of the group and 64-row query tiles at or after the tile.  A
// lane's key sits in gate block u / B, so its bias for a row depends on both
// (the row's qs and lam are staged with the tile, the lane's ks row is in
// registers).
template <int HD, int DS>
__global__ __launch_bounds__(64) void bwd_dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, const float* __restrict__ qs, const float* __restrict__ ks,
    const float* __restrict__ lam, float* __restrict__ dk, float* __restrict__ dv, Dims D) {
  __shared__ float Qt[64][HD + 1];
  __shared__ float Ot[64][HD + 1];
  __shared__ float QS[64][DS + 1];
  __shared__ float Ls[64], Ds[64], Lm[64];
  __shared__ int Cs[64];
  const int lane = threadIdx.x;
  const int jt = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int B = D.blk;
  const int u = jt * kBlock + lane, bu = u / B;
  const size_t kvrow = ((size_t)b * D.hkv + g) * D.tk + u;
  float kr[HD], vr[HD], dka[HD], dva[HD], ksl[DS];
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    kr[e] = k[kvrow * HD + e];
    vr[e] = v[kvrow * HD + e];
    dka[e] = 0.f;
    dva[e] = 0.f;
  }
  const int i_first = max(0, jt * kBlock - D.qoff);
  for (int hl = 0; hl < D.hpg; ++hl) {
    const int h = g * D.hpg + hl;
    const size_t base = ((size_t)b * D.hq + h) * D.tq;
    const float* ksr = ks + (((size_t)b * D.hks + h / D.hps) * D.nb + bu) * DS;
#pragma unroll
    for (int e = 0; e < DS; ++e) ksl[e] = ksr[e];
    for (int i0 = (i_first / 64) * 64; i0 < D.tq; i0 += 64) {
      __syncthreads();
      for (int x = lane; x < 64 * HD; x += 64) {
        const int r = x / HD, e = x % HD;
        const int i = i0 + r;
        Qt[r][e] = i < D.tq ? q[(base + i) * HD + e] : 0.f;
        Ot[r][e] = i < D.tq ? dout[(base + i) * HD + e] : 0.f;
      }
      for (int x = lane; x < 64 * DS; x += 64) {
        const int r = x / DS, e = x % DS;
        const int i = i0 + r;
        QS[r][e] = i < D.tq ? qs[(base + i) * DS + e] : 0.f;
      }
      {
        const int i = i0 + lane;
        const bool ok = i < D.tq;
        const size_t rw = base + (ok ? i : 0);
        const int t = D.qoff + i;
        Ls[lane] = ok ? lse[rw] : 0.f;
        Ds[lane] = ok ? delta[rw] : 0.f;
        Cs[lane] = ok ? t / B : -1;
        Lm[lane] = ok && t / B > 0 ? lam[rw] : 0.f;
      }
      __syncthreads();
      for (int r = 0; r < 64; ++r) {
        const int t = D.qoff + i0 + r, cr = Cs[r];
        if (cr < 0 || u > t) continue;
        // bu <= cr here (u <= t): historical block with its gate, or the current block
        const float off = bu < cr ? D.sel_scale * dot_sel<DS>(&QS[r][0], ksl) - Lm[r] : 0.f;
        float a = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < HD; ++e) {
          a = fmaf(Qt[r][e], kr[e], a);
          dp = fmaf(Ot[r][e], vr[e], dp);
        }
        const float p = expf(a * D.sm_scale + off - Ls[r]);
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
  dim3 g2(D.tk / kBlock, D.hkv, D.batch);
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
