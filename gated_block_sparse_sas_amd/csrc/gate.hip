// gate.hip -- selector scores and the gate normaliser (training step 1).
//
// z[t,j] = sel_scale * <qs[t], ks[j]> for the historical blocks j < c(t);
// lam[t] = log sum_j exp z[t,j]; optionally beta[t,j] = z - lam (j < c),
// 0 (j = c), -inf (j > c).  SAS paper abstracts (NeurIPS poster page,
// Hugging Face page): the gate is a softmax over the historical blocks and its
// log enters the attention logits; the current block is always retained.
//
// Layout: one lane per query row.  Rows of a wave are consecutive positions,
// so the block index j is uniform across the wave and every ks row is a
// wave-uniform (scalar-cache) load.  HBM traffic is one qs row in and one
// float out per query row; ks (<= a few hundred KB) stays in cache.
#include "sas_device.h"
#include "sas_internal.h"

#include <type_traits>

namespace sas {

template <int DS, typename ST>
__global__ __launch_bounds__(256) void gate_lse_kernel(const ST* __restrict__ qs,
                                                       const ST* __restrict__ ks,
                                                       float* __restrict__ lam, Dims D) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int wave_first = blockIdx.x * 256 + (threadIdx.x & ~63);
  if (wave_first >= D.tq) return;  // whole wave past the end
  const int ic = i < D.tq ? i : D.tq - 1;
  const int c = (D.qoff + ic) / D.blk;
  const int cw = (D.qoff + min(wave_first + 63, D.tq - 1)) / D.blk;  // wave max of c
  const size_t row = ((size_t)b * D.hq + h) * D.tq + ic;
  SelQ<DS, ST> qsv;  // bf16 rows: packed bf16 dot products
  qsv.load(qs + row * DS);
  const ST* ksb = ks + ((size_t)b * D.hks + h / D.hps) * (size_t)D.nb * DS;
  const float zs = D.sel_scale * kLog2e;  // scores kept in log2 units
  float m = -INFINITY, s = 0.f;
  for (int j0 = 0; j0 < cw; j0 += 8) {
    float zz[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = j0 + k;
      zz[k] = -INFINITY;
      if (j < cw) {
        const float z = zs * qsv.dot(ksb + (size_t)j * DS);
        if (j < c) zz[k] = z;
      }
    }
    float mc = zz[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) mc = fmaxf(mc, zz[k]);
    const float mn = fmaxf(m, mc);
    if (mn == -INFINITY) continue;
    float acc = s * exp2f(m - mn);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += exp2f(zz[k] - mn);
    s = acc;
    m = mn;
  }
  if (i < D.tq) lam[row] = c == 0 ? -INFINITY : (m + log2f(s)) * kLn2;
}

// lam with matrix products (bf16 selectors, every unit size): a workgroup
// of 8 waves takes 256 consecutive rows of one (b, h),
// each wave 32 rows (one per lane column, as in the attention forward).  Unit
// tiles of 64 ks rows go global -> registers -> LDS, one tile ahead;
// Z^T = KS QS^T on 32x32x16 MFMA puts 16 units per M-tile of a lane's row in
// registers, so the running max and sum are in-lane plus one exchange between
// the lane halves.  The max is only moved when it grows by more than 8 (log2
// units), as in the forward.
constexpr int kGateRows = 256;

template <int DS>
__global__ __launch_bounds__(512) void gate_lse_mfma_kernel(const bf16* __restrict__ qs,
                                                            const bf16* __restrict__ ks,
                                                            float* __restrict__ lam, Dims D) {
  constexpr int XP = DS + 8;           // LDS row pitch (elements)
  constexpr int CH = DS / 8;           // 16-byte chunks per ks row
  constexpr int NL = 64 * CH;          // chunks per tile (<= 512 threads)
  __shared__ __align__(16) bf16 X0[64 * XP];
  __shared__ __align__(16) bf16 X1[64 * XP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int r0 = blockIdx.x * kGateRows;
  const int qi = r0 + wave * 32 + l32;
  const int qc = min(qi, D.tq - 1);
  const int c = (D.qoff + qc) / D.blk;  // historical units of the row
  const int wlast = min(r0 + wave * 32 + 31, D.tq - 1);
  const int cw = (D.qoff + wlast) / D.blk;                           // wave max of c
  const int cg = (D.qoff + min(r0 + kGateRows - 1, D.tq - 1)) / D.blk;  // workgroup max
  const int ntiles = (cg + 63) / 64;
  const size_t row = ((size_t)b * D.hq + h) * D.tq + qc;
  bf16x8 qf[DS / 16];
#pragma unroll
  for (int s = 0; s < DS / 16; ++s) qf[s] = *(const bf16x8*)(qs + row * DS + 16 * s + 8 * hh);
  const bf16* ksb = ks + ((size_t)b * D.hks + h / D.hps) * (size_t)D.nb * DS;
  const float zs = D.sel_scale * kLog2e;
  bf16x8 reg = bf16x8{};
  auto gload = [&](int j) {
    const int u = 64 * j + tid / CH;
    if (tid < NL) reg = u < D.nb ? *(const bf16x8*)(ksb + (size_t)u * DS + (tid % CH) * 8)
                                 : bf16x8{};
  };
  auto sstore = [&](bf16* Xd) {
    if (tid < NL) *(bf16x8*)&Xd[(tid / CH) * XP + (tid % CH) * 8] = reg;
  };
  float m_run = -INFINITY, s_run = 0.f;
  if (ntiles > 0) {
    gload(0);
    sstore(X0);
  }
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) {
    const bf16* Xs = (j & 1) ? X1 : X0;
    if (j + 1 < ntiles) gload(j + 1);
    if (64 * j < cw) {
      f32x16 z[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int s = 0; s < DS / 16; ++s)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          z[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              *(const bf16x8*)&Xs[(32 * mt + l32) * XP + 16 * s + 8 * hh], qf[s], z[mt], 0, 0, 0);
      // units past the row's history (only in the wave's last tiles)
      if (64 * j + 63 >= (D.qoff + r0 + wave * 32) / D.blk) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (64 * j + 32 * mt + 8 * (r / 4) + 4 * hh + (r % 4) >= c) z[mt][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, z[mt][r]);
      mx = halves_max(mx) * zs;
      if (__any(mx > m_run + 8.f)) {
        const float m_new = fmaxf(m_run, mx);
        if (m_new > -INFINITY) {
          s_run *= exp2_raw(m_run - m_new);
          m_run = m_new;
        }
      }
      float ps = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) ps += exp2_raw(fmaf(z[mt][r], zs, -m_run));
      s_run += m_run > -INFINITY ? ps : 0.f;
    }
    if (j + 1 < ntiles) sstore((j & 1) ? X0 : X1);
    __syncthreads();
  }
  s_run = halves_sum(s_run);
  if (qi < D.tq && hh == 0) lam[row] = c == 0 ? -INFINITY : (m_run + log2f(s_run)) * kLn2;
}

// beta[t, j] for every (row, j): one thread per entry, rows along blockIdx.y.
template <int DS, typename ST>
__global__ __launch_bounds__(256) void gate_bias_kernel(const ST* __restrict__ qs,
                                                        const ST* __restrict__ ks,
                                                        const float* __restrict__ lam,
                                                        float* __restrict__ beta, Dims D) {
  const size_t row = blockIdx.y + (size_t)gridDim.y * blockIdx.z;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (row >= (size_t)D.batch * D.hq * D.tq || j >= D.nb) return;
  const int i = (int)(row % D.tq);
  const int h = (int)((row / D.tq) % D.hq);
  const int b = (int)(row / ((size_t)D.tq * D.hq));
  const int c = (D.qoff + i) / D.blk;
  float out;
  if (j < c) {
    SelQ<DS, ST> qsv;
    qsv.load(qs + row * DS);
    const ST* ksr = ks + (((size_t)b * D.hks + h / D.hps) * D.nb + j) * DS;
    out = D.sel_scale * qsv.dot(ksr) - lam[row];
  } else {
    out = j == c ? 0.f : -INFINITY;
  }
  beta[row * D.nb + j] = out;
}

template <int DS, typename ST>
static hipError_t launch_gate_t(const void* qs, const void* ks, float* lam, float* beta,
                                const Dims& D, hipStream_t st) {
  dim3 grid((D.tq + 255) / 256, D.hq, D.batch);
  if (std::is_same<ST, bf16>::value)
    hipLaunchKernelGGL((gate_lse_mfma_kernel<DS>), dim3((D.tq + kGateRows - 1) / kGateRows,
                                                        D.hq, D.batch),
                       dim3(512), 0, st, (const bf16*)qs, (const bf16*)ks, lam, D);
  else
    hipLaunchKernelGGL((gate_lse_kernel<DS, ST>), grid, dim3(256), 0, st, (const ST*)qs,
                       (const ST*)ks, lam, D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !beta) return e;
  const size_t rows = (size_t)D.batch * D.hq * D.tq;
  const unsigned gy = rows < 65535 ? (unsigned)rows : 65535u;
  const unsigned gz = (unsigned)((rows + gy - 1) / gy);
  dim3 g2((D.nb + 255) / 256, gy, gz);
  hipLaunchKernelGGL((gate_bias_kernel<DS, ST>), g2, dim3(256), 0, st, (const ST*)qs,
                     (const ST*)ks, (const float*)lam, beta, D);
  return hipGetLastError();
}

hipError_t launch_gate(const void* qs, const void* ks, float* lam, float* beta, const Dims& D,
                       bool sel_bf16, hipStream_t st) {
#define SAS_GATE_CASE(DSV)                                                      \
  case DSV:                                                                     \
    return sel_bf16 ? launch_gate_t<DSV, bf16>(qs, ks, lam, beta, D, st)        \
                    : launch_gate_t<DSV, float>(qs, ks, lam, beta, D, st);
  switch (D.ds) {
    SAS_GATE_CASE(16)
    SAS_GATE_CASE(32)
    SAS_GATE_CASE(64)
  }
#undef SAS_GATE_CASE
  return hipErrorInvalidValue;
}

}  // namespace sas
