// attn_bwd.hip -- backward of the dense-active gated attention.
//
// With P = softmax of the gated logits, O = P V and upstream dO:
//   D_t = <dO_t, O_t>,  dP = dO V^T,  dS = P o (dP - D)
//   dQ = sm_scale dS K,  dK = sm_scale dS^T Q,  dV = P^T dO   (dK, dV summed over
//   the query heads of each kv head)
//   dbeta_{t,j} = sum_{u in block j} dS_{t,u}                    (j < c(t))
//   dz_{t,j} = dbeta_{t,j} - g_{t,j} sum_{j'<c(t)} dbeta_{t,j'},  g = exp(beta)
//   dqs_t = sel_scale sum_j dz_{t,j} ks_j,  dks_j = sel_scale sum_t dz_{t,j} qs_t
// SAS (blog "SAS Learns Token Importance for Sparse Attention", "The Logit
// Injection Mechanism"; NeurIPS abstract): because the gate sits in the logits,
// the loss gradient reaches the selector scores through the softmax.
//
// Kernels:
//  * bwd_dq (query-stationary, same tiling as the forward): S^T, dP^T, dQ^T
//    with the query in the MFMA column, so dbeta is an in-lane row sum.  Key
//    tiles run from the diagonal down, so sum_j dbeta_{t,j} is known (it equals
//    minus the row sum of dS over the current block, because every row of dS
//    sums to zero) before the first historical tile: dz and dqs are produced on
//    the fly and dz is written once.  D is computed here and kept for bwd_dkdv.
//  * bwd_dkdv (key-stationary): 128 keys per workgroup, 32 per wave, K and V
//    in registers; loops over the query heads of the group and the query tiles
//    at or after the keys.  S = Q K^T with the key in the MFMA column, so P and
//    dS feed dV^T += dO^T P and dK^T += Q^T dS straight from registers; Q and
//    dO are staged in LDS both row-major and transposed.
//  * dks: a reduction over rows of dz^T qs into an fp32 accumulator.
// At d = 128 the same steps run on gfx950 MFMA tiles: bwd_dq32 (32 query rows
// per wave, 32x32x16; selectors up to ds = 32), bwd_dq16 (16 rows per wave,
// 16x16x32; wider selectors) and bwd_dkdv16 (16 keys per wave, 16x16x32).
#include "sas_device.h"
#include "sas_internal.h"

#include <algorithm>
#include <type_traits>

namespace sas {

// --------------------------------------------------------------------------
// Query-stationary: dQ, D, dz, dqs.
// --------------------------------------------------------------------------
template <int HD, int DS>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ o, const bf16* __restrict__ dout, const float* __restrict__ lse,
    const bf16* __restrict__ qs, const bf16* __restrict__ ks, const float* __restrict__ lam,
    bf16* __restrict__ dq, bf16* __restrict__ dqs, float* __restrict__ dz,
    float* __restrict__ delta, Dims D, int nqt, int xcd_groups) {
  constexpr int KP = HD + 8;
  constexpr int TP = kBlock + 8;
  constexpr int KS = HD / 16;
  constexpr int DM = HD / 32;
  constexpr int ITEMS = 16 * (HD / 8);  // (4 keys x 8 dims) items per tile
  constexpr int IT = (ITEMS + 255) / 256;
  __shared__ __align__(16) bf16 Ks[kBlock * KP];
  __shared__ __align__(16) bf16 Vs[kBlock * KP];
  __shared__ __align__(16) bf16 Kt[HD * TP];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, hh = lane >> 5;
  const QTile tm = map_q_tile(blockIdx.x, nqt, D, xcd_groups);
  const int b = tm.b, h = tm.h, qt = tm.qt;
  const int g = h / D.hpg, sh = h / D.hps;
  const int wq0 = qt * 128 + wave * 32;
  const int qi = wq0 + l32;
  const bool valid = qi < D.tq;
  const int qc = min(qi, D.tq - 1);
  const int t = D.qoff + qc;
  const int c = t / kBlock;
  const int c_hi = (D.qoff + min(wq0 + 31, D.tq - 1)) / kBlock;
  const int c_lo = (D.qoff + min(wq0, D.tq - 1)) / kBlock;
  const int c_end = (D.qoff + min(qt * 128 + 127, D.tq - 1)) / kBlock;
  const size_t row = ((size_t)b * D.hq + h) * D.tq + qc;

  // zero dz[row, j] for j >= c(row) for this workgroup's rows (coalesced)
  for (int r = 0; r < 128; ++r) {
    const int i = qt * 128 + r;
    if (i >= D.tq) break;
    const int cr = (D.qoff + i) / kBlock;
    float* zr = dz + (((size_t)b * D.hq + h) * D.tq + i) * D.nb;
    for (int j = cr + tid; j < D.nb; j += 256) zr[j] = 0.f;
  }

  bf16x8 qf[KS], df[KS];
  float dlt = 0.f;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qf[s] = *(const bf16x8*)(q + row * HD + 16 * s + 8 * hh);
    df[s] = *(const bf16x8*)(dout + row * HD + 16 * s + 8 * hh);
    const bf16x8 of = *(const bf16x8*)(o + row * HD + 16 * s + 8 * hh);
#pragma unroll
    for (int e = 0; e < 8; ++e) dlt = fmaf(to_f32(df[s][e]), to_f32(of[e]), dlt);
  }
  dlt += __shfl_xor(dlt, 32);
  if (valid && hh == 0) delta[row] = dlt;
  float qsv[DS / 2];
#pragma unroll
  for (int e = 0; e < DS / 2; ++e) qsv[e] = to_f32(qs[row * DS + hh * (DS / 2) + e]);
  const float lam_t = c > 0 ? lam[row] : 0.f;
  const float l2 = lse[row] * kLog2e;
  const bf16* ksb = ks + ((size_t)b * D.hks + sh) * (size_t)D.nb * DS + hh * (DS / 2);
  const bf16* kb = k + ((size_t)b * D.hkv + g) * (size_t)D.tk * HD;
  const bf16* vb = v + ((size_t)b * D.hkv + g) * (size_t)D.tk * HD;
  const float c1 = D.sm_scale * kLog2e;

  f32x16 dqacc[DM];
#pragma unroll
  for (int dm = 0; dm < DM; ++dm) dqacc[dm] = f32x16{};
  float dqsacc[DS / 2];
#pragma unroll
  for (int e = 0; e < DS / 2; ++e) dqsacc[e] = 0.f;
  float sdb = 0.f;  // sum over history of dbeta for this row

  const bf16x8 zero8 = bf16x8{};
  bf16x8 kreg[IT][4], vreg[IT][4];
  auto gload = [&](int j) {
#pragma unroll
    for (int x = 0; x < IT; ++x) {
      const int id = tid + 256 * x;
      if (id < ITEMS) {
        const int kg = id % 16, dc = id / 16;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          const int key = j * kBlock + kg * 4 + i2;
          const bool in = key < D.tk;
          kreg[x][i2] = in ? *(const bf16x8*)(kb + (size_t)key * HD + dc * 8) : zero8;
          vreg[x][i2] = in ? *(const bf16x8*)(vb + (size_t)key * HD + dc * 8) : zero8;
        }
      }
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int x = 0; x < IT; ++x) {
      const int id = tid + 256 * x;
      if (id < ITEMS) {
        const int kg = id % 16, dc = id / 16;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          *(bf16x8*)&Ks[(kg * 4 + i2) * KP + dc * 8] = kreg[x][i2];
          *(bf16x8*)&Vs[(kg * 4 + i2) * KP + dc * 8] = vreg[x][i2];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bf16x4 w = {kreg[x][0][e], kreg[x][1][e], kreg[x][2][e], kreg[x][3][e]};
          *(bf16x4*)&Kt[(dc * 8 + e) * TP + kg * 4] = w;
        }
      }
    }
  };

  gload(c_end);
  for (int j = c_end; j >= 0; --j) {
    __syncthreads();
    sstore();
    __syncthreads();
    if (j > 0) gload(j - 1);
    if (j > c_hi) continue;

    float bias2 = 0.f;
    float ksv[DS / 2];
    if (j < c_hi) {
      const bf16* kr = ksb + (size_t)j * DS;
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < DS / 2; ++e) {
        ksv[e] = to_f32(kr[e]);
        part = fmaf(qsv[e], ksv[e], part);
      }
      part += __shfl_xor(part, 32);
      if (j < c) bias2 = (D.sel_scale * part - lam_t) * kLog2e;
    }
    const float off = bias2 - l2;

    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    f32x16 pacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 a = *(const bf16x8*)&Ks[(32 * mt + l32) * KP + 16 * s + 8 * hh];
        sacc[mt] = mfma32(a, qf[s], sacc[mt]);
        const bf16x8 av = *(const bf16x8*)&Vs[(32 * mt + l32) * KP + 16 * s + 8 * hh];
        pacc[mt] = mfma32(av, df[s], pacc[mt]);
      }
    }
    float dsum = 0.f;
    auto softmax_ds = [&](auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = exp2_raw(fmaf(sacc[mt][r], c1, off));
          if constexpr (MASK) {
            const int u = j * kBlock + 32 * mt + (r / 4) * 8 + 4 * hh + (r % 4);
            if (u > t) p = 0.f;
          }
          const float ds = p * (pacc[mt][r] - dlt);
          sacc[mt][r] = ds;
          dsum += ds;
        }
      }
    };
    if (j < c_lo)
      softmax_ds(std::false_type{});
    else
      softmax_ds(std::true_type{});
    dsum += __shfl_xor(dsum, 32);
    if (j == c) {
      sdb = -dsum;  // sum_{j'<c} dbeta = - sum over the current block of dS
    } else if (j < c) {
      const float dzv = dsum - exp2_raw(bias2) * sdb;
      if (valid && hh == 0) dz[row * D.nb + j] = dzv;
#pragma unroll
      for (int e = 0; e < DS / 2; ++e) dqsacc[e] = fmaf(dzv, ksv[e], dqsacc[e]);
    }

    // dQ^T += K^T dS^T
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        bf16x8 sb;
#pragma unroll
        for (int e = 0; e < 8; ++e) sb[e] = (bf16)sacc[mt][8 * pp + e];
#pragma unroll
        for (int dm = 0; dm < DM; ++dm) {
          const bf16* kp = &Kt[(32 * dm + l32) * TP + 32 * mt + 16 * pp + 4 * hh];
          const bf16x4 lo = *(const bf16x4*)kp;
          const bf16x4 hi = *(const bf16x4*)(kp + 8);
          const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          dqacc[dm] = mfma32(a, sb, dqacc[dm]);
        }
      }
    }
  }

  if (valid) {
    bf16* qr = dq + row * HD;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(dqacc[dm][4 * rr + e] * D.sm_scale);
        *(bf16x4*)(qr + 32 * dm + 8 * rr + 4 * hh) = w;
      }
    }
#pragma unroll
    for (int e = 0; e < DS / 2; ++e)
      dqs[row * DS + hh * (DS / 2) + e] = (bf16)(dqsacc[e] * D.sel_scale);
  }
}

// --------------------------------------------------------------------------
// Query-stationary dQ, D, dz, dqs for d = 128 on 16x16x32 MFMA tiles: a
// workgroup owns 64 query rows, each wave 16 (the query sits in the MFMA
// column, so D, the dS row sums and the selector terms are per-lane values
// plus two cross-group adds).  64-key K and V tiles (and the block's ks row)
// stream global -> LDS with direct loads into two buffers, diagonal tile
// first; K^T for dQ^T = K^T dS^T comes from transposing reads of the K tile.
// --------------------------------------------------------------------------
constexpr int kDqWaves = 8, kDqThreads = 64 * kDqWaves, kDqRows = 16 * kDqWaves;

// UB gate units per 64-key tile (1: 64-token blocks; 2, 4: 32, 16 tokens).
template <int DS, int UB>
__global__ __launch_bounds__(kDqThreads, 1) void bwd_dq16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ o, const bf16* __restrict__ dout, const float* __restrict__ lse,
    const bf16* __restrict__ qs, const bf16* __restrict__ ks, const float* __restrict__ lam,
    bf16* __restrict__ dq, bf16* __restrict__ dqs, float* __restrict__ dz,
    float* __restrict__ rowd, int tqp, Dims D, int nqt, int xcd_groups) {
  constexpr int HD = 128, TE = kBlock * 144;  // tile elements (72-dword rows)
  constexpr int NCH = kBlock * 16 / kDqThreads;  // 16-byte chunks per thread and tensor
  constexpr int DQ = DS / 4;                   // selector dims per lane group
  __shared__ __align__(16) bf16 K0[TE];
  __shared__ __align__(16) bf16 K1[TE];
  __shared__ __align__(16) bf16 V0[TE];
  __shared__ __align__(16) bf16 V1[TE];
  __shared__ __align__(16) bf16 S0[UB * DS];
  __shared__ __align__(16) bf16 S1[UB * DS];
  constexpr int BU = kBlock / UB;  // tokens per gate unit

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, g4 = lane >> 4;
  const int k4 = i16 >> 2, a4 = i16 & 3;
  const QTile tm = map_q_tile(blockIdx.x, nqt, D, xcd_groups);
  const int b = tm.b, h = tm.h, qt = tm.qt;
  const int g = h / D.hpg, sh = h / D.hps;
  const int wq0 = qt * kDqRows + wave * 16;
  const int qi = wq0 + i16;
  const bool valid = qi < D.tq;
  const int qc = min(qi, D.tq - 1);
  const int t = D.qoff + qc;
  const int c = t / BU;       // historical units of the row
  const int ct = t / kBlock;  // the row's own 64-key tile
  const int c_lo = (D.qoff + min(wq0, D.tq - 1)) / kBlock;
  const int c_hi = (D.qoff + min(wq0 + 15, D.tq - 1)) / kBlock;
  const int c_end = (D.qoff + min(qt * kDqRows + kDqRows - 1, D.tq - 1)) / kBlock;
  const size_t row = ((size_t)b * D.hq + h) * D.tq + qc;

  // zero dz[row, j] for j >= c(row) (coalesced over the workgroup's rows)
  for (int r = 0; r < kDqRows; ++r) {
    const int i = qt * kDqRows + r;
    if (i >= D.tq) break;
    const int cr = (D.qoff + i) / BU;
    float* zr = dz + (((size_t)b * D.hq + h) * D.tq + i) * D.nb;
    for (int jj = cr + tid; jj < D.nb; jj += kDqThreads) zr[jj] = 0.f;
  }

  bf16x8 qf[4], df[4];
  float dlt = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    qf[s] = *(const bf16x8*)(q + row * HD + 32 * s + 8 * g4);
    df[s] = *(const bf16x8*)(dout + row * HD + 32 * s + 8 * g4);
    const bf16x8 of = *(const bf16x8*)(o + row * HD + 32 * s + 8 * g4);
#pragma unroll
    for (int e = 0; e < 8; ++e) dlt = fmaf(to_f32(df[s][e]), to_f32(of[e]), dlt);
  }
  dlt += __shfl_xor(dlt, 16);
  dlt += __shfl_xor(dlt, 32);
  // Row data for the dK/dV kernel, unit-major so that the rows of one unit
  // are contiguous: slot u < nb holds, for each row, the log2-domain offset
  // of unit u's logits (gate bias minus the row's log-sum-exp; -inf past the
  // row's own unit), slot nb the row's D; rows padded to tqp (padding: -inf,
  // D 0).  The offsets are the ones this kernel applies itself.
  const size_t rbase = ((size_t)b * D.hq + h) * (size_t)(D.nb + 1) * tqp + qi;
  const bool rw = g4 == 0 && qi < tqp;
  if (rw) rowd[rbase + (size_t)D.nb * tqp] = valid ? dlt : 0.f;
  float qsv[DQ], dqsa[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) {
    qsv[e] = to_f32(qs[row * DS + g4 * DQ + e]);
    dqsa[e] = 0.f;
  }
  const float lam_t = c > 0 ? lam[row] : 0.f;
  const float l2 = lse[row] * kLog2e;
  const bf16* ksb = ks + ((size_t)b * D.hks + sh) * (size_t)D.nb * DS;
  const bf16* kb = k + ((size_t)b * D.hkv + g) * (size_t)D.tk * HD;
  const bf16* vb = v + ((size_t)b * D.hkv + g) * (size_t)D.tk * HD;
  const float c1 = D.sm_scale * kLog2e;
  f32x4 dqa[8];
#pragma unroll
  for (int dm = 0; dm < 8; ++dm) dqa[dm] = f32x4{};
  float sdb = 0.f;

  // the next tile goes global -> registers at the start of a step and
  // registers -> LDS at its end: thread tid holds 16-byte chunks
  // tid + kDqThreads x of K and V (row = chunk / 16), threads 0 .. DS/8-1 a
  // chunk of the block's ks row
  bf16x8 kreg[NCH], vreg[NCH], sreg = bf16x8{};
  auto gload = [&](int j) {
    const bf16* kt = kb + (size_t)j * kBlock * HD;
    const bf16* vt = vb + (size_t)j * kBlock * HD;
#pragma unroll
    for (int x = 0; x < NCH; ++x) {
      const int id = tid + kDqThreads * x;
      kreg[x] = *(const bf16x8*)(kt + (id >> 4) * HD + (id & 15) * 8);
      vreg[x] = *(const bf16x8*)(vt + (id >> 4) * HD + (id & 15) * 8);
    }
    if (tid < UB * DS / 8) sreg = *(const bf16x8*)(ksb + (size_t)j * UB * DS + tid * 8);
  };
  auto sstore = [&](bf16* Kd, bf16* Vd, bf16* Sd) {
#pragma unroll
    for (int x = 0; x < NCH; ++x) {
      const int id = tid + kDqThreads * x;
      *(bf16x8*)&Kd[trow(id >> 4) + (id & 15) * 8] = kreg[x];
      *(bf16x8*)&Vd[trow(id >> 4) + (id & 15) * 8] = vreg[x];
    }
    if (tid < UB * DS / 8) *(bf16x8*)&Sd[tid * 8] = sreg;
  };

  auto compute = [&](int j, const bf16* Ks, const bf16* Vs, const bf16* Ss) {
    if (j > c_hi) return;
    float bias2[UB];
    float ksv[UB][DQ];
#pragma unroll
    for (int ub = 0; ub < UB; ++ub) {
      bias2[ub] = 0.f;
#pragma unroll
      for (int e = 0; e < DQ; ++e) ksv[ub][e] = to_f32(Ss[ub * DS + g4 * DQ + e]);
    }
    if (UB == 1 ? j < c_hi : j <= c_hi) {
#pragma unroll
      for (int ub = 0; ub < UB; ++ub) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < DQ; ++e) part = fmaf(qsv[e], ksv[ub][e], part);
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        if (j * UB + ub < c) bias2[ub] = (D.sel_scale * part - lam_t) * kLog2e;
      }
    }
    if (rw) {
#pragma unroll
      for (int ub = 0; ub < UB; ++ub) {
        const int ju = j * UB + ub;
        rowd[rbase + (size_t)ju * tqp] = valid && ju <= c ? bias2[ub] - l2 : -INFINITY;
      }
    }
    // unit of this lane's keys 16 mk + 4 g4 + r within the tile
    auto unit = [](int mk) { return UB == 1 ? 0 : (UB == 2 ? mk / 2 : mk); };
    f32x4 sacc[4], pacc[4];
#pragma unroll
    for (int mk = 0; mk < 4; ++mk) {
      sacc[mk] = f32x4{};
      pacc[mk] = f32x4{};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int mk = 0; mk < 4; ++mk) {
        const int oo = trow(i16) + 2304 * mk + 32 * s + 8 * g4;
        sacc[mk] = mfma16(*(const bf16x8*)&Ks[oo], qf[s], sacc[mk]);
        pacc[mk] = mfma16(*(const bf16x8*)&Vs[oo], df[s], pacc[mk]);
      }
    }
    float pv[4][4];
#pragma unroll
    for (int mk = 0; mk < 4; ++mk)
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[mk][r] = exp2_raw(fmaf(sacc[mk][r], c1, bias2[unit(mk)] - l2));
    if (j >= c_lo) {  // tile meets some row's own tile: cut keys after the row (or the tile)
      const int mlim = j < ct ? kBlock : (j > ct ? -1 : t - j * kBlock - 4 * g4);
#pragma unroll
      for (int mk = 0; mk < 4; ++mk)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * mk + r > mlim) pv[mk][r] = 0.f;
    }
    float dsum[UB];
#pragma unroll
    for (int ub = 0; ub < UB; ++ub) dsum[ub] = 0.f;
#pragma unroll
    for (int mk = 0; mk < 4; ++mk) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ds = pv[mk][r] * (pacc[mk][r] - dlt);
        sacc[mk][r] = ds;
        dsum[unit(mk)] += ds;
      }
    }
#pragma unroll
    for (int ub = 0; ub < UB; ++ub) {
      dsum[ub] += __shfl_xor(dsum[ub], 16);
      dsum[ub] += __shfl_xor(dsum[ub], 32);
    }
    if constexpr (UB == 1) {
      if (j == c) {
        sdb = -dsum[0];  // sum_{j'<c} dbeta = - sum over the current block of dS
      } else if (j < c) {
        const float dzv = dsum[0] - exp2_raw(bias2[0]) * sdb;
        if (valid && g4 == 0) dz[row * D.nb + j] = dzv;
#pragma unroll
        for (int e = 0; e < DQ; ++e) dqsa[e] = fmaf(dzv, ksv[0][e], dqsa[e]);
      }
    } else {
      // the row's own tile comes first (tiles run from the diagonal down):
      // its current unit gives sum_{j'<c} dbeta before any historical unit
      if (j == ct) {
#pragma unroll
        for (int ub = 0; ub < UB; ++ub)
          if (j * UB + ub == c) sdb = -dsum[ub];
      }
#pragma unroll
      for (int ub = 0; ub < UB; ++ub) {
        if (j * UB + ub < c) {
          const float dzv = dsum[ub] - exp2_raw(bias2[ub]) * sdb;
          if (valid && g4 == 0) dz[row * D.nb + j * UB + ub] = dzv;
#pragma unroll
          for (int e = 0; e < DQ; ++e) dqsa[e] = fmaf(dzv, ksv[ub][e], dqsa[e]);
        }
      }
    }
    // dQ^T += K^T dS^T over two 32-key steps; B slots: keys 32ks + 4g4 + r, +16
#pragma unroll
    for (int kst = 0; kst < 2; ++kst) {
      bf16x8 sb;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sb[r] = (bf16)sacc[2 * kst][r];
        sb[4 + r] = (bf16)sacc[2 * kst + 1][r];
      }
      const int t0 = trow(4 * g4 + k4) + 4608 * kst + 4 * a4, t1 = t0 + 2304;
#pragma unroll
      for (int dm = 0; dm < 8; ++dm) {
        const bf16x4 lo = ds_read_tr(&Ks[t0 + 16 * dm]);
        const bf16x4 hi = ds_read_tr(&Ks[t1 + 16 * dm]);
        dqa[dm] = mfma16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), sb, dqa[dm]);
      }
    }
  };

  const int ntiles = c_end + 1;  // tiles c_end, c_end - 1, ..., 0
  gload(c_end);
  sstore(K0, V0, S0);
  __syncthreads();
  for (int it = 0; it < ntiles; it += 2) {
    if (it + 1 < ntiles) gload(c_end - it - 1);
    compute(c_end - it, K0, V0, S0);
    if (it + 1 < ntiles) sstore(K1, V1, S1);
    __syncthreads();
    if (it + 1 >= ntiles) break;
    if (it + 2 < ntiles) gload(c_end - it - 2);
    compute(c_end - it - 1, K1, V1, S1);
    if (it + 2 < ntiles) sstore(K0, V0, S0);
    __syncthreads();
  }

  if (valid) {
    bf16* qr = dq + row * HD + 4 * g4;
#pragma unroll
    for (int dm = 0; dm < 8; ++dm) {
      bf16x4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = (bf16)(dqa[dm][r] * D.sm_scale);
      *(bf16x4*)(qr + 16 * dm) = w;
    }
#pragma unroll
    for (int e = 0; e < DQ; ++e) dqs[row * DS + g4 * DQ + e] = (bf16)(dqsa[e] * D.sel_scale);
  }
}

// --------------------------------------------------------------------------
// Query-stationary dQ, D, dz, dqs for d = 128 on 32x32x16 MFMA tiles: a
// workgroup owns 256 query rows, each wave 32 (two waves per SIMD).  Each K,
// V or K^T operand read from LDS feeds 32 query columns, so the LDS bytes per
// product are about 0.6 of the 16-row kernel's (whose Q sits in registers).
// The query sits in the MFMA column: D, the dS
// row sums and the selector terms are per-lane values plus one exchange
// between the two 32-lane halves.  Q sits in LDS, dO in registers.  64-key K
// and V tiles (and the ks rows of the tile's units) arrive by direct global ->
// LDS loads into two buffers, diagonal tile first; K^T for dQ^T = K^T dS^T
// comes from transposing reads in the key order of the dS^T operand slots.
// --------------------------------------------------------------------------
constexpr int kDq32Waves = 8, kDq32Threads = 64 * kDq32Waves, kDq32Rows = 32 * kDq32Waves;

template <int DS, int UB>
__global__ __launch_bounds__(kDq32Threads, 1) void bwd_dq32_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ o, const bf16* __restrict__ dout, const float* __restrict__ lse,
    const bf16* __restrict__ qs, const bf16* __restrict__ ks, const float* __restrict__ lam,
    bf16* __restrict__ dq, bf16* __restrict__ dqs, float* __restrict__ dz,
    float* __restrict__ rowd, int tqp, Dims D, int nqt, int xcd_groups) {
  constexpr int HD = 128, KP = 144, TE = kBlock * KP;  // 72-dword LDS rows
  constexpr int NI = TE / 512;                         // 1 KB direct loads per tile and tensor
  constexpr int XI = (NI + kDq32Waves - 1) / kDq32Waves;
  constexpr int DH = DS / 2;                           // selector dims per lane half
  constexpr int BU = UB > 0 ? kBlock / UB : 1;         // tokens per gate unit (UB > 0)
  // UB = 0 (units of D.blk = 1 .. 8 tokens): the tile's 64 per-key ks rows
  // (each key's unit row, expanded beforehand) sit in LDS, XS 16-byte slots
  // per row (one padding slot), read as Z^T operands and transposed for dqs
  constexpr int XS = DS / 8 + 1, XP = XS * 8;
  constexpr int SN = UB > 0 ? UB * DS : kBlock * XP;
  static_assert(UB > 0 || DS == 32, "token units: ds = 32 (five waves load the ks tile)");
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  __shared__ __align__(16) bf16 K0[TE];
  __shared__ __align__(16) bf16 K1[TE];
  __shared__ __align__(16) bf16 V0[TE];
  __shared__ __align__(16) bf16 V1[TE];
  __shared__ __align__(16) bf16 S0[SN];
  __shared__ __align__(16) bf16 S1[SN];
  __shared__ __align__(16) bf16 Qs[kDq32Rows * KP];  // the workgroup's Q rows

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const QTile tm = map_q_tile(blockIdx.x, nqt, D, xcd_groups);
  const int b = tm.b, h = tm.h, qt = tm.qt;
  const int g = h / D.hpg, sh = h / D.hps;
  const int wq0 = qt * kDq32Rows + wave * 32;
  const int qi = wq0 + l32;
  const bool valid = qi < D.tq;
  const int qc = min(qi, D.tq - 1);
  const int t = D.qoff + qc;
  const int lb = __builtin_ctz(UB > 0 ? BU : D.blk);  // log2 of the unit size
  const int c = t >> lb;       // historical units of the row
  const int tcur0 = c << lb;   // first key of the row's own unit
  const int ct = t / kBlock;  // the row's own 64-key tile
  const int c_lo = (D.qoff + min(wq0, D.tq - 1)) / kBlock;
  const int c_hi = (D.qoff + min(wq0 + 31, D.tq - 1)) / kBlock;
  const int c_end = (D.qoff + min(qt * kDq32Rows + kDq32Rows - 1, D.tq - 1)) / kBlock;
  const size_t row = ((size_t)b * D.hq + h) * D.tq + qc;

  // zero dz[row, j] for j >= c(row) (coalesced over the workgroup's rows);
  // UB = 0 writes dz only when the caller asks for it
  if (UB > 0 || dz != nullptr) {
    for (int r = 0; r < kDq32Rows; ++r) {
      const int i = qt * kDq32Rows + r;
      if (i >= D.tq) break;
      const int cr = (D.qoff + i) >> lb;
      float* zr = dz + (((size_t)b * D.hq + h) * D.tq + i) * D.nb;
      for (int jj = cr + tid; jj < D.nb; jj += kDq32Threads) zr[jj] = 0.f;
    }
  }

  // Q and dO as B operands (lane: query l32, dims 16 s + 8 hh .. + 7): dO in
  // registers, Q in LDS (each lane reads back only what it wrote), which
  // leaves the registers for two waves per SIMD
  const int qbase = (32 * wave + l32) * KP + 8 * hh;
  bf16x8 df[8];
  float dlt = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    *(bf16x8*)&Qs[qbase + 16 * s] = *(const bf16x8*)(q + row * HD + 16 * s + 8 * hh);
    df[s] = *(const bf16x8*)(dout + row * HD + 16 * s + 8 * hh);
    const bf16x8 of = *(const bf16x8*)(o + row * HD + 16 * s + 8 * hh);
#pragma unroll
    for (int e = 0; e < 8; ++e) dlt = fmaf(to_f32(df[s][e]), to_f32(of[e]), dlt);
  }
  dlt = halves_sum(dlt);
  // Row data for the dK/dV kernel, unit-major so that the rows of one unit
  // are contiguous: slot u < nb holds, for each row, the log2-domain offset
  // of unit u's logits (gate bias minus the row's log-sum-exp; -inf past the
  // row's own unit), slot nb the row's D; rows padded to tqp (padding: -inf,
  // D 0).  The offsets are the ones this kernel applies itself.
  // UB = 0: four slots per row instead (written at the end): lam log2 e,
  // lse log2 e (+inf for padding rows), D, and sum_j dbeta / blk.
  const size_t rbase = ((size_t)b * D.hq + h) * (size_t)(UB > 0 ? D.nb + 1 : 4) * tqp + qi;
  const bool rw = hh == 0 && qi < tqp;
  if (UB > 0 && rw) rowd[rbase + (size_t)D.nb * tqp] = valid ? dlt : 0.f;
  // this lane's half of the row's qs as bf16 pairs (packed dot products, as
  // in the forward), and its half of the dqs accumulator
  bf16x2 qsv[DS / 4];
  float dqsa[DH];
#pragma unroll
  for (int e = 0; e < DS / 4; ++e) qsv[e] = *(const bf16x2*)(qs + row * DS + hh * DH + 2 * e);
#pragma unroll
  for (int e = 0; e < DH; ++e) dqsa[e] = 0.f;
  const float lam_t = c > 0 ? lam[row] : 0.f;
  const float l2 = lse[row] * kLog2e;
  // UB > 0: ks rows of the selector head; UB = 0: the per-key rows [tk][DS]
  const bf16* ksb = ks + ((size_t)b * D.hks + sh) * (size_t)(UB > 0 ? D.nb : D.tk) * DS;
  // UB = 0: the row's qs as Z^T B operands, the dqs^T accumulator, and the
  // log2-domain selector constants
  bf16x8 qsf[UB == 0 ? DS / 16 : 1];
  f32x16 dqsz[UB == 0 ? DS / 32 : 1];
  if constexpr (UB == 0) {
#pragma unroll
    for (int s = 0; s < DS / 16; ++s) qsf[s] = *(const bf16x8*)(qs + row * DS + 16 * s + 8 * hh);
#pragma unroll
    for (int x = 0; x < DS / 32; ++x) dqsz[x] = f32x16{};
  }
  const float zs2 = D.sel_scale * kLog2e, lam2 = lam_t * kLog2e;
  const float inv_blk = 1.f / (float)(1 << lb);
  const bf16* kb = k + ((size_t)b * D.hkv + g) * (size_t)D.tk * HD;
  const bf16* vb = v + ((size_t)b * D.hkv + g) * (size_t)D.tk * HD;
  const float c1 = D.sm_scale * kLog2e;
  f32x16 dqa[4];
#pragma unroll
  for (int dm = 0; dm < 4; ++dm) dqa[dm] = f32x16{};
  float sdb = 0.f;

  // Tiles go global -> LDS by direct loads: 1 KB instruction ins = wave +
  // kDq32Waves x fills LDS slots 64 ins .. 64 ins + 63 of K and of V (18
  // 16-byte slots per row, the two padding slots reloading chunk 0); wave 0
  // loads the ks rows of the tile's units.
  unsigned toff[XI];
#pragma unroll
  for (int x = 0; x < XI; ++x)
    toff[x] = 2 * tslot_src(min((wave + kDq32Waves * x) * 64 + lane, kBlock * 18 - 1));
  auto issue = [&](int j, bf16* Kd, bf16* Vd, bf16* Sd) {
    const char* const kt = (const char*)(kb + (size_t)j * kBlock * HD);
    const char* const vt = (const char*)(vb + (size_t)j * kBlock * HD);
#pragma unroll
    for (int x = 0; x < XI; ++x) {
      const int ins = wave + kDq32Waves * x;
      if (ins < NI) {
        __builtin_amdgcn_global_load_lds(kt + toff[x], Kd + ins * 512, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vt + toff[x], Vd + ins * 512, 16, 0, 0);
      }
    }
    if constexpr (UB == 0) {
      // slot s = 64 wave + lane: key row s / XS, chunk s % XS (the padding
      // chunk reloads chunk 0)
      if (wave < XS) {
        const int sl = 64 * wave + lane, kr = sl / XS, ch = sl % XS;
        const bf16* const src = ksb + ((size_t)j * kBlock + kr) * DS + (ch < DS / 8 ? ch : 0) * 8;
        __builtin_amdgcn_global_load_lds(src, Sd + wave * 512, 16, 0, 0);
      }
    } else if (wave == 0 && lane < UB * DS / 8) {
      const bf16* const src = ksb + (size_t)j * UB * DS + lane * 8;
      __builtin_amdgcn_global_load_lds(src, Sd, 16, 0, 0);
    }
  };
  // per-lane part of the transposing K^T reads: lane 4 kk + a of each 16-lane
  // group points at key row 4 hh + kk, columns 16 ((lane >> 4) & 1) + 4 a
  const int kbase = (2 * ((lane & 15) >> 2) + hh) * KP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // key row supplied as A-operand row l32 of the S^T / dP^T products: keys
  // 8 q + 2 i + hh sit in accumulator rows 8 q + 4 hh + i, so that a
  // transposing read gives each lane half rows of one parity
  const int prow = (l32 & ~7) | ((l32 & 3) << 1) | ((l32 >> 2) & 1);
  // unit of this lane's key 32 mt + 8 (r / 4) + 2 (r % 4) + hh within the tile
  auto unit = [](int mt, int r) { return UB <= 1 ? 0 : (UB == 2 ? mt : 2 * mt + r / 8); };
  // UB = 0: the same transposing reads over the per-key ks rows (pitch XP)
  const int xbase = (2 * ((lane & 15) >> 2) + hh) * XP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // UB = 0, dz requested: dz[row, unit] = sum of e over the unit's keys.  A
  // lane half holds the keys of one parity of each group of 8 (32 mt + 8 q +
  // hh + 2 i); units of 2 or more keys join the two halves.
  auto write_dz_units = [&](const f32x16 (&e)[2], int j, size_t rw_, bool ok) {
    // element (mt, 4 q + i) of lane half hh is key 32 mt + 8 q + 2 i + hh
    const int bsz = 1 << lb;
    float* zr = dz + rw_ * D.nb;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int k0 = j * kBlock + 32 * mt + 8 * q4;  // first key of the group of 8
        float er[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) er[i] = e[mt][4 * q4 + i];
        if (bsz == 1) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (ok && k0 + 2 * i + hh < tcur0) zr[k0 + 2 * i + hh] = er[i];
        } else if (bsz == 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = halves_sum(er[i]);
            if (ok && hh == 0 && k0 + 2 * i < tcur0) zr[(k0 + 2 * i) >> 1] = v;
          }
        } else if (bsz == 4) {
          float v0 = er[0] + er[1], v1 = er[2] + er[3];
          v0 = halves_sum(v0);
          v1 = halves_sum(v1);
          if (ok && hh == 0 && k0 < tcur0) zr[k0 >> 2] = v0;
          if (ok && hh == 0 && k0 + 4 < tcur0) zr[(k0 >> 2) + 1] = v1;
        } else {
          float v = er[0] + er[1] + er[2] + er[3];
          v = halves_sum(v);
          if (ok && hh == 0 && k0 < tcur0) zr[k0 >> 3] = v;
        }
      }
    }
  };

  auto compute = [&](int j, const bf16* Ks, const bf16* Vs, const bf16* Ss) {
    if (j > c_hi) return;
    constexpr int NU = UB > 0 ? UB : 1;
    float bias2[NU];
#pragma unroll
    for (int ub = 0; ub < NU; ++ub) bias2[ub] = 0.f;
    // UB = 0: Z^T = KS QS^T of the tile (selector scores of each (key, row))
    auto zt = [&](f32x16 (&za)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < DS / 16; ++s) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x8 a = *(const bf16x8*)&Ss[(32 * mt + prow) * XP + 16 * s + 8 * hh];
          za[mt] = mfma32(a, qsf[s], za[mt]);
        }
      }
    };
    if constexpr (UB == 0) {
    } else if (UB == 1 ? j < c_hi : j <= c_hi) {
#pragma unroll
      for (int ub = 0; ub < UB; ++ub) {
        const bf16x2* kr = (const bf16x2*)(Ss + ub * DS + hh * DH);
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < DS / 4; ++e)
          part = __builtin_amdgcn_fdot2_f32_bf16(qsv[e], kr[e], part, false);
        part = halves_sum(part);
        if (j * UB + ub < c) bias2[ub] = (D.sel_scale * part - lam_t) * kLog2e;
      }
    }
    if (UB > 0 && rw) {
#pragma unroll
      for (int ub = 0; ub < NU; ++ub) {
        const int ju = j * UB + ub;
        rowd[rbase + (size_t)ju * tqp] = valid && ju <= c ? bias2[ub] - l2 : -INFINITY;
      }
    }
    // S^T and dP^T: two 32-key M-tiles x 32 queries each
    f32x16 sacc[2] = {f32x16{}, f32x16{}}, pacc[2] = {f32x16{}, f32x16{}};
    if constexpr (UB == 0) {
      // a historical key's logit is sm_scale (s + (sel_scale z - lam) / sm_scale):
      // its S accumulator starts at the second term (keys of the row's own
      // unit and later ones at 0), so that no bias array stays live through
      // the products
      zt(sacc);
      const float zsc = D.sel_scale / D.sm_scale, zoff = -lam_t / D.sm_scale;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int u = j * kBlock + 32 * mt + 8 * (r / 4) + 2 * (r % 4) + hh;
          sacc[mt][r] = u < tcur0 ? fmaf(sacc[mt][r], zsc, zoff) : 0.f;
        }
      }
    }
    // operand i (step i / 4, M-tile (i / 2) % 2, K or V by i % 2) is read
    // while product i - 1 runs; the step's Q operand after its last use
    auto opnd = [&](int i) __attribute__((always_inline)) {
      const int oo = (32 * ((i >> 1) & 1) + prow) * KP + 16 * (i >> 2) + 8 * hh;
      return *(const bf16x8*)&((i & 1) ? Vs : Ks)[oo];
    };
    bf16x8 ob[2], qb = *(const bf16x8*)&Qs[qbase];
    ob[0] = opnd(0);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i < 31) ob[(i + 1) & 1] = opnd(i + 1);
      if ((i & 3) == 3 && i < 31) qb = *(const bf16x8*)&Qs[qbase + 16 * ((i >> 2) + 1)];
      const int s = i >> 2, mt = (i >> 1) & 1;
      if (i & 1)
        pacc[mt] = mfma32(ob[i & 1], df[s], pacc[mt]);
      else
        sacc[mt] = mfma32(ob[i & 1], qb, sacc[mt]);
    }
    float pv[2][16];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        pv[mt][r] = exp2_raw(fmaf(sacc[mt][r], c1, (UB == 0 ? 0.f : bias2[unit(mt, r)]) - l2));
    if (j >= c_lo) {  // tile meets some row's own tile: cut keys after the row (or the tile)
      const int mlim = j < ct ? kBlock : (j > ct ? -1 : t - j * kBlock - hh);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * mt + 8 * (r / 4) + 2 * (r % 4) > mlim) pv[mt][r] = 0.f;
    }
    float dsum[NU];
#pragma unroll
    for (int ub = 0; ub < NU; ++ub) dsum[ub] = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float ds = pv[mt][r] * (pacc[mt][r] - dlt);
        sacc[mt][r] = ds;
        if constexpr (UB == 0) {
          // the row's own unit (keys tcur0 .. t; later keys have ds = 0)
          const int u = j * kBlock + 32 * mt + 8 * (r / 4) + 2 * (r % 4) + hh;
          if (u >= tcur0) dsum[0] += ds;
        } else {
          dsum[unit(mt, r)] += ds;
        }
      }
    }
#pragma unroll
    for (int ub = 0; ub < NU; ++ub) dsum[ub] = halves_sum(dsum[ub]);
    // the row's own tile comes first (tiles run from the diagonal down): its
    // current unit gives sum_{j'<c} dbeta before any historical unit
    if (j == ct) {
      if constexpr (UB == 0) {
        sdb = -dsum[0];
      } else {
#pragma unroll
        for (int ub = 0; ub < NU; ++ub)
          if (j * UB + ub == c) sdb = -dsum[ub];
      }
    }
    if constexpr (UB == 0) {
      // e = dS - g sdb / blk on historical keys (0 elsewhere): summed over a
      // unit's keys it is dz; dqs^T += KS^T e^T over the tile's keys
      // (Z^T again, now that dP's registers are free: the gate g = 2^(z log2 e
      // sel_scale - lam log2 e))
      const float sb_k = sdb * inv_blk;
      f32x16 zb[2] = {f32x16{}, f32x16{}};
      zt(zb);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int u = j * kBlock + 32 * mt + 8 * (r / 4) + 2 * (r % 4) + hh;
          zb[mt][r] =
              u < tcur0 ? sacc[mt][r] - exp2_raw(fmaf(zb[mt][r], zs2, -lam2)) * sb_k : 0.f;
        }
      }
      if (dz != nullptr) write_dz_units(zb, j, row, valid);
      // e enters as a bf16 pair (e_hi + e_lo: 16 mantissa bits), so that dqs
      // keeps fp32-like accuracy where its terms cancel
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          bf16x8 eh, el;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            eh[e] = (bf16)zb[mt][8 * pp + e];
            el[e] = (bf16)(zb[mt][8 * pp + e] - (float)eh[e]);
          }
#pragma unroll
          for (int x = 0; x < DS / 32; ++x) {
            const bf16* xp = &Ss[xbase + (32 * mt + 16 * pp) * XP + 32 * x];
            const bf16x4 lo = ds_read_tr(xp);
            const bf16x4 hi = ds_read_tr(xp + 8 * XP);
            const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            dqsz[x] = mfma32(a, eh, dqsz[x]);
            dqsz[x] = mfma32(a, el, dqsz[x]);
          }
        }
      }
    }
#pragma unroll
    for (int ub = 0; ub < (UB > 0 ? UB : 0); ++ub) {
      if (j * UB + ub < c) {
        const float dzv = dsum[ub] - exp2_raw(bias2[ub]) * sdb;
        if (valid && hh == 0) dz[row * D.nb + j * UB + ub] = dzv;
        const bf16x2* kr = (const bf16x2*)(Ss + ub * DS + hh * DH);
#pragma unroll
        for (int e = 0; e < DS / 4; ++e) {
          const bf16x2 kv = kr[e];
          dqsa[2 * e] = fmaf(dzv, to_f32(kv[0]), dqsa[2 * e]);
          dqsa[2 * e + 1] = fmaf(dzv, to_f32(kv[1]), dqsa[2 * e + 1]);
        }
      }
    }
    // dQ^T += K^T dS^T: the B slots of a lane are keys 16 pp + hh + 2 (0..3)
    // and 16 pp + 8 + hh + 2 (0..3) of M-tile mt, and the transposing reads
    // give K^T in that order
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        bf16x8 sb;
#pragma unroll
        for (int e = 0; e < 8; ++e) sb[e] = (bf16)sacc[mt][8 * pp + e];
#pragma unroll
        for (int dm = 0; dm < 4; ++dm) {
          const bf16* kp = &Ks[kbase + (32 * mt + 16 * pp) * KP + 32 * dm];
          const bf16x4 lo = ds_read_tr(kp);
          const bf16x4 hi = ds_read_tr(kp + 8 * KP);
          dqa[dm] = mfma32(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), sb, dqa[dm]);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  const int ntiles = c_end + 1;  // tiles c_end, c_end - 1, ..., 0
  issue(c_end, K0, V0, S0);
  wait_vmem();
  __syncthreads();
  for (int it = 0; it < ntiles; it += 2) {
    if (it + 1 < ntiles) issue(c_end - it - 1, K1, V1, S1);
    compute(c_end - it, K0, V0, S0);
    wait_vmem();
    __syncthreads();
    if (it + 1 >= ntiles) break;
    if (it + 2 < ntiles) issue(c_end - it - 2, K0, V0, S0);
    compute(c_end - it - 1, K1, V1, S1);
    wait_vmem();
    __syncthreads();
  }

  if (valid) {
    bf16* qr = dq + row * HD + 4 * hh;
#pragma unroll
    for (int dm = 0; dm < 4; ++dm) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(dqa[dm][4 * rr + e] * D.sm_scale);
        *(bf16x4*)(qr + 32 * dm + 8 * rr) = w;
      }
    }
    if constexpr (UB == 0) {
      bf16* sr = dqs + row * DS + 4 * hh;
#pragma unroll
      for (int x = 0; x < DS / 32; ++x) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (bf16)(dqsz[x][4 * rr + e] * D.sel_scale);
          *(bf16x4*)(sr + 32 * x + 8 * rr) = w;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < DH; ++e) dqs[row * DS + hh * DH + e] = (bf16)(dqsa[e] * D.sel_scale);
    }
  }
  if (UB == 0 && rw) {
    const size_t sl = (size_t)tqp;
    rowd[rbase] = valid ? lam2 : 0.f;
    rowd[rbase + sl] = valid ? l2 : INFINITY;
    rowd[rbase + 2 * sl] = valid ? dlt : 0.f;
    rowd[rbase + 3 * sl] = valid ? sdb * inv_blk : 0.f;
  }
}

// --------------------------------------------------------------------------
// Key-stationary: dK, dV.
// --------------------------------------------------------------------------
template <int HD, int DS>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, const bf16* __restrict__ qs, const bf16* __restrict__ ks,
    const float* __restrict__ lam, bf16* __restrict__ dk, bf16* __restrict__ dv, Dims D,
    int nkt, int xcd_groups) {
  constexpr int KP = HD + 8;
  constexpr int TP = 64 + 8;
  constexpr int KS = HD / 16;
  constexpr int DM = HD / 32;
  constexpr int ITEMS = 16 * (HD / 8);  // (4 rows x 8 dims) items per 64-row tile
  constexpr int IT = (ITEMS + 255) / 256;
  __shared__ __align__(16) bf16 Qs[64 * KP];
  __shared__ __align__(16) bf16 Os[64 * KP];  // dO rows
  __shared__ __align__(16) bf16 Qt[HD * TP];
  __shared__ __align__(16) bf16 Ot[HD * TP];  // dO^T
  __shared__ __align__(16) float offs[2][64];  // log2 offset of (block, row)
  __shared__ __align__(16) float dls[64];      // D of row

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, hh = lane >> 5;
  // work item: (b, kv head g, key tile kt), key tiles issued longest first
  int b, g, kt;
  {
    const int L = blockIdx.x;
    if (xcd_groups > 0) {
      const int xcd = L & 7, s = L >> 3;
      const int rank = s / xcd_groups, gi = s % xcd_groups;
      const int G = gi * 8 + xcd;
      b = G / D.hkv;
      g = G % D.hkv;
      kt = rank;
    } else {
      const int bg = D.batch * D.hkv;
      kt = L / bg;
      b = (L % bg) / D.hkv;
      g = L % D.hkv;
    }
  }
  const int kbase = kt * 128;
  const int key = kbase + wave * 32 + l32;  // this lane's key (column)
  const int blk0 = kbase / kBlock;          // first of the two blocks
  const int wblk = wave >> 1;               // this wave's block (0/1 within the tile)
  const bool key_ok = key < D.tk;
  const size_t kvrow = ((size_t)b * D.hkv + g) * D.tk + (key_ok ? key : D.tk - 1);

  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    kf[s] = *(const bf16x8*)(k + kvrow * HD + 16 * s + 8 * hh);
    vf[s] = *(const bf16x8*)(v + kvrow * HD + 16 * s + 8 * hh);
  }
  f32x16 dkacc[DM], dvacc[DM];
#pragma unroll
  for (int dm = 0; dm < DM; ++dm) {
    dkacc[dm] = f32x16{};
    dvacc[dm] = f32x16{};
  }
  const float c1 = D.sm_scale * kLog2e;
  const int i_first = max(0, kbase - D.qoff);  // first row that can see a key of the tile
  const int qt0 = i_first / 64;
  const int nqt64 = (D.tq + 63) / 64;
  const int n_items = D.hpg * (nqt64 - qt0);
  if (kbase >= D.tk) return;

  const bf16x8 zero8 = bf16x8{};
  bf16x8 qreg[IT][4], oreg[IT][4];
  auto gload = [&](int it) {
    const int hl = it / (nqt64 - qt0), qtile = qt0 + it % (nqt64 - qt0);
    const int h = g * D.hpg + hl;
    const size_t base = ((size_t)b * D.hq + h) * D.tq;
#pragma unroll
    for (int x = 0; x < IT; ++x) {
      const int id = tid + 256 * x;
      if (id < ITEMS) {
        const int rg = id % 16, dc = id / 16;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          const int i = qtile * 64 + rg * 4 + i2;
          const bool in = i < D.tq;
          qreg[x][i2] = in ? *(const bf16x8*)(q + (base + i) * HD + dc * 8) : zero8;
          oreg[x][i2] = in ? *(const bf16x8*)(dout + (base + i) * HD + dc * 8) : zero8;
        }
      }
    }
  };
  auto sstore = [&](int it) {
#pragma unroll
    for (int x = 0; x < IT; ++x) {
      const int id = tid + 256 * x;
      if (id < ITEMS) {
        const int rg = id % 16, dc = id / 16;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          *(bf16x8*)&Qs[(rg * 4 + i2) * KP + dc * 8] = qreg[x][i2];
          *(bf16x8*)&Os[(rg * 4 + i2) * KP + dc * 8] = oreg[x][i2];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bf16x4 w = {qreg[x][0][e], qreg[x][1][e], qreg[x][2][e], qreg[x][3][e]};
          *(bf16x4*)&Qt[(dc * 8 + e) * TP + rg * 4] = w;
          bf16x4 w2 = {oreg[x][0][e], oreg[x][1][e], oreg[x][2][e], oreg[x][3][e]};
          *(bf16x4*)&Ot[(dc * 8 + e) * TP + rg * 4] = w2;
        }
      }
    }
    // per-row offsets for the two blocks of this key tile, and D
    const int hl = it / (nqt64 - qt0), qtile = qt0 + it % (nqt64 - qt0);
    const int h = g * D.hpg + hl;
    if (tid < 128) {
      const int r = tid & 63, bl = tid >> 6;
      const int i = qtile * 64 + r;
      const int blk = blk0 + bl;
      float off = -INFINITY;
      if (i < D.tq && blk < D.nb) {
        const size_t rw = ((size_t)b * D.hq + h) * D.tq + i;
        const int t = D.qoff + i;
        const int c = t / kBlock;
        const float l2 = lse[rw] * kLog2e;
        if (blk == c) {
          off = -l2;
        } else if (blk < c) {
          const bf16* qsr = qs + rw * DS;
          const bf16* ksr = ks + (((size_t)b * D.hks + h / D.hps) * D.nb + blk) * DS;
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < DS; ++e) acc = fmaf(to_f32(qsr[e]), to_f32(ksr[e]), acc);
          off = (D.sel_scale * acc - lam[rw]) * kLog2e - l2;
        }
      }
      offs[bl][r] = off;
    } else if (tid < 192) {
      const int r = tid - 128;
      const int i = qtile * 64 + r;
      dls[r] = i < D.tq ? delta[((size_t)b * D.hq + h) * D.tq + i] : 0.f;
    }
  };

  gload(0);
  for (int it = 0; it < n_items; ++it) {
    __syncthreads();
    sstore(it);
    __syncthreads();
    if (it + 1 < n_items) gload(it + 1);
    const int qtile = qt0 + it % (nqt64 - qt0);
    const int row0 = qtile * 64;
    // skip if every row of the tile is before this wave's keys
    if (D.qoff + min(row0 + 63, D.tq - 1) < kbase + wave * 32) continue;

    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    f32x16 pacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int mq = 0; mq < 2; ++mq) {
        const bf16x8 a = *(const bf16x8*)&Qs[(32 * mq + l32) * KP + 16 * s + 8 * hh];
        sacc[mq] = mfma32(a, kf[s], sacc[mq]);
        const bf16x8 ao = *(const bf16x8*)&Os[(32 * mq + l32) * KP + 16 * s + 8 * hh];
        pacc[mq] = mfma32(ao, vf[s], pacc[mq]);
      }
    }
    const bool nomask = D.qoff + row0 >= kbase + 127;
    auto softmax_ds = [&](auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
      for (int mq = 0; mq < 2; ++mq) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int rb = 32 * mq + r4 * 8 + 4 * hh;  // 4 consecutive rows
          const f32x4 of4 = *(const f32x4*)&offs[wblk][rb];
          const f32x4 dl4 = *(const f32x4*)&dls[rb];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = r4 * 4 + e;
            float p = exp2_raw(fmaf(sacc[mq][r], c1, of4[e]));
            if constexpr (MASK) {
              if (key > D.qoff + row0 + rb + e) p = 0.f;
            }
            sacc[mq][r] = p;
            pacc[mq][r] = p * (pacc[mq][r] - dl4[e]);
          }
        }
      }
    };
    if (nomask)
      softmax_ds(std::false_type{});
    else
      softmax_ds(std::true_type{});
    // dV^T += dO^T P ;  dK^T += Q^T dS
#pragma unroll
    for (int mq = 0; mq < 2; ++mq) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        bf16x8 pb, sb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[e] = (bf16)sacc[mq][8 * pp + e];
          sb[e] = (bf16)pacc[mq][8 * pp + e];
        }
#pragma unroll
        for (int dm = 0; dm < DM; ++dm) {
          const int off = (32 * dm + l32) * TP + 32 * mq + 16 * pp + 4 * hh;
          const bf16x4 olo = *(const bf16x4*)&Ot[off];
          const bf16x4 ohi = *(const bf16x4*)&Ot[off + 8];
          dvacc[dm] = mfma32(__builtin_shufflevector(olo, ohi, 0, 1, 2, 3, 4, 5, 6, 7), pb,
                             dvacc[dm]);
          const bf16x4 qlo = *(const bf16x4*)&Qt[off];
          const bf16x4 qhi = *(const bf16x4*)&Qt[off + 8];
          dkacc[dm] = mfma32(__builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7), sb,
                             dkacc[dm]);
        }
      }
    }
  }

  if (key_ok) {
    bf16* kr = dk + kvrow * HD;
    bf16* vr = dv + kvrow * HD;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        bf16x4 wk, wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wk[e] = (bf16)(dkacc[dm][4 * rr + e] * D.sm_scale);
          wv[e] = (bf16)dvacc[dm][4 * rr + e];
        }
        *(bf16x4*)(kr + 32 * dm + 8 * rr + 4 * hh) = wk;
        *(bf16x4*)(vr + 32 * dm + 8 * rr + 4 * hh) = wv;
      }
    }
  }
}

// --------------------------------------------------------------------------
// Key-stationary dK, dV for d = 128 on 16x16x32 MFMA tiles: a workgroup owns
// one 64-key block (one gate block), each wave 16 keys whose K and V rows
// stay in registers as B operands; the 16 x 128 dK and dV accumulators are
// 32 registers each, so the kernel runs three waves per SIMD with no
// accumulator spills.  Work items are (query head of the group, 32-row query
// tile).  The Q and dO tiles of an item stream global -> LDS with direct
// loads into two buffers; the transposed operands (dO^T for dV, Q^T for dK)
// come from transposing LDS reads of the same row-major tiles, laid out by
// trow() so that both kinds of read hit disjoint banks.  The per-row data of
// an item (each unit's log2 logit offset and D, written unit-major by the dQ
// kernel) arrives the same way: one direct load of (UB + 1) x 128 bytes, so
// the item loop does no per-row arithmetic of its own.  In the
// S / dP products each 16-byte operand read is issued one product ahead (two
// operand registers in turn: the register budget of three waves per SIMD
// leaves no room for more), and a wave raises its issue priority while it
// runs its matrix products so that the other waves of the SIMD fill the gaps
// with their exponentials.
// --------------------------------------------------------------------------
template <int DS, int UB>
__global__ __launch_bounds__(256, 2) void bwd_dkdv16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ rowd, int tqp,
    const bf16* __restrict__ qs, const bf16* __restrict__ ks, float* __restrict__ dks_acc,
    bf16* __restrict__ dk, bf16* __restrict__ dv, Dims D, int xcd_groups) {
  constexpr int HD = 128, QT = 32, TS = QT * 18, TE = TS * 8;  // tile slots, elements
  constexpr int NI = TS / 64;              // direct-load instructions per tile and tensor
  constexpr int XI = (NI + 3) / 4;         // ... per wave (at most)
  constexpr int BU = UB > 0 ? kBlock / UB : 1;  // tokens per gate unit (UB units per 64-key tile)
  // UB = 0 (units of D.blk = 1 .. 8 tokens): an item also brings its 32 qs
  // rows (XS 16-byte slots per row, one of them padding; three direct loads)
  // and four row values (lam log2 e, lse log2 e, D, sum_j dbeta / blk); the
  // kernel forms Z = QS KS^T, the gate g and e = dS - g sum_j dbeta / blk per
  // (row, key), and dks^T += QS^T e, summed over each unit's keys at the end.
  constexpr int XS = DS / 8 + 1, XP = XS * 8, XN = UB > 0 ? 8 : 3 * 512;
  constexpr int NF = UB > 0 ? UB + 1 : 4;
  static_assert(UB > 0 || DS == 32, "token units: ds = 32 (three waves load the qs tile)");
  __shared__ __align__(16) bf16 Q0[TE];
  __shared__ __align__(16) bf16 Q1[TE];
  __shared__ __align__(16) bf16 O0[TE];
  __shared__ __align__(16) bf16 O1[TE];
  __shared__ __align__(16) float F0[NF * QT];  // log2 offset of (unit, row), then D
  __shared__ __align__(16) float F1[NF * QT];
  __shared__ __align__(16) bf16 X0[XN];
  __shared__ __align__(16) bf16 X1[XN];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, g4 = lane >> 4;
  const int k4 = i16 >> 2, a4 = i16 & 3;
  int b, g, j;
  {
    const int L = blockIdx.x;
    int G;
    if (xcd_groups > 0) {
      const int xcd = L & 7, s = L >> 3;
      G = (s % xcd_groups) * 8 + xcd;
      j = s / xcd_groups;
    } else {
      const int bg = D.batch * D.hkv;
      j = L / bg;
      G = L % bg;
    }
    b = G / D.hkv;
    g = G % D.hkv;
  }
  const int key0 = j * kBlock + wave * 16;
  const int key = key0 + i16;
  const size_t kvrow = ((size_t)b * D.hkv + g) * D.tk + key;
  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    kf[s] = *(const bf16x8*)(k + kvrow * HD + 32 * s + 8 * g4);
    vf[s] = *(const bf16x8*)(v + kvrow * HD + 32 * s + 8 * g4);
  }
  f32x4 dka[8], dva[8];
#pragma unroll
  for (int dm = 0; dm < 8; ++dm) {
    dka[dm] = f32x4{};
    dva[dm] = f32x4{};
  }
  const float c1 = D.sm_scale * kLog2e;
  const int lb = __builtin_ctz(UB > 0 ? BU : D.blk);
  // UB = 0: this lane's key's unit row of ks (the Z B operand), reloaded when
  // the selector head changes from one query head of the group to the next;
  // dks^T of the wave's 16 keys (16 dims x 16 keys per block)
  bf16x8 xf[UB == 0 ? DS / 32 : 1];
  f32x4 dksa[UB == 0 ? DS / 16 : 1];
  int shc = -1;
  const float zs2 = D.sel_scale * kLog2e;
  auto load_x = [&](int shn) {
    const bf16* kr = ks + (((size_t)b * D.hks + shn) * D.nb + (key >> lb)) * DS + 8 * g4;
#pragma unroll
    for (int s = 0; s < DS / 32; ++s) xf[s] = *(const bf16x8*)(kr + 32 * s);
#pragma unroll
    for (int x = 0; x < DS / 16; ++x) dksa[x] = f32x4{};
    shc = shn;
  };
  // sum dks^T over each unit's keys (lanes i16 of one unit are adjacent) and
  // add it to the fp32 accumulator of selector head shc
  auto flush_x = [&]() {
    const int bsz = 1 << lb;
#pragma unroll
    for (int x = 0; x < DS / 16; ++x) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = dksa[x][r];
        for (int o = 1; o < bsz; o <<= 1) v += __shfl_xor(v, o);
        if ((i16 & (bsz - 1)) == 0)
          atomicAdd(dks_acc + (((size_t)b * D.hks + shc) * D.nb + (key >> lb)) * DS + 16 * x +
                        4 * g4 + r,
                    v);
      }
    }
  };
  const int qt0 = max(0, j * kBlock - D.qoff) / QT;
  const int per_h = (D.tq + QT - 1) / QT - qt0;
  const int nitems = D.hpg * per_h;

  // byte offsets, within a tile, of this lane's direct loads (row clamp aside)
  unsigned toff[XI];
  int trw[XI];
#pragma unroll
  for (int x = 0; x < XI; ++x) {
    const unsigned so = tslot_src(min((wave + 4 * x) * 64 + lane, TS - 1));
    trw[x] = so / HD;
    toff[x] = so * 2;
  }

  // work item: head hl of the group, query tile t (rows i0 = (qt0 + t) QT ..);
  // qo: element offset of its first row in q / dout, fo: of its first row in
  // slot 0 of the row data (both advanced by additions from item to item)
  struct Item {
    int hl, t;
    size_t qo, fo;
  };
  const size_t hq0 = (size_t)b * D.hq + g * D.hpg;  // first query head of the group
  auto first = [&](int hl) {
    Item x;
    x.hl = hl;
    x.t = 0;
    x.qo = ((hq0 + hl) * D.tq + (size_t)qt0 * QT) * HD;
    x.fo = (hq0 + hl) * (size_t)(UB > 0 ? D.nb + 1 : 4) * tqp + (size_t)qt0 * QT;
    return x;
  };
  auto next = [&](Item x) {
    if (++x.t == per_h) return first(x.hl + 1);
    x.qo += (size_t)QT * HD;
    x.fo += QT;
    return x;
  };
  auto row0 = [&](Item x) { return (qt0 + x.t) * QT; };
  // this lane's part of the row-data address: slot (unit s of tile j, or D
  // for s = UB) and rows 4 e .. 4 e + 3 for lane 8 s + e
  const int fsl = min(lane >> 3, NF - 1);
  const size_t flane =
      (UB == 0 ? (size_t)fsl : (fsl < UB ? (size_t)j * UB + fsl : (size_t)D.nb)) * tqp +
      4 * (lane & 7);
  // UB = 0: slot s = 64 (wave - 1) + lane of the qs tile: row s / XS, chunk
  // s % XS (padding chunk and slots past the tile reload chunk 0 / row 31)
  const int xsl = max(64 * (wave - 1) + lane, 0);
  const int xrow = min(xsl / XS, QT - 1), xch = xsl < QT * XS ? xsl % XS : 0;
  const int xoff = xrow * DS + (xch < DS / 8 ? xch : 0) * 8;

  // direct loads of an item's Q and dO tiles (all waves; rows past the end
  // reload the last row) and of its row data (wave 0, lanes 0 .. 8 UB + 7)
  auto issue = [&](Item x, bf16* Qd, bf16* Od, float* Fd, bf16* Xd) {
    if constexpr (UB == 0) {
      if (wave >= 1) {  // waves 1 .. 3: one 1 KB load each of the qs tile
        const int r0 = row0(x);
        const int rr = min(xrow, D.tq - 1 - r0);
        const bf16* const src =
            qs + ((hq0 + x.hl) * D.tq + r0 + rr) * (size_t)DS + (xoff - xrow * DS);
        __builtin_amdgcn_global_load_lds(src, Xd + (wave - 1) * 512, 16, 0, 0);
      }
    }
    if (wave == 0 && lane < 8 * NF) {
      // (through a named pointer: passing the sum straight to the builtin
      // makes the host pass drop this kernel's launch stub)
      const float* const src = rowd + x.fo + flane;
      __builtin_amdgcn_global_load_lds(src, Fd, 16, 0, 0);
    }
    const bf16* const qb = q + x.qo;
    const bf16* const ob = dout + x.qo;
    const int rmax = D.tq - 1 - row0(x);
    if (rmax >= QT - 1) {  // uniform: every row of the tile exists
#pragma unroll
      for (int xi = 0; xi < XI; ++xi) {
        const int ins = wave + 4 * xi;
        if (ins < NI) {
          __builtin_amdgcn_global_load_lds((const char*)qb + toff[xi], Qd + ins * 512, 16, 0, 0);
          __builtin_amdgcn_global_load_lds((const char*)ob + toff[xi], Od + ins * 512, 16, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int xi = 0; xi < XI; ++xi) {
        const int ins = wave + 4 * xi;
        if (ins < NI) {
          unsigned off = toff[xi];
          if (trw[xi] > rmax) off -= (unsigned)(trw[xi] - rmax) * HD * 2;
          __builtin_amdgcn_global_load_lds((const char*)qb + off, Qd + ins * 512, 16, 0, 0);
          __builtin_amdgcn_global_load_lds((const char*)ob + off, Od + ins * 512, 16, 0, 0);
        }
      }
    }
  };
  // the unit of this wave's 16 keys within the tile
  const int uw = UB <= 1 ? 0 : (wave * 16) / BU;

  auto compute = [&](Item x, const bf16* Qs, const bf16* Os, const float* Fs, const bf16* Xs) {
    const int i0 = row0(x);
    if constexpr (UB == 0) {
      const int shn = (int)((hq0 + x.hl - (size_t)b * D.hq) / D.hps);
      if (shn != shc) {
        if (shc >= 0) flush_x();
        load_x(shn);
      }
    }
    if (D.qoff + min(i0 + QT - 1, D.tq - 1) < key0) return;  // every row before these keys
    // keys after a row's position are cut: slot (16 mq + r) of this lane is
    // cut when it is below mlim (no cut away from the diagonal)
    const bool mlim_on = D.qoff + i0 < key0 + 15;  // uniform over the workgroup
    const int mlim = key - (D.qoff + i0 + 4 * g4);
    f32x4 sacc[2] = {f32x4{}, f32x4{}};
    f32x4 pacc[2] = {f32x4{}, f32x4{}};
    __builtin_amdgcn_s_setprio(1);
    // operand i (step i / 4, M-tile (i / 2) % 2, Q or dO by i % 2) is read
    // while product i - 1 runs: two operand registers in turn
    auto opnd = [&](int i) __attribute__((always_inline)) {
      const int o = trow(i16) + 2304 * ((i >> 1) & 1) + 32 * (i >> 2) + 8 * g4;
      return *(const bf16x8*)&((i & 1) ? Os : Qs)[o];
    };
    bf16x8 ob[2];
    ob[0] = opnd(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < 15) ob[(i + 1) & 1] = opnd(i + 1);
      const int s = i >> 2, mq = (i >> 1) & 1;
      if (i & 1)
        pacc[mq] = mfma16(ob[i & 1], vf[s], pacc[mq]);
      else
        sacc[mq] = mfma16(ob[i & 1], kf[s], sacc[mq]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < 15; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_s_setprio(0);
    // P and dS; the causal cut only on items that meet the diagonal
    // UB = 0: Z = QS KS^T for the same (row, key) slots, and e (in zacc)
    f32x4 zacc[2] = {f32x4{}, f32x4{}};
    if constexpr (UB == 0) {
#pragma unroll
      for (int mq = 0; mq < 2; ++mq)
#pragma unroll
        for (int s = 0; s < DS / 32; ++s)
          zacc[mq] = mfma16(*(const bf16x8*)&Xs[(16 * mq + i16) * XP + 32 * s + 8 * g4], xf[s],
                            zacc[mq]);
    }
    auto softmax_ds = [&](auto mask_tag) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
      if constexpr (UB == 0) {
        const int tr0 = D.qoff + i0 + 4 * g4;  // position of row 4 g4 (M-tile 0)
#pragma unroll
        for (int mq = 0; mq < 2; ++mq) {
          const f32x4 la = *(const f32x4*)&Fs[16 * mq + 4 * g4];
          const f32x4 ll = *(const f32x4*)&Fs[QT + 16 * mq + 4 * g4];
          const f32x4 dl = *(const f32x4*)&Fs[2 * QT + 16 * mq + 4 * g4];
          const f32x4 sb = *(const f32x4*)&Fs[3 * QT + 16 * mq + 4 * g4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool hist = (key >> lb) < ((tr0 + 16 * mq + r) >> lb);
            const float zl = fmaf(zacc[mq][r], zs2, -la[r]);
            float p = exp2_raw(fmaf(sacc[mq][r], c1, (hist ? zl : 0.f) - ll[r]));
            if (MASK && 16 * mq + r < mlim) p = 0.f;
            sacc[mq][r] = p;
            const float ds = p * (pacc[mq][r] - dl[r]);
            pacc[mq][r] = ds;
            zacc[mq][r] = hist ? ds - exp2_raw(zl) * sb[r] : 0.f;
          }
        }
        return;
      }
#pragma unroll
      for (int mq = 0; mq < 2; ++mq) {
        const f32x4 of = *(const f32x4*)&Fs[uw * QT + 16 * mq + 4 * g4];
        const f32x4 dl = *(const f32x4*)&Fs[UB * QT + 16 * mq + 4 * g4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float p = exp2_raw(fmaf(sacc[mq][r], c1, of[r]));
          if (MASK && 16 * mq + r < mlim) p = 0.f;
          sacc[mq][r] = p;
          pacc[mq][r] = p * (pacc[mq][r] - dl[r]);
        }
      }
    };
    if (mlim_on)
      softmax_ds(std::true_type{});
    else
      softmax_ds(std::false_type{});
    // B operands over the 32 rows: slots 0..3 = rows 4*g4 + r, 4..7 = 16 + 4*g4 + r
    bf16x8 pb, sb;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pb[r] = (bf16)sacc[0][r];
      pb[4 + r] = (bf16)sacc[1][r];
      sb[r] = (bf16)pacc[0][r];
      sb[4 + r] = (bf16)pacc[1][r];
    }
    const int t0 = trow(4 * g4 + k4) + 4 * a4, t1 = t0 + 2304;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dm = 0; dm < 8; ++dm) {
      const bf16x4 olo = ds_read_tr(&Os[t0 + 16 * dm]);
      const bf16x4 ohi = ds_read_tr(&Os[t1 + 16 * dm]);
      dva[dm] = mfma16(__builtin_shufflevector(olo, ohi, 0, 1, 2, 3, 4, 5, 6, 7), pb, dva[dm]);
      const bf16x4 qlo = ds_read_tr(&Qs[t0 + 16 * dm]);
      const bf16x4 qhi = ds_read_tr(&Qs[t1 + 16 * dm]);
      dka[dm] = mfma16(__builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7), sb, dka[dm]);
    }
    if constexpr (UB == 0) {
      // dks^T += QS^T e: the same transposing reads over the qs tile; e as a
      // bf16 pair (e_hi + e_lo), so that dks keeps fp32-like accuracy where
      // the terms of a unit cancel
      bf16x8 eh, el;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        eh[r] = (bf16)zacc[0][r];
        eh[4 + r] = (bf16)zacc[1][r];
        el[r] = (bf16)(zacc[0][r] - (float)eh[r]);
        el[4 + r] = (bf16)(zacc[1][r] - (float)eh[4 + r]);
      }
      const int x0 = (4 * g4 + k4) * XP + 4 * a4, x1 = x0 + 16 * XP;
#pragma unroll
      for (int x = 0; x < DS / 16; ++x) {
        const bf16x4 slo = ds_read_tr(&Xs[x0 + 16 * x]);
        const bf16x4 shi = ds_read_tr(&Xs[x1 + 16 * x]);
        const bf16x8 a = __builtin_shufflevector(slo, shi, 0, 1, 2, 3, 4, 5, 6, 7);
        dksa[x] = mfma16(a, eh, dksa[x]);
        dksa[x] = mfma16(a, el, dksa[x]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  if (nitems > 0) {
    Item cur = first(0);
    issue(cur, Q0, O0, F0, X0);
    wait_vmem();
    __syncthreads();
    // Item it: the tiles and row data of it + 1 load while it computes.
    // Unrolled by two so that both buffers' code sits in one loop body.
    for (int it = 0; it < nitems; it += 2) {
      const Item n1 = next(cur), n2 = next(n1);
      if (it + 1 < nitems) issue(n1, Q1, O1, F1, X1);
      compute(cur, Q0, O0, F0, X0);
      wait_vmem();
      __syncthreads();
      if (it + 1 >= nitems) break;
      if (it + 2 < nitems) issue(n2, Q0, O0, F0, X0);
      compute(n1, Q1, O1, F1, X1);
      wait_vmem();
      __syncthreads();
      cur = n2;
    }
  }
  if constexpr (UB == 0) {
    if (shc >= 0) flush_x();
  }
  bf16* kr = dk + kvrow * HD + 4 * g4;
  bf16* vr = dv + kvrow * HD + 4 * g4;
#pragma unroll
  for (int dm = 0; dm < 8; ++dm) {
    bf16x4 wk, wv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      wk[r] = (bf16)(dka[dm][r] * D.sm_scale);
      wv[r] = (bf16)dva[dm][r];
    }
    *(bf16x4*)(kr + 16 * dm) = wk;
    *(bf16x4*)(vr + 16 * dm) = wv;
  }
}

// --------------------------------------------------------------------------
// dks[b, s, j, :] = sel_scale * sum over rows (h of s, t with c(t) > j) of
// dz[t, j] qs[t, :]: per (32-block tile, head of the selector group, row
// chunk) a contraction over rows on fp32 32x32x2 MFMA (A = dz^T: block x
// row, B = qs: row x dim; dz is zero for j >= c(t), so only rows before the
// tile's first visible one are skipped).  The four waves take alternate row
// pairs; their tiles are summed in LDS and added to an fp32 accumulator with
// atomics.
// --------------------------------------------------------------------------
constexpr int kDksChunk = 2048;  // rows per workgroup

template <int DS, typename ST>
__global__ __launch_bounds__(256) void dks_kernel(const float* __restrict__ dz,
                                                  const ST* __restrict__ qs,
                                                  float* __restrict__ acc, Dims D) {
  constexpr int NT = (DS + 31) / 32;  // 32-dim N-tiles
  __shared__ float red[4][NT][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j0 = blockIdx.x * 32;
  const int bs = blockIdx.z, b = bs / D.hks, s = bs % D.hks;
  const int nch = (D.tq + kDksChunk - 1) / kDksChunk;
  const int hl = blockIdx.y / nch, i0 = (blockIdx.y % nch) * kDksChunk;
  const int i_min = max(0, (j0 + 1) * D.blk - D.qoff);  // first row with c(t) > j0
  const int istart = max(i0, i_min), iend = min(i0 + kDksChunk, D.tq);
  if (istart >= iend) return;  // uniform over the workgroup
  const size_t hrow = ((size_t)b * D.hq + s * D.hps + hl) * D.tq;
  const int blk = j0 + (lane & 31), rsub = lane >> 5;
  f32x16 dacc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) dacc[nt] = f32x16{};
  constexpr int U = 8;  // row pairs whose loads are in flight together
  for (int i = istart + 2 * wave; i < iend; i += 8 * U) {
    // loads without branches (row, block and dim clamped into range, the
    // values past the ends masked to 0), so that all of them are in flight
    // together
    float a[U], bq[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ii = i + 8 * u + rsub;
      const bool ok = ii < iend;
      const size_t ri = hrow + (size_t)min(ii, iend - 1);
      const float zv = dz[ri * D.nb + min(blk, D.nb - 1)];
      a[u] = ok && blk < D.nb ? zv : 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int dim = 32 * nt + (lane & 31);
        const float qv = to_f32(qs[ri * DS + min(dim, DS - 1)]);
        bq[u][nt] = ok && dim < DS ? qv : 0.f;
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // the loads stay ahead of the products
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        dacc[nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[u], bq[u][nt], dacc[nt], 0, 0, 0);
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave][nt][r][lane] = dacc[nt][r];
  __syncthreads();
  // accumulator lane l, register r: dim 32 nt + l % 32, block 8 (r / 4) + 4 (l / 32) + r % 4
  for (int x = threadIdx.x; x < NT * 16 * 64; x += 256) {
    const int nt = x / 1024, r = (x / 64) % 16, l = x % 64;
    const float v = red[0][nt][r][l] + red[1][nt][r][l] + red[2][nt][r][l] + red[3][nt][r][l];
    const int j = j0 + 8 * (r / 4) + 4 * (l / 32) + r % 4, dim = 32 * nt + l % 32;
    if (j < D.nb && dim < DS && v != 0.f)
      atomicAdd(acc + (((size_t)b * D.hks + s) * D.nb + j) * DS + dim, v);
  }
}

// The same reduction with 16-byte loads of dz (nb % 4 == 0): lane l reads
// blocks j0 + 4 (l % 32) .. + 3 of its row in one load, and the four values
// feed four 32-block MFMA tiles (tile q holds blocks j0 + 4 m + q), so a
// workgroup covers 128 blocks and a load instruction moves 1 KB instead of
// 256 bytes; the qs operand of a row pair serves all four tiles.  The
// waves' tiles are summed through LDS one tile at a time.
constexpr int kDks4Blocks = 128;

template <int DS, typename ST>
__global__ __launch_bounds__(256) void dks4_kernel(const float* __restrict__ dz,
                                                   const ST* __restrict__ qs,
                                                   float* __restrict__ acc, Dims D) {
  constexpr int NT = (DS + 31) / 32;  // 32-dim N-tiles
  __shared__ float red[4][NT][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j0 = blockIdx.x * kDks4Blocks;
  const int bs = blockIdx.z, b = bs / D.hks, s = bs % D.hks;
  const int nch = (D.tq + kDksChunk - 1) / kDksChunk;
  const int hl = blockIdx.y / nch, i0 = (blockIdx.y % nch) * kDksChunk;
  const int i_min = max(0, (j0 + 1) * D.blk - D.qoff);  // first row with c(t) > j0
  const int istart = max(i0, i_min), iend = min(i0 + kDksChunk, D.tq);
  if (istart >= iend) return;  // uniform over the workgroup
  const size_t hrow = ((size_t)b * D.hq + s * D.hps + hl) * D.tq;
  const int jl = j0 + 4 * (lane & 31), rsub = lane >> 5;
  f32x16 dacc[4][NT];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) dacc[q][nt] = f32x16{};
  constexpr int U = 8;  // row pairs whose loads are in flight together
  for (int i = istart + 2 * wave; i < iend; i += 8 * U) {
    // loads without branches (row and dim clamped into range, the values
    // past the ends masked to 0), so that all of them are in flight together;
    // with nb % 4 == 0 a lane's four blocks all exist or none does
    f32x4 a[U];
    float bq[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ii = i + 8 * u + rsub;
      const bool ok = ii < iend && jl < D.nb;
      const size_t ri = hrow + (size_t)min(ii, iend - 1);
      const f32x4 zv = *(const f32x4*)(dz + ri * D.nb + min(jl, D.nb - 4));
#pragma unroll
      for (int q = 0; q < 4; ++q) a[u][q] = ok ? zv[q] : 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int dim = 32 * nt + (lane & 31);
        const float qv = to_f32(qs[ri * DS + min(dim, DS - 1)]);
        bq[u][nt] = ii < iend && dim < DS ? qv : 0.f;
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // the loads stay ahead of the products
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          dacc[q][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[u][q], bq[u][nt], dacc[q][nt], 0,
                                                              0, 0);
  }
  // accumulator of tile q, lane l, register r: dim 32 nt + l % 32, block
  // j0 + 4 (8 (r / 4) + 4 (l / 32) + r % 4) + q
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[wave][nt][r][lane] = dacc[q][nt][r];
    __syncthreads();
    for (int x = threadIdx.x; x < NT * 16 * 64; x += 256) {
      const int nt = x / 1024, r = (x / 64) % 16, l = x % 64;
      const float v = red[0][nt][r][l] + red[1][nt][r][l] + red[2][nt][r][l] + red[3][nt][r][l];
      const int j = j0 + 4 * (8 * (r / 4) + 4 * (l / 32) + r % 4) + q, dim = 32 * nt + l % 32;
      if (j < D.nb && dim < DS && v != 0.f)
        atomicAdd(acc + (((size_t)b * D.hks + s) * D.nb + j) * DS + dim, v);
    }
    __syncthreads();
  }
}

__global__ void fill_zero_kernel(float* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

template <typename ST>
__global__ void scale_convert_kernel(const float* __restrict__ src, ST* __restrict__ dst,
                                     float scale, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = from_f32<ST>(src[i] * scale);
}

// Per-key selector rows for token-level units: ksx[b, s, u, :] = ks[b, s, u / blk, :].
__global__ void ks_expand_kernel(const bf16* __restrict__ ks, bf16* __restrict__ ksx, int lb,
                                 int tk, int ds8, size_t n8) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t ch = i % ds8, u = (i / ds8) % tk, bs = i / ((size_t)ds8 * tk);
    const size_t src = (bs * (size_t)(tk >> lb) + (u >> lb)) * ds8 + ch;
    ((bf16x8*)ksx)[i] = ((const bf16x8*)ks)[src];
  }
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// bf16, d = 128 with units of fewer than 16 tokens: the token-unit kernels
static bool token_units(const Dims& D) { return D.d == 128 && D.blk < 16; }

BwdWs bwd_workspace(const Dims& D, bool need_dz) {
  BwdWs W;
  const size_t rows = (size_t)D.batch * D.hq * D.tq;
  const bool tok = token_units(D);
  size_t off = 0;
  W.off_delta = off;
  off += align256(rows * sizeof(float));
  W.off_dz = off;
  if (need_dz && !tok) off += align256(rows * (size_t)D.nb * sizeof(float));
  W.off_dks = off;
  off += align256((size_t)D.batch * D.hks * D.nb * D.ds * sizeof(float));
  W.tqp = (D.tq + 31) / 32 * 32;
  W.off_rows = off;
  if (D.d == 128)
    off += align256((size_t)D.batch * D.hq * (tok ? 4 : D.nb + 1) * W.tqp * sizeof(float));
  W.off_ksx = off;
  if (tok && D.blk > 1)
    off += align256((size_t)D.batch * D.hks * D.tk * D.ds * sizeof(bf16));
  W.total = off;
  return W;
}

template <typename ST>
hipError_t launch_dks(const float* dz, const void* qs, float* acc, void* dks, const Dims& D,
                      hipStream_t st) {
  const size_t n = (size_t)D.batch * D.hks * D.nb * D.ds;
  const unsigned fg = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(fg), dim3(256), 0, st, acc, n);
  if (D.nb % 4 == 0) {
    dim3 grid4((D.nb + kDks4Blocks - 1) / kDks4Blocks,
               D.hps * ((D.tq + kDksChunk - 1) / kDksChunk), D.batch * D.hks);
    switch (D.ds) {
      case 16:
        hipLaunchKernelGGL((dks4_kernel<16, ST>), grid4, dim3(256), 0, st, dz, (const ST*)qs, acc, D);
        break;
      case 32:
        hipLaunchKernelGGL((dks4_kernel<32, ST>), grid4, dim3(256), 0, st, dz, (const ST*)qs, acc, D);
        break;
      case 64:
        hipLaunchKernelGGL((dks4_kernel<64, ST>), grid4, dim3(256), 0, st, dz, (const ST*)qs, acc, D);
        break;
      default:
        return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL((scale_convert_kernel<ST>), dim3(fg), dim3(256), 0, st, (const float*)acc,
                       (ST*)dks, D.sel_scale, n);
    return hipGetLastError();
  }
  dim3 grid((D.nb + 31) / 32, D.hps * ((D.tq + kDksChunk - 1) / kDksChunk), D.batch * D.hks);
  switch (D.ds) {
    case 16:
      hipLaunchKernelGGL((dks_kernel<16, ST>), grid, dim3(256), 0, st, dz, (const ST*)qs, acc, D);
      break;
    case 32:
      hipLaunchKernelGGL((dks_kernel<32, ST>), grid, dim3(256), 0, st, dz, (const ST*)qs, acc, D);
      break;
    case 64:
      hipLaunchKernelGGL((dks_kernel<64, ST>), grid, dim3(256), 0, st, dz, (const ST*)qs, acc, D);
      break;
    default:
      return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL((scale_convert_kernel<ST>), dim3(fg), dim3(256), 0, st, (const float*)acc,
                     (ST*)dks, D.sel_scale, n);
  return hipGetLastError();
}
template hipError_t launch_dks<float>(const float*, const void*, float*, void*, const Dims&,
                                      hipStream_t);

template <int HD, int DS, int UB>
static hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const void* o,
                               const void* dout, const float* lse, const void* qs,
                               const void* ks, const float* lam, void* dq, void* dk, void* dv,
                               void* dqs, void* dks, float* dz, char* ws, const BwdWs& W,
                               const Dims& D, const StageEvents& E, hipStream_t st) {
  float* delta = (float*)(ws + W.off_delta);
  float* dzp = dz ? dz : (float*)(ws + W.off_dz);
  float* acc = (float*)(ws + W.off_dks);
  float* rowd = (float*)(ws + W.off_rows);
  const int groups = D.batch * D.hkv;
  const int xg = groups % 8 == 0 ? groups / 8 : 0;
  hipError_t e;
  if constexpr (UB == 0) {
    // token-level units: dz only when the caller asks for it; dks from the
    // dK/dV kernel (fp32 accumulator, scaled and converted at the end)
    const size_t nacc = (size_t)D.batch * D.hks * D.nb * D.ds;
    const unsigned fg = (unsigned)std::min<size_t>((nacc + 255) / 256, 4096);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(fg), dim3(256), 0, st, acc, nacc);
    const bf16* ksx = (const bf16*)ks;
    if (D.blk > 1) {
      const size_t n8 = (size_t)D.batch * D.hks * D.tk * (D.ds / 8);
      const unsigned xgd = (unsigned)std::min<size_t>((n8 + 255) / 256, 4096);
      hipLaunchKernelGGL(ks_expand_kernel, dim3(xgd), dim3(256), 0, st, (const bf16*)ks,
                         (bf16*)(ws + W.off_ksx), __builtin_ctz(D.blk), D.tk, D.ds / 8, n8);
      ksx = (const bf16*)(ws + W.off_ksx);
    }
    const int nqtw = (D.tq + kDq32Rows - 1) / kDq32Rows;
    hipLaunchKernelGGL((bwd_dq32_kernel<DS, 0>), dim3(D.batch * D.hq * nqtw), dim3(kDq32Threads),
                       0, st, (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)o,
                       (const bf16*)dout, lse, (const bf16*)qs, ksx, lam, (bf16*)dq,
                       (bf16*)dqs, dz, rowd, W.tqp, D, nqtw, xg);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    E.record(0, st);
    hipLaunchKernelGGL((bwd_dkdv16_kernel<DS, 0>), dim3(groups * (D.tk / kBlock)), dim3(256), 0,
                       st, (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout,
                       (const float*)rowd, W.tqp, (const bf16*)qs, (const bf16*)ks, acc,
                       (bf16*)dk, (bf16*)dv, D, xg);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    E.record(1, st);
    hipLaunchKernelGGL((scale_convert_kernel<bf16>), dim3(fg), dim3(256), 0, st,
                       (const float*)acc, (bf16*)dks, D.sel_scale, nacc);
    E.record(2, st);
    return hipGetLastError();
  } else if constexpr (HD == 128) {
    // The 32-row kernel fits two waves per SIMD (256 registers each) while
    // the selector terms of a tile (ds / 2 qs and dqs values per lane, UB ks
    // rows) stay small; wider selectors take the 16-row kernel.
    if constexpr (DS <= 32 && DS * UB <= 64) {
      const int nqtw = (D.tq + kDq32Rows - 1) / kDq32Rows;
      hipLaunchKernelGGL((bwd_dq32_kernel<DS, UB>), dim3(D.batch * D.hq * nqtw),
                         dim3(kDq32Threads), 0, st, (const bf16*)q, (const bf16*)k,
                         (const bf16*)v, (const bf16*)o, (const bf16*)dout, lse,
                         (const bf16*)qs, (const bf16*)ks, lam, (bf16*)dq, (bf16*)dqs, dzp, rowd,
                         W.tqp, D, nqtw, xg);
    } else {
      const int nqtw = (D.tq + kDqRows - 1) / kDqRows;
      hipLaunchKernelGGL((bwd_dq16_kernel<DS, UB>), dim3(D.batch * D.hq * nqtw),
                         dim3(kDqThreads), 0, st, (const bf16*)q, (const bf16*)k,
                         (const bf16*)v, (const bf16*)o, (const bf16*)dout, lse,
                         (const bf16*)qs, (const bf16*)ks, lam, (bf16*)dq, (bf16*)dqs, dzp, rowd,
                         W.tqp, D, nqtw, xg);
    }
  } else {
  const int nqt = (D.tq + 127) / 128;
  hipLaunchKernelGGL((bwd_dq_kernel<HD, DS>), dim3(D.batch * D.hq * nqt), dim3(256), 0, st,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)o,
                     (const bf16*)dout, lse, (const bf16*)qs, (const bf16*)ks, lam, (bf16*)dq,
                     (bf16*)dqs, dzp, delta, D, nqt, xg);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  E.record(0, st);
  if constexpr (HD == 128) {
    hipLaunchKernelGGL((bwd_dkdv16_kernel<DS, UB>), dim3(groups * (D.tk / kBlock)), dim3(256), 0,
                       st, (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout,
                       (const float*)rowd, W.tqp, nullptr, nullptr, nullptr, (bf16*)dk,
                       (bf16*)dv, D, xg);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    E.record(1, st);
    e = launch_dks<bf16>(dzp, qs, acc, dks, D, st);
    E.record(2, st);
    return e;
  }
  const int nkt = (D.tk + 127) / 128;
  hipLaunchKernelGGL((bwd_dkdv_kernel<HD, DS>), dim3(groups * nkt), dim3(256), 0, st,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout, lse,
                     (const float*)delta, (const bf16*)qs, (const bf16*)ks, lam, (bf16*)dk,
                     (bf16*)dv, D, nkt, xg);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  E.record(1, st);
  e = launch_dks<bf16>(dzp, qs, acc, dks, D, st);
  E.record(2, st);
  return e;
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, const void* qs, const void* ks,
                           const float* lam, void* dq, void* dk, void* dv, void* dqs, void* dks,
                           float* dz, char* ws, const BwdWs& W, const Dims& D,
                           const StageEvents& E, hipStream_t st) {
#define SAS_BWD_CALL(HDV, DSV, UBV)                                                           \
  return launch_bwd_t<HDV, DSV, UBV>(q, k, v, o, dout, lse, qs, ks, lam, dq, dk, dv, dqs, dks, \
                                     dz, ws, W, D, E, st);
  // d = 128: gate units of 64, 32 or 16 tokens, and (ds = 32) of 8, 4, 2 or
  // 1 token; d = 64: 64
  if (D.d == 128 && D.ds == 32 && D.blk < 16) SAS_BWD_CALL(128, 32, 0)
#define SAS_BWD_CASE128(DSV)                        \
  if (D.d == 128 && D.ds == DSV) {                  \
    if (D.blk == 64) SAS_BWD_CALL(128, DSV, 1)      \
    if (D.blk == 32) SAS_BWD_CALL(128, DSV, 2)      \
    if (D.blk == 16) SAS_BWD_CALL(128, DSV, 4)      \
    return hipErrorInvalidValue;                    \
  }
#define SAS_BWD_CASE64(DSV) \
  if (D.d == 64 && D.ds == DSV && D.blk == 64) SAS_BWD_CALL(64, DSV, 1)
  SAS_BWD_CASE128(32)
  SAS_BWD_CASE128(16)
  SAS_BWD_CASE128(64)
  SAS_BWD_CASE64(32)
  SAS_BWD_CASE64(16)
  SAS_BWD_CASE64(64)
#undef SAS_BWD_CASE128
#undef SAS_BWD_CASE64
#undef SAS_BWD_CALL
  return hipErrorInvalidValue;
}

}  // namespace sas
