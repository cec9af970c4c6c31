// attn_fwd.hip -- dense-active gated causal attention forward (training).
//
// For query t (block c = t/64) and key u <= t:
//   logit = sm_scale <q_t, k_u> + beta_{t, u/64},
//   beta_{t,j} = sel_scale <qs_t, ks_j> - lam_t  (j < c),   beta_{t,c} = 0,
//   o_t = softmax_u(logit) v,   lse_t = log sum_u exp(logit).
// SAS abstracts (NeurIPS poster page, Hugging Face page): the gate enters the
// attention softmax in log form, every context unit stays active in training,
// the current block is always retained; the authors fuse it into a
// FlashAttention-style kernel so the T x T matrix is never materialised.
//
// gfx950 design (bf16 in, fp32 accumulate):
//  * workgroup = 8 waves = 256 query rows of one (batch, head); each wave owns
//    32 consecutive rows (two waves per SIMD; eight waves share each K/V
//    tile, which halves the registers that stage the next tile).  Key tiles are 64 keys = one gate block, so the gate
//    bias is a single scalar per (row, tile).
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the accumulator puts one query
//    per lane (column) and 16 keys per 32-key M-tile in registers, so the
//    row max / row sum are in-lane, plus one exchange between the two
//    32-lane halves.  Q stays in registers as the B operand for the whole
//    kernel.
//  * O^T = V^T P^T: P never leaves registers.  The B-operand k slots of a lane
//    are exactly the keys its S^T accumulator holds (two runs of 4), and the
//    V^T operand is read from LDS with the same key order.
//  * LDS: K and V tiles row-major (K in two buffers, V in three); the next
//    tile is loaded into registers at the start of a tile and stored to LDS
//    at its end (one barrier per tile); V^T operands come from transposing
//    LDS reads.  A 72-dword row pitch keeps both kinds of operand read
//    bank-conflict free.
//  * the two waves of a SIMD come from different halves of the workgroup,
//    and the second half runs each tile's PV product one tile late, so that
//    one wave's softmax overlaps the other's matrix products.
//  * the gate bias of (row, tile) is recomputed in-kernel: the lane's half of
//    qs (ds/2 values in registers) times the block's ks row (staged in LDS
//    with the tile), one cross-half add; lam comes from the gate kernel.
//  * exp2 domain throughout; tiles past a wave's last block are skipped, the
//    only masked tiles are the (at most two) diagonal ones.
#include "sas_device.h"
#include "sas_internal.h"

#include <type_traits>

namespace sas {

// workgroup: kFwdWaves waves of 32 query rows (kFwdRows rows) sharing each K/V tile
constexpr int kFwdWaves = 8, kFwdThreads = 64 * kFwdWaves, kFwdRows = 32 * kFwdWaves;

// UB gate units per 64-key tile (UB = 1: 64-token blocks; 2, 4: units of 32,
// 16 tokens, whose bias then changes inside the tile).  UB = 0: units of
// D.blk = 1, 2, 4 or 8 tokens (token-level units), where the bias changes
// from key to key: the selector scores of a tile, Z^T = KS QS^T over the ks
// rows of its 64 / blk units, come from matrix products too, and the key
// products accumulate on top of the historical keys' bias (see tile()).  GIVEN: the bias of
// each historical (row, block) is read from bt [b * hq][tq / 8][nb][8]
// (-inf for a block the row does not attend) instead of being computed from
// the selector: the same kernel then runs a sparse forward whose selection is
// dense enough that streaming every block beats gathering the selected ones
// (qs, ks and lam are unused).
template <int HD, int DS, int UB, bool GIVEN>
__global__ __launch_bounds__(kFwdThreads, 1) void attn_fwd_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ qs, const bf16* __restrict__ ks, const float* __restrict__ lam,
    const float* __restrict__ bt, bf16* __restrict__ o, float* __restrict__ lse, Dims D,
    int nqt, int xcd_groups) {
  constexpr int DC = HD / 8;                 // 16-byte chunks of a row
  constexpr int SP = HD == 128 ? 18 : 10;    // LDS row pitch in 16-byte slots (K and V)
  constexpr int KP = SP * 8, VP = KP;        // row pitches (elements)
  constexpr int NCH = kBlock * DC / kFwdThreads;  // 16-byte chunks per thread and tensor
  constexpr int KS = HD / 16;      // k-steps over the head dim
  constexpr int DM = HD / 32;      // 32-row M-tiles of O^T
  constexpr int BU = UB > 0 ? kBlock / UB : 1;  // tokens per gate unit (UB > 0)
  constexpr int XP = DS + 8;  // UB = 0: LDS pitch of the tile's ks rows (elements)
  constexpr int SN = UB > 0 ? UB * DS : kBlock * XP;
  // Key tiles in LDS, K and V row-major (V read transposed, as the V^T
  // operand, by transposing 8-byte reads); K in two buffers, V in three
  // (the PV products of half the waves run one tile late).  The next
  // tile goes global -> registers at the start of a tile and registers ->
  // LDS at its end: the LDS operand reads then never wait behind an
  // outstanding global -> LDS transfer.
  __shared__ __align__(16) bf16 K0[kBlock * KP];
  __shared__ __align__(16) bf16 K1[kBlock * KP];
  __shared__ __align__(16) bf16 V0[kBlock * VP];
  __shared__ __align__(16) bf16 V1[kBlock * VP];
  __shared__ __align__(16) bf16 V2[kBlock * VP];
  __shared__ __align__(16) bf16 S0[SN];  // ks rows of the tile's units
  __shared__ __align__(16) bf16 S1[SN];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6;  // (a wave-uniform copy here costs registers: keep it per lane)
  const int l32 = lane & 31, hh = lane >> 5;
  const QTile tm = map_q_tile(blockIdx.x, nqt, D, xcd_groups);
  const int b = tm.b, h = tm.h, qt = tm.qt;
  const int g = h / D.hpg, sh = h / D.hps;
  const int wq0 = qt * kFwdRows + wave * 32;
  const int qi = wq0 + l32;
  const int qc = min(qi, D.tq - 1);
  const int t = D.qoff + qc;
  const int blk = UB > 0 ? BU : D.blk;
  const int lb = __builtin_ctz(blk);  // blk is a power of two
  const int c = t >> lb;  // historical units of this row (tile bounds below are in 64-key tiles)
  const int tcur0 = c << lb;  // UB = 0: first key of the row's own unit
  const int c_lo = (D.qoff + min(wq0, D.tq - 1)) / kBlock;
  const int c_hi = (D.qoff + min(wq0 + 31, D.tq - 1)) / kBlock;
  const int c_end = (D.qoff + min(qt * kFwdRows + kFwdRows - 1, D.tq - 1)) / kBlock;


  const size_t qrow = ((size_t)b * D.hq + h) * D.tq + qc;
  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qf[s] = *(const bf16x8*)(q + qrow * HD + 16 * s + 8 * hh);
  // this lane's half of the row's qs, as bf16 pairs for packed dot products
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 qsv[DS / 4];
#pragma unroll
  for (int e = 0; e < DS / 4; ++e)
    qsv[e] = GIVEN ? bf16x2{} : *(const bf16x2*)(qs + qrow * DS + hh * (DS / 2) + 2 * e);
  const float lam_t = !GIVEN && c > 0 ? lam[qrow] : 0.f;
  // UB = 0: the lane's k-slots of the row's qs, the B operand of Z^T
  bf16x8 qsf[UB == 0 ? DS / 16 : 1];
  if constexpr (UB == 0) {
#pragma unroll
    for (int s = 0; s < DS / 16; ++s) qsf[s] = *(const bf16x8*)(qs + qrow * DS + 16 * s + 8 * hh);
  }
  // (UB = 0 keeps the selector constants in score units: see tile())
  const float zsc = D.sel_scale / D.sm_scale;
  const bf16* ksb0 = GIVEN ? ks : ks + ((size_t)b * D.hks + sh) * (size_t)D.nb * DS;
  const int urows = kBlock >> lb;  // UB = 0: units (ks rows) per tile
  // GIVEN: this row's bias of block j is btr[8 j]
  const float* btr =
      GIVEN ? bt + ((((size_t)b * D.hq + h) * ((D.tq + 7) / 8) + qc / 8) * D.nb) * 8 + qc % 8
            : nullptr;
  // GIVEN: the bias of the tile being scored and of the next one (loaded a tile ahead)
  float bcur = 0.f, bnext = GIVEN && 0 < c ? btr[0] : 0.f;
  const bf16* kb = k + ((size_t)b * D.hkv + g) * (size_t)D.tk * HD;
  const bf16* vb = v + ((size_t)b * D.hkv + g) * (size_t)D.tk * HD;
  const float c1 = D.sm_scale * kLog2e;

  f32x16 oacc[DM];
#pragma unroll
  for (int dm = 0; dm < DM; ++dm) oacc[dm] = f32x16{};
  // GIVEN: a large finite start, so a block with bias -inf before the row's
  // first visible key gives exp2(-inf) = 0 rather than -inf - -inf
  float m_run = GIVEN ? -1e30f : -INFINITY, l_run = 0.f;

  // next tile staged in registers: thread tid holds 16-byte chunks tid + kFwdThreads x
  // (row = chunk / DC, column chunk = chunk % DC) of K and of V, and threads
  // 0 .. DS/8-1 a chunk of the block's ks row
  bf16x8 kreg[NCH], vreg[NCH], sreg = bf16x8{};
  auto gload = [&](int j) __attribute__((always_inline)) {
    const bf16* kt = kb + (size_t)j * kBlock * HD;
    const bf16* vt = vb + (size_t)j * kBlock * HD;
#pragma unroll
    for (int x = 0; x < NCH; ++x) {
      const int id = tid + kFwdThreads * x;
      kreg[x] = *(const bf16x8*)(kt + (id / DC) * HD + (id % DC) * 8);
      vreg[x] = *(const bf16x8*)(vt + (id / DC) * HD + (id % DC) * 8);
    }
    if constexpr (UB == 0) {
      if (tid < urows * (DS / 8)) sreg = *(const bf16x8*)(ksb0 + (size_t)j * urows * DS + tid * 8);
    } else if (!GIVEN && tid < UB * DS / 8) {
      sreg = *(const bf16x8*)(ksb0 + (size_t)j * UB * DS + tid * 8);
    }
  };
  auto sstore = [&](bf16* Kd, bf16* Vd, bf16* Sd) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < NCH; ++x) {
      const int id = tid + kFwdThreads * x;
      *(bf16x8*)&Kd[(id / DC) * KP + (id % DC) * 8] = kreg[x];
      *(bf16x8*)&Vd[(id / DC) * VP + (id % DC) * 8] = vreg[x];
    }
    if constexpr (UB == 0) {
      if (tid < urows * (DS / 8)) *(bf16x8*)&Sd[(tid / (DS / 8)) * XP + (tid % (DS / 8)) * 8] = sreg;
    } else if (!GIVEN && tid < UB * DS / 8) {
      *(bf16x8*)&Sd[tid * 8] = sreg;
    }
  };
  // Key order: A-operand row l32 of the S^T products is key row prow, so
  // accumulator row 8 q + 4 hh + i of a 32-key M-tile holds key 8 q + 2 i + hh.
  // A transposing V^T read then gives each lane half key rows of one parity
  // (0, 2, 4, 6 or 1, 3, 5, 7: bank offsets 16 dwords apart at the 72-dword
  // pitch) instead of four adjacent rows whose 64-byte spans overlap in the
  // LDS banks.  Lane 4k + a of each 16-lane group points at key row 2 k + hh,
  // columns 16 ((lane >> 4) & 1) + 4 a.
  const int vbase = (2 * ((lane & 15) >> 2) + hh) * VP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int prow = (l32 & ~7) | ((l32 & 3) << 1) | ((l32 >> 2) & 1);

  bf16x8 pb[2][2];  // P of the last softmax, the B operand of the PV products

  // Scores and softmax of one key tile (P into pb).  MASK: causal mask and
  // per-lane block test (only the at most two tiles that hold some lane's
  // current block need it).
  auto tile = [&](int j, auto mask_tag, const bf16* Ks, const bf16* Ss)
      __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // log2-domain gate bias of this lane's row for each unit of tile j (UB = 0:
    // zero, the bias is in the score accumulator)
    float bias2[UB > 0 ? UB : 1];
#pragma unroll
    for (int ub = 0; ub < (UB > 0 ? UB : 1); ++ub) bias2[ub] = 0.f;
    if constexpr (GIVEN) {
      bias2[0] = j < c ? bcur * kLog2e : 0.f;
    } else if (UB > 0 && (UB == 1 ? j < c_hi : j <= c_hi)) {
#pragma unroll
      for (int ub = 0; ub < UB; ++ub) {
        const bf16x2* kr = (const bf16x2*)(Ss + ub * DS + hh * (DS / 2));
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < DS / 4; ++e)
          part = __builtin_amdgcn_fdot2_f32_bf16(qsv[e], kr[e], part, false);
        part = halves_sum(part);
        if (j * UB + ub < c) bias2[ub] = (D.sel_scale * part - lam_t) * kLog2e;
      }
    }
    // S^T tile: two 32-key M-tiles x 32 queries
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    if constexpr (UB == 0) {
      // Z^T = KS QS^T: key 32 mt + l32 of the tile reads its unit's ks row.
      // A historical key's logit is sm_scale (s + (sel_scale z - lam) /
      // sm_scale): its accumulator starts at the second term and the key
      // products add s; keys of the row's own unit start at 0.
#pragma unroll
      for (int s = 0; s < DS / 16; ++s) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x8 a = *(const bf16x8*)&Ss[((32 * mt + prow) >> lb) * XP + 16 * s + 8 * hh];
          sacc[mt] = mfma32(a, qsf[s], sacc[mt]);
        }
      }
      const float zoff = -lam_t / D.sm_scale;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float zb = fmaf(sacc[mt][r], zsc, zoff);
          if constexpr (MASK) {
            const int u = j * kBlock + 32 * mt + (r / 4) * 8 + 2 * (r % 4) + hh;
            sacc[mt][r] = u < tcur0 ? zb : 0.f;
          } else {
            sacc[mt][r] = zb;  // every key of a tile before the wave's first block is historical
          }
        }
      }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 a = *(const bf16x8*)&Ks[(32 * mt + prow) * KP + 16 * s + 8 * hh];
        sacc[mt] = mfma32(a, qf[s], sacc[mt]);
      }
    }
    // row max: with one unit per tile on the raw scores (c1 > 0, the bias is
    // constant over the tile); with several, on the biased log2 logits, which
    // then replace the raw scores in sacc
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (MASK) {
          const int u = j * kBlock + 32 * mt + (r / 4) * 8 + 2 * (r % 4) + hh;
          if (u > t) sacc[mt][r] = -INFINITY;
        }
        if constexpr (UB > 1) {
          // unit of key 32 mt + 8 (r / 4) + 2 (r % 4) + hh within the tile
          const int ub = UB == 2 ? mt : 2 * mt + r / 8;
          sacc[mt][r] = fmaf(sacc[mt][r], c1, bias2[ub]);
        }
        mx = fmaxf(mx, sacc[mt][r]);
      }
    }
    mx = halves_max(mx);
    if constexpr (UB <= 1) mx = fmaf(mx, c1, bias2[0]);
    // Lazy rescaling: the running max only moves when it grows by more than
    // 8 (log2 units) in some row of the wave, so P <= 2^8 between updates.
    if (__any(mx > m_run + 8.f)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2_raw(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) oacc[dm] *= alpha;
      m_run = m_new;
    }
    // (m_run is -inf only for a row with no visible key yet: all p are 0)
    const float off = bias2[0] - m_run;
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = UB <= 1 ? exp2_raw(fmaf(sacc[mt][r], c1, off))
                                : exp2_raw(sacc[mt][r] - m_run);
        pb[mt][r / 8][r % 8] = (bf16)p;
        psum += p;
      }
    }
    l_run += psum;
  };
  // O^T += V^T P^T: the B slots of a lane are keys 16 pp + hh + 2 (0..3) and
  // 16 pp + 8 + hh + 2 (0..3) of M-tile mt (accumulator rows 16 pp + 4 hh +
  // (0..3, 8..11)), and the transposing reads give V^T in the same key order
  auto pv = [&](const bf16* Vs) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
#pragma unroll
        for (int dm = 0; dm < DM; ++dm) {
          const bf16* vp = &Vs[vbase + (32 * mt + 16 * pp) * VP + 32 * dm];
          const bf16x4 lo = ds_read_tr(vp);
          const bf16x4 hi = ds_read_tr(vp + 8 * VP);
          const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[dm] = mfma32(a, pb[mt][pp], oacc[dm]);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  auto run = [&](int j) __attribute__((always_inline)) {
    const bf16* Ks = (j & 1) ? K1 : K0;
    const bf16* Ss = (j & 1) ? S1 : S0;
    if (j < c_lo)
      tile(j, std::false_type{}, Ks, Ss);
    else
      tile(j, std::true_type{}, Ks, Ss);
  };
  auto vbuf = [&](int j) __attribute__((always_inline)) {
    const int r = j % 3;
    return r == 0 ? V0 : (r == 1 ? V1 : V2);
  };

  // The two waves of a SIMD belong to different halves of the workgroup
  // (waves 0-3 and 4-7).  Half 0 takes each tile in the order scores,
  // softmax, PV; half 1 runs the PV of the previous tile first, then the
  // scores and softmax of this one.  Between two barriers one half is then
  // in its softmax while the other multiplies for two of the three phases,
  // so the matrix cores and the vector ALUs of a SIMD work at the same time.
  // K tiles alternate between two buffers, V tiles rotate over three (half
  // 1 still reads V of tile j - 1 while tile j + 1 is staged).
  auto loop = [&](auto half_tag) __attribute__((always_inline)) {
    constexpr int H = decltype(half_tag)::value;
    for (int j = 0; j <= c_end; ++j) {
      // (the bias load goes out before the next tile's loads, so waiting for
      // it does not wait for them)
      if constexpr (GIVEN) {
        bcur = bnext;
        bnext = j + 1 < c ? btr[(size_t)(j + 1) * 8] : 0.f;
      }
      if (j + 1 <= c_end) gload(j + 1);
      if constexpr (H == 0) {
        if (j <= c_hi) {
          run(j);
          pv(vbuf(j));
        }
      } else {
        if (j >= 1 && j - 1 <= c_hi) pv(vbuf(j - 1));
        if (j <= c_hi) run(j);
      }
      if (j + 1 <= c_end) sstore((j & 1) ? K0 : K1, vbuf(j + 1), (j & 1) ? S0 : S1);
      __syncthreads();
    }
    if constexpr (H == 1) {
      if (c_end <= c_hi) pv(vbuf(c_end));
    }
  };
  gload(0);
  sstore(K0, V0, S0);
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(tid >> 8) == 0)
    loop(std::integral_constant<int, 0>{});
  else
    loop(std::integral_constant<int, 1>{});

  l_run = halves_sum(l_run);
  if (qi < D.tq) {
    const float inv = 1.f / l_run;
    bf16* orow = o + qrow * HD;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(oacc[dm][4 * rr + e] * inv);
        *(bf16x4*)(orow + 32 * dm + 8 * rr + 4 * hh) = w;
      }
    }
    if (hh == 0 && lse != nullptr) lse[qrow] = (m_run + log2f(l_run)) * kLn2;
  }
}

template <int HD, int DS, int UB, bool GIVEN>
static hipError_t launch_fwd_t(const void* q, const void* k, const void* v, const void* qs,
                               const void* ks, const float* lam, const float* bt, void* o,
                               float* lse, const Dims& D, hipStream_t st) {
  const int nqt = (D.tq + kFwdRows - 1) / kFwdRows;
  const int groups = D.batch * D.hkv;
  const int xcd_groups = groups % 8 == 0 ? groups / 8 : 0;
  const unsigned grid = (unsigned)(D.batch * D.hq * nqt);
  hipLaunchKernelGGL((attn_fwd_kernel<HD, DS, UB, GIVEN>), dim3(grid), dim3(kFwdThreads), 0, st,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)qs,
                     (const bf16*)ks, lam, bt, (bf16*)o, lse, D, nqt, xcd_groups);
  return hipGetLastError();
}

// Sparse forward through the dense kernel: bt [b * hq][nb][tq] holds each
// (row, historical block) bias, -inf where the row does not attend the block.
hipError_t launch_fwd_given_bias(const void* q, const void* k, const void* v, const float* bt,
                                 void* o, float* lse, const Dims& D, hipStream_t st) {
  if (D.blk != kBlock) return hipErrorInvalidValue;
  if (D.d == 128)
    return launch_fwd_t<128, 16, 1, true>(q, k, v, nullptr, nullptr, nullptr, bt, o, lse, D, st);
  if (D.d == 64)
    return launch_fwd_t<64, 16, 1, true>(q, k, v, nullptr, nullptr, nullptr, bt, o, lse, D, st);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, const void* qs,
                           const void* ks, const float* lam, void* o, float* lse, const Dims& D,
                           hipStream_t st) {
#define SAS_FWD_CASE(HDV, DSV)                                                                  \
  if (D.d == HDV && D.ds == DSV) {                                                              \
    if (D.blk == 64)                                                                            \
      return launch_fwd_t<HDV, DSV, 1, false>(q, k, v, qs, ks, lam, nullptr, o, lse, D, st);   \
    if (D.blk == 32)                                                                            \
      return launch_fwd_t<HDV, DSV, 2, false>(q, k, v, qs, ks, lam, nullptr, o, lse, D, st);   \
    if (D.blk == 16)                                                                            \
      return launch_fwd_t<HDV, DSV, 4, false>(q, k, v, qs, ks, lam, nullptr, o, lse, D, st);   \
    if (D.blk == 8 || D.blk == 4 || D.blk == 2 || D.blk == 1)                                   \
      return launch_fwd_t<HDV, DSV, 0, false>(q, k, v, qs, ks, lam, nullptr, o, lse, D, st);   \
    return hipErrorInvalidValue;                                                                \
  }
  SAS_FWD_CASE(128, 32)
  SAS_FWD_CASE(128, 16)
  SAS_FWD_CASE(128, 64)
  SAS_FWD_CASE(64, 32)
  SAS_FWD_CASE(64, 16)
  SAS_FWD_CASE(64, 64)
#undef SAS_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace sas
