// select_device.h -- row-selection helpers shared by the top-K kernels and
// the fused decode kernel: where a row's selector keys live, the 64-bit
// selection keys, and the best-K of one row by one wavefront.
#pragma once
#include "sas_device.h"

namespace sas {

// Where a row's selector keys live.  DenseSel: contiguous [B, Hks, NB, ds]
// rows, row t has c(t) = t / 64 historical blocks.  PagedSel: one ks row per
// page in a pool [pages, Hks, ds], a sequence's block j on page
// table[b, j]; the decode row of sequence b sits at t = len[b] - 1.  A row
// with a length out of range has no history; a block whose page id is out of
// range is never read and scores -inf.
template <typename ST>
struct DenseSel {
  const ST* ks;
  __device__ int hist(const Dims& D, size_t row) const {
    return (D.qoff + (int)(row % D.tq)) / D.blk;
  }
  __device__ const ST* ks_row(const Dims& D, int b, int h, int j) const {
    return ks + (((size_t)b * D.hks + h / D.hps) * (size_t)D.nb + j) * D.ds;
  }
  // A row that may always be read for block j (0 <= j < nb) and whether it
  // is block j's selector key (always, for a contiguous cache).
  __device__ const ST* ks_row_readable(const Dims& D, int b, int h, int j, bool* own) const {
    *own = true;
    return ks_row(D, b, h, j);
  }
};

template <typename ST>
struct PagedSel {
  const ST* ks;
  const int* table;
  const int* lens;
  int pages;
  __device__ int hist(const Dims& D, size_t row) const {
    const int len = lens[row / D.hq];
    return (len >= 1 && len <= D.nb * kBlock) ? (len - 1) / kBlock : 0;
  }
  __device__ const ST* ks_row(const Dims& D, int b, int h, int j) const {
    const int pg = table[(size_t)b * D.nb + j];
    if (pg < 0 || pg >= pages) return nullptr;
    return ks + ((size_t)pg * D.hks + h / D.hps) * D.ds;
  }
  // A row that may always be read for block j: its page's, or page 0's
  // (pages >= 1) when the page id is out of range (*own false then).
  __device__ const ST* ks_row_readable(const Dims& D, int b, int h, int j, bool* own) const {
    const int pg = table[(size_t)b * D.nb + j];
    *own = pg >= 0 && pg < pages;
    return ks + ((size_t)(*own ? pg : 0) * D.hks + h / D.hps) * D.ds;
  }
};

// A selector key row held in registers, loaded ahead of its dot product
// (16-byte loads), scored with exactly the operations of SelQ::dot in the
// same order, so the score is the same number.
template <int DS, typename ST>
struct KsRow;
template <int DS>
struct KsRow<DS, bf16> {
  bf16x8 x[DS / 8];
  __device__ __forceinline__ void load(const bf16* p) {
#pragma unroll
    for (int c = 0; c < DS / 8; ++c) x[c] = *(const bf16x8*)(p + 8 * c);
  }
  __device__ __forceinline__ float dot(const SelQ<DS, bf16>& q) const {
    typedef __bf16 pair_t __attribute__((ext_vector_type(2)));
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < DS / 2; ++e) {
      const pair_t pr = {x[e / 4][2 * (e % 4)], x[e / 4][2 * (e % 4) + 1]};
      acc = __builtin_amdgcn_fdot2_f32_bf16(q.v[e], pr, acc, false);
    }
    return acc;
  }
};
template <int DS>
struct KsRow<DS, float> {
  f32x4 x[DS / 4];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int c = 0; c < DS / 4; ++c) x[c] = *(const f32x4*)(p + 4 * c);
  }
  __device__ __forceinline__ float dot(const SelQ<DS, float>& q) const {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < DS; ++e) acc = fmaf(q.v[e], x[e / 4][e % 4], acc);
    return acc;
  }
};

// Order-preserving 32-bit key of a score (larger z, larger key; -0 counts as
// +0, as in a floating-point comparison), and the selection order on (key,
// block): key descending, then block ascending.
__device__ __forceinline__ unsigned ord_key(float z) {
  const unsigned u = __float_as_uint(z + 0.0f);  // -0 + 0 = +0
  return u ^ ((unsigned)((int)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key_value(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
__device__ __forceinline__ bool key_before(unsigned ka, int ja, unsigned kb, int jb) {
  return ka > kb || (ka == kb && ja < jb);
}

// Compare-exchange of two selection keys into descending order.
__device__ __forceinline__ void ce_desc(unsigned long long& a, unsigned long long& b) {
  const unsigned long long hi = b > a ? b : a;
  // the other one, a ^ b ^ hi: a three-input XOR (v_bitop3, table 0x96) per
  // half, where a second 64-bit comparison would cost one more instruction
  const unsigned lo0 = __builtin_amdgcn_bitop3_b32((unsigned)a, (unsigned)b, (unsigned)hi, 0x96);
  const unsigned lo1 = __builtin_amdgcn_bitop3_b32((unsigned)(a >> 32), (unsigned)(b >> 32),
                                                   (unsigned)(hi >> 32), 0x96);
  b = ((unsigned long long)lo1 << 32) | lo0;
  a = hi;
}

// The best KM blocks of one query row by one wavefront (few rows: decode,
// paged decode, small calls) among blocks first, first + stride, ... below
// c(t) (a wave alone: first = lane, stride = 64; W waves of a row: first =
// 64 w + lane, stride = 64 W): each lane folds its candidates in batches of
// 8 into a sorted list of its best KM keys (ord_key of z above, the
// complemented block below: one unsigned comparison gives z descending,
// block ascending; the batch sorted by a 19-comparator network, each of the
// list's last 8 entries keeps the larger of itself and its mirror in the
// batch, a bitonic merge sorts again), and six butterfly steps (lane l with
// l ^ 1, ^ 2, ..., ^ 32) leave every lane with the wave's best KM.  The
// log-sum-exp of the scores is kept per lane (log2 domain: *m, *s).  Scores
// use SelQ, as every selection kernel does.
template <int KM>
__device__ __forceinline__ void merge_desc(unsigned long long (&tk)[KM],
                                           const unsigned long long (&other)[KM]) {
  // the best KM of two descending lists: the larger of each entry and its
  // mirror (a bitonic sequence), sorted again
#pragma unroll
  for (int r = 0; r < KM; ++r) tk[r] = other[KM - 1 - r] > tk[r] ? other[KM - 1 - r] : tk[r];
#pragma unroll
  for (int st = KM / 2; st >= 1; st >>= 1)
#pragma unroll
    for (int r = 0; r < KM; ++r)
      if ((r & st) == 0) ce_desc(tk[r], tk[r + st]);
}

// One butterfly step: lane l merges its list with lane l ^ O's.
template <int O, int KM>
__device__ __forceinline__ void merge_lanes(unsigned long long (&tk)[KM], int lane) {
  unsigned long long p[KM];
#pragma unroll
  for (int r = 0; r < KM; ++r) p[r] = lane_xor_u64<O>(tk[r], lane);
  merge_desc<KM>(tk, p);
}

template <int DS, typename ST, typename Sel, int KM, int RIF = 4>
__device__ __forceinline__ void wave_best(const ST* __restrict__ qs, const Sel& S, const Dims& D,
                                          size_t row, int c, int first, int stride,
                                          unsigned long long (&tk)[KM], float* m_out,
                                          float* s_out) {
  const int h = (int)((row / D.tq) % D.hq);
  const int b = (int)(row / ((size_t)D.tq * D.hq));
  SelQ<DS, ST> qsv;
  qsv.load(qs + row * DS);
#pragma unroll
  for (int r = 0; r < KM; ++r) tk[r] = 0ull;  // 0 = empty
  float m = -INFINITY, s = 0.f;
  for (int j0 = first; j0 < c; j0 += stride * 8) {
    // the batch's rows are read without branches, RIF at a time, so that
    // RIF rows' loads are in flight together: a candidate past the history
    // reads block c - 1 and one on an unreadable page reads a readable row;
    // both score -inf
    static_assert(RIF == 1 || RIF == 2 || RIF == 4 || RIF == 8, "rows in flight");
    float zz[8];
#pragma unroll
    for (int k4 = 0; k4 < 8; k4 += RIF) {
      const ST* kr[RIF];
      bool own[RIF];
#pragma unroll
      for (int kk = 0; kk < RIF; ++kk) {
        const int j = j0 + stride * (k4 + kk);
        kr[kk] = S.ks_row_readable(D, b, h, j < c ? j : c - 1, &own[kk]);
        own[kk] = own[kk] && j < c;
      }
      KsRow<DS, ST> rv[RIF];
#pragma unroll
      for (int kk = 0; kk < RIF; ++kk) rv[kk].load(kr[kk]);
      __builtin_amdgcn_sched_barrier(0);  // the group's loads before its products
#pragma unroll
      for (int kk = 0; kk < RIF; ++kk) {
        const float z = D.sel_scale * rv[kk].dot(qsv);
        zz[k4 + kk] = own[kk] ? z : -INFINITY;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    float mc = zz[0];
#pragma unroll
    for (int kk = 1; kk < 8; ++kk) mc = fmaxf(mc, zz[kk]);
    const float mn = fmaxf(m, mc * kLog2e);
    if (mn != -INFINITY) {
      float acc = s * exp2f(m - mn);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) acc += exp2f(zz[kk] * kLog2e - mn);
      s = acc;
      m = mn;
    }
    unsigned long long bk[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int j = j0 + stride * kk;
      bk[kk] = j < c ? ((unsigned long long)ord_key(zz[kk]) << 32) | (unsigned)~j : 0ull;
    }
    ce_desc(bk[0], bk[2]); ce_desc(bk[1], bk[3]); ce_desc(bk[4], bk[6]); ce_desc(bk[5], bk[7]);
    ce_desc(bk[0], bk[4]); ce_desc(bk[1], bk[5]); ce_desc(bk[2], bk[6]); ce_desc(bk[3], bk[7]);
    ce_desc(bk[0], bk[1]); ce_desc(bk[2], bk[3]); ce_desc(bk[4], bk[5]); ce_desc(bk[6], bk[7]);
    ce_desc(bk[2], bk[4]); ce_desc(bk[3], bk[5]);
    ce_desc(bk[1], bk[4]); ce_desc(bk[3], bk[6]);
    ce_desc(bk[1], bk[2]); ce_desc(bk[3], bk[4]); ce_desc(bk[5], bk[6]);
#pragma unroll
    for (int r = KM - 8; r < KM; ++r) {
      const unsigned long long o = bk[KM - 1 - r];
      tk[r] = o > tk[r] ? o : tk[r];
    }
#pragma unroll
    for (int st = KM / 2; st >= 1; st >>= 1)
#pragma unroll
      for (int r = 0; r < KM; ++r)
        if ((r & st) == 0) ce_desc(tk[r], tk[r + st]);
  }
  // merge the wave's 64 lists (partners by register exchanges)
  const int lane = __lane_id();
  merge_lanes<1, KM>(tk, lane);
  merge_lanes<2, KM>(tk, lane);
  merge_lanes<4, KM>(tk, lane);
  merge_lanes<8, KM>(tk, lane);
  merge_lanes<16, KM>(tk, lane);
  merge_lanes<32, KM>(tk, lane);
  *m_out = m;
  *s_out = s;
}

// Entry r = lane (< K) of a row's selection from its best-KM list and the
// log2-domain log-sum-exp (M, Ssum) of all its scores: *j (-1 past min(c, K))
// and *bs (z - lam, or z - log sum over the kept blocks of exp z when
// renorm; -inf past min(c, K)).
template <int KM>
__device__ __forceinline__ void select_entry(const unsigned long long (&tk)[KM], float M,
                                             float Ssum, int c, int K, int renorm, int lane,
                                             int* j_out, float* bs_out) {
  const int n = c < K ? c : K;
  float norm = c == 0 ? -INFINITY : (M + log2f(Ssum)) * kLn2;
  if (renorm) {
    const float mm = key_value((unsigned)(tk[0] >> 32));
    float ss = 0.f;
#pragma unroll
    for (int r = 0; r < KM; ++r)
      if (r < n) ss += exp2f((key_value((unsigned)(tk[r] >> 32)) - mm) * kLog2e);
    norm = n == 0 ? -INFINITY : mm + log2f(ss) * kLn2;
  }
  unsigned long long mine = 0ull;
#pragma unroll
  for (int r = 0; r < KM; ++r)
    if (lane == r) mine = tk[r];
  *j_out = lane < n ? (int)~(unsigned)mine : -1;
  *bs_out = lane < n ? key_value((unsigned)(mine >> 32)) - norm : -INFINITY;
}

// One wave selects a row alone (RIF: selector rows in flight per lane).
template <int DS, typename ST, typename Sel, int KM, int RIF = 4>
__device__ __forceinline__ void wave_best_entry(const ST* __restrict__ qs, const Sel& S,
                                                const Dims& D, size_t row, int K, int renorm,
                                                int lane, int* j_out, float* bs_out) {
  const int c = S.hist(D, row);
  unsigned long long tk[KM];
  float m, s;
  wave_best<DS, ST, Sel, KM, RIF>(qs, S, D, row, c, lane, 64, tk, &m, &s);
  const float M = wave_max(m);
  const float Ssum = wave_sum(M == -INFINITY ? 0.f : s * exp2f(m - M));
  select_entry<KM>(tk, M, Ssum, c, K, renorm, lane, j_out, bs_out);
}

}  // namespace sas
