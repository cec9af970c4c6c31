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
// Three kernels, chosen by shape (launch_topk_t): a lane per row with the
// best blocks in registers for many rows and K <= 32 (topk_lane_kernel), a
// wave per row with an LDS radix select for budgets and K >= 16 otherwise
// (topk_select_kernel), and the wave-per-row kernel below for the rest.  All
// rank the same fp32 scores (SelQ: packed bf16 products for bf16 inputs, as
// in the gate kernel) in the same order, so they pick the same blocks.
//
// Wave per row: the row's scores are computed once into LDS (lane j % 64
// owns block j), lam comes from a wave max + sum, then K rounds each pick the
// best remaining block with a 64-lane argmax on (z, -j): round r takes the
// best candidate strictly after round r-1's winner in that total order, so
// no "already taken" set is needed.
#include "sas_device.h"
#include "sas_internal.h"

namespace sas {

__device__ __forceinline__ bool better(float za, int ja, float zb, int jb) {
  return za > zb || (za == zb && ja < jb);
}

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
};

template <int DS, typename ST, typename Sel>
__global__ __launch_bounds__(256) void topk_wave_kernel(const ST* __restrict__ qs, Sel S, int K,
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
    const int h = (int)((row / D.tq) % D.hq);
    const int b = (int)(row / ((size_t)D.tq * D.hq));
    const int c = S.hist(D, row);
    SelQ<DS, ST> qsv;
    qsv.load(qs + row * DS);
    float m = -INFINITY;
    for (int j = lane; j < c; j += 64) {
      const ST* kr = S.ks_row(D, b, h, j);
      const float z = kr ? D.sel_scale * qsv.dot(kr) : -INFINITY;
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

// Order-preserving 32-bit key of a score (larger z, larger key; -0 counts as
// +0, as in a floating-point comparison), and the selection order on (key,
// block): key descending, then block ascending.
__device__ __forceinline__ unsigned ord_key(float z) {
  unsigned u = __float_as_uint(z);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
__device__ __forceinline__ bool key_before(unsigned ka, int ja, unsigned kb, int jb) {
  return ka > kb || (ka == kb && ja < jb);
}

// Lane-per-row variant for many rows and K <= 32: the 64 rows of a wave are
// consecutive positions of one (batch, head), so every ks row is a
// wave-uniform load.  Each lane keeps its best KMAX (>= K) blocks in
// registers as 64-bit keys (ord_key of z above, the complement of the block
// below), so that one unsigned comparison gives the selection order (z
// descending, block ascending) and no two candidates tie.  Candidates come in
// batches of 8: the batch is sorted by a 19-comparator network, each of the
// last 8 list entries keeps the larger of itself and its mirror in the batch
// (the list then holds the best KMAX of both, in bitonic order), and a
// bitonic merge sorts it again; every step is branch-free, so the lanes of a
// wave never wait on each other's insertions.  Scores use the same SelQ dot
// product.
__device__ __forceinline__ void ce_desc(unsigned long long& a, unsigned long long& b) {
  const bool sw = b > a;
  const unsigned long long hi = sw ? b : a, lo = sw ? a : b;
  a = hi;
  b = lo;
}

template <int DS, typename ST, int KMAX>
__global__ __launch_bounds__(256) void topk_lane_kernel(const ST* __restrict__ qs,
                                                        const ST* __restrict__ ks, int K,
                                                        int renorm, int* __restrict__ idx,
                                                        float* __restrict__ bias, Dims D) {
  static_assert(KMAX >= 8 && (KMAX & (KMAX - 1)) == 0, "KMAX: a power of two >= 8");
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int wave_first = __builtin_amdgcn_readfirstlane(blockIdx.x * 256 + (threadIdx.x & ~63));
  if (wave_first >= D.tq) return;
  const int ic = min(i, D.tq - 1);
  const int c = (D.qoff + ic) / D.blk;
  const int cw = (D.qoff + min(wave_first + 63, D.tq - 1)) / D.blk;  // wave max of c
  const size_t row = ((size_t)b * D.hq + h) * D.tq + ic;
  SelQ<DS, ST> qsv;
  qsv.load(qs + row * DS);
  const ST* ksb = ks + ((size_t)b * D.hks + h / D.hps) * (size_t)D.nb * DS;
  unsigned long long tk[KMAX];  // best blocks, key descending; 0 = empty
#pragma unroll
  for (int r = 0; r < KMAX; ++r) tk[r] = 0ull;
  float m = -INFINITY, s = 0.f;  // log2-domain running log-sum-exp of z
  for (int j0 = 0; j0 < cw; j0 += 8) {
    float zz[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int j = j0 + kk;
      zz[kk] = (j < cw) ? D.sel_scale * qsv.dot(ksb + (size_t)j * DS) : -INFINITY;
      if (j >= c) zz[kk] = -INFINITY;
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
    // the batch as keys (blocks at or after c: 0, never selected), sorted
    unsigned long long bk[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int j = j0 + kk;
      bk[kk] = j < c ? ((unsigned long long)ord_key(zz[kk]) << 32) | (unsigned)~j : 0ull;
    }
    ce_desc(bk[0], bk[2]); ce_desc(bk[1], bk[3]); ce_desc(bk[4], bk[6]); ce_desc(bk[5], bk[7]);
    ce_desc(bk[0], bk[4]); ce_desc(bk[1], bk[5]); ce_desc(bk[2], bk[6]); ce_desc(bk[3], bk[7]);
    ce_desc(bk[0], bk[1]); ce_desc(bk[2], bk[3]); ce_desc(bk[4], bk[5]); ce_desc(bk[6], bk[7]);
    ce_desc(bk[2], bk[4]); ce_desc(bk[3], bk[5]);
    ce_desc(bk[1], bk[4]); ce_desc(bk[3], bk[6]);
    ce_desc(bk[1], bk[2]); ce_desc(bk[3], bk[4]); ce_desc(bk[5], bk[6]);
    // best KMAX of list and batch: the list descends, the mirrored batch
    // ascends, their larger elements form a bitonic sequence
#pragma unroll
    for (int r = KMAX - 8; r < KMAX; ++r) {
      const unsigned long long o = bk[KMAX - 1 - r];
      tk[r] = o > tk[r] ? o : tk[r];
    }
#pragma unroll
    for (int st = KMAX / 2; st >= 1; st >>= 1)
#pragma unroll
      for (int r = 0; r < KMAX; ++r)
        if ((r & st) == 0) ce_desc(tk[r], tk[r + st]);
  }
  if (i >= D.tq) return;
  const int n = c < K ? c : K;
  float norm = c == 0 ? -INFINITY : (m + log2f(s)) * kLn2;
  if (renorm) {
    float mm = key_value((unsigned)(tk[0] >> 32));
    float ss = 0.f;
#pragma unroll
    for (int r = 0; r < KMAX; ++r)
      if (r < n) ss += exp2f((key_value((unsigned)(tk[r] >> 32)) - mm) * kLog2e);
    norm = n == 0 ? -INFINITY : mm + log2f(ss) * kLn2;
  }
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    if (r < K) {
      idx[row * K + r] = r < n ? (int)~(unsigned)tk[r] : -1;
      bias[row * K + r] = r < n ? key_value((unsigned)(tk[r] >> 32)) - norm : -INFINITY;
    }
  }
}

// Budgeted / large-K variant: one wavefront per query row keeps the
// n_t = min(kmax, c(t), ceil(frac c(t))) best blocks (frac <= 0: no
// fraction).  Scores go to LDS (same SelQ dot product as above) and become
// order-preserving 32-bit keys; a radix select (8 bits per pass, LDS
// histogram) narrows down the n_t-th largest key, stopping early once the bin
// that holds it is needed whole; keys tied with it are taken in block order;
// the n_t winners are then sorted (bitonic network in LDS) by key
// descending, block ascending — the same order as the other kernels.

template <int DS, typename ST>
__global__ __launch_bounds__(256) void topk_select_kernel(const ST* __restrict__ qs,
                                                          const ST* __restrict__ ks, int kmax,
                                                          float frac, int renorm,
                                                          int* __restrict__ idx,
                                                          float* __restrict__ bias, Dims D,
                                                          int kp2, int wpg) {
  extern __shared__ unsigned tsm[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int per = D.nb + 256 + 2 * kp2;
  float* zc = (float*)(tsm + (size_t)wave * per);  // scores of this row's blocks
  unsigned* hist = tsm + (size_t)wave * per + D.nb;  // radix histogram
  unsigned* sk = hist + 256;                         // selected keys
  int* sj = (int*)(sk + kp2);                        // selected blocks
  const size_t nrows = (size_t)D.batch * D.hq * D.tq;
  const size_t row = (size_t)blockIdx.x * wpg + wave;
  if (row >= nrows) return;  // whole wave (no workgroup barrier below)
  const int i = (int)(row % D.tq);
  const int h = (int)((row / D.tq) % D.hq);
  const int b = (int)(row / ((size_t)D.tq * D.hq));
  const int c = (D.qoff + i) / D.blk;
  int n = min(kmax, c);
  if (frac > 0.f) n = min(n, (int)ceil((double)frac * (double)c));
  // scores and the gate normaliser over the whole history
  SelQ<DS, ST> qsv;
  qsv.load(qs + row * DS);
  const ST* ksb = ks + ((size_t)b * D.hks + h / D.hps) * (size_t)D.nb * DS;
  float m = -INFINITY;
  for (int j = lane; j < c; j += 64) {
    const float z = D.sel_scale * qsv.dot(ksb + (size_t)j * DS);
    zc[j] = z;
    m = fmaxf(m, z);
  }
  m = wave_max(m);
  float sum = 0.f;
  if (m != -INFINITY)
    for (int j = lane; j < c; j += 64) sum += exp2f((zc[j] - m) * kLog2e);
  sum = wave_sum(sum);
  const float lam = c == 0 ? -INFINITY : m + log2f(sum) * kLn2;
  // radix select of the n-th largest key
  unsigned prefix = 0, pmask = 0;
  int need = n;
  if (n > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int x = lane; x < 256; x += 64) hist[x] = 0;
      for (int j = lane; j < c; j += 64) {
        const unsigned kk = ord_key(zc[j]);
        if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & 255u], 1u);
      }
      // lane l owns digits 255 - 4l .. 252 - 4l (from the top)
      unsigned cnt[4], tot = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        cnt[u] = hist[255 - 4 * lane - u];
        tot += cnt[u];
      }
      // inclusive prefix of tot over lanes (from the top digit down)
      unsigned inc = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
      }
      const unsigned exc = inc - tot;
      // the digit where the count from the top first reaches need
      int dsel = -1;
      unsigned above = 0, inbin = 0;
      if (exc < (unsigned)need && inc >= (unsigned)need) {
        unsigned run = exc;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (dsel < 0 && run + cnt[u] >= (unsigned)need) {
            dsel = 255 - 4 * lane - u;
            above = run;
            inbin = cnt[u];
          }
          run += cnt[u];
        }
      }
      const unsigned long long bal = __ballot(dsel >= 0);
      const int src = __ffsll((long long)bal) - 1;
      const int dg = __shfl(dsel, src);
      need -= (int)__shfl(above, src);
      prefix |= (unsigned)dg << shift;
      pmask |= 255u << shift;
      // every key of the digit's bin is needed: the selection is settled
      if (__shfl(inbin, src) == (unsigned)need) break;
    }
  }
  // gather: keys whose resolved bits lie above the prefix, then the first
  // `need` keys on it by block (all of them when the passes stopped early)
  int cnt_sel = 0, ties_left = need;
  for (int j0 = 0; j0 < c; j0 += 64) {
    const int j = j0 + lane;
    const unsigned kfull = j < c ? ord_key(zc[j]) : 0u, kk = kfull & pmask;
    const bool above = n > 0 && j < c && kk > prefix;
    const bool tie = n > 0 && j < c && kk == prefix;
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const unsigned long long bt = __ballot(tie);
    const int trank = __popcll(bt & lt);
    const bool take = above || (tie && trank < ties_left);
    const unsigned long long bs = __ballot(take);
    if (take) {
      const int pos = cnt_sel + __popcll(bs & lt);
      sk[pos] = kfull;
      sj[pos] = j;
    }
    cnt_sel += __popcll(bs);
    ties_left -= min(ties_left, __popcll(bt));
  }
  // bitonic sort of the n winners (padded to a power of two with the worst key)
  int p2 = 1;
  while (p2 < n) p2 <<= 1;
  for (int x = n + lane; x < p2; x += 64) {
    sk[x] = 0u;
    sj[x] = 0x7fffffff;
  }
  for (int size = 2; size <= p2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int pr = lane; pr < (p2 >> 1); pr += 64) {
        const int lo = 2 * stride * (pr / stride) + (pr % stride), hi = lo + stride;
        const unsigned ka = sk[lo], kb2 = sk[hi];
        const int ja = sj[lo], jb = sj[hi];
        const bool first_better = key_before(ka, ja, kb2, jb);
        const bool want_better_first = (lo & size) == 0;
        if (first_better != want_better_first) {
          sk[lo] = kb2;
          sk[hi] = ka;
          sj[lo] = jb;
          sj[hi] = ja;
        }
      }
    }
  }
  // outputs
  float norm = lam;
  if (renorm) {
    float mm = -INFINITY;
    for (int r = lane; r < n; r += 64) mm = fmaxf(mm, zc[sj[r]]);
    mm = wave_max(mm);
    float ss = 0.f;
    for (int r = lane; r < n; r += 64) ss += exp2f((zc[sj[r]] - mm) * kLog2e);
    ss = wave_sum(ss);
    norm = n == 0 ? -INFINITY : mm + log2f(ss) * kLn2;
  }
  for (int r = lane; r < kmax; r += 64) {
    if (r < n) {
      const int j = sj[r];
      idx[row * kmax + r] = j;
      bias[row * kmax + r] = zc[j] - norm;
    } else {
      idx[row * kmax + r] = -1;
      bias[row * kmax + r] = -INFINITY;
    }
  }
}

template <int DS, typename ST>
static hipError_t launch_select_t(const void* qs, const void* ks, int kmax, float frac, int renorm,
                                  int* idx, float* bias, const Dims& D, hipStream_t st) {
  int kp2 = 1;
  while (kp2 < kmax) kp2 <<= 1;
  const size_t per = (size_t)(D.nb + 256 + 2 * kp2) * sizeof(unsigned);
  int wpg = 4;  // rows (waves) per workgroup, as many as 64 KiB of LDS holds
  while (wpg > 1 && per * wpg > 65536) wpg >>= 1;
  const size_t nrows = (size_t)D.batch * D.hq * D.tq;
  hipLaunchKernelGGL((topk_select_kernel<DS, ST>), dim3((unsigned)((nrows + wpg - 1) / wpg)),
                     dim3(64 * wpg), per * wpg, st, (const ST*)qs, (const ST*)ks, kmax, frac,
                     renorm, idx, bias, D, kp2, wpg);
  return hipGetLastError();
}

bool topk_budget_supported(const Dims& D, int kmax) {
  int kp2 = 1;
  while (kp2 < kmax) kp2 <<= 1;
  return kmax <= 1024 && (size_t)(D.nb + 256 + 2 * kp2) * sizeof(unsigned) <= 65536;
}

hipError_t launch_topk_budget(const void* qs, const void* ks, int kmax, float frac, int renorm,
                              int* idx, float* bias, const Dims& D, bool sel_bf16,
                              hipStream_t st) {
#define SAS_SEL_CASE(DSV)                                                                     \
  case DSV:                                                                                   \
    return sel_bf16 ? launch_select_t<DSV, bf16>(qs, ks, kmax, frac, renorm, idx, bias, D, st) \
                    : launch_select_t<DSV, float>(qs, ks, kmax, frac, renorm, idx, bias, D, st);
  switch (D.ds) {
    SAS_SEL_CASE(16)
    SAS_SEL_CASE(32)
    SAS_SEL_CASE(64)
  }
#undef SAS_SEL_CASE
  return hipErrorInvalidValue;
}

// The lane-per-row kernel needs no LDS: many rows, K <= 32.
static bool use_lane_kernel(const Dims& D, int K) {
  const size_t nrows = (size_t)D.batch * D.hq * D.tq;
  return nrows >= 16384 && K <= 32 && D.hq <= 65535 && D.batch <= 65535;
}

template <int DS, typename ST>
static hipError_t launch_topk_t(const void* qs, const void* ks, int K, int renorm, int* idx,
                                float* bias, const Dims& D, hipStream_t st) {
  if (use_lane_kernel(D, K)) {
    dim3 grid((D.tq + 255) / 256, D.hq, D.batch);
    if (K <= 8)
      hipLaunchKernelGGL((topk_lane_kernel<DS, ST, 8>), grid, dim3(256), 0, st, (const ST*)qs,
                         (const ST*)ks, K, renorm, idx, bias, D);
    else if (K <= 16)
      hipLaunchKernelGGL((topk_lane_kernel<DS, ST, 16>), grid, dim3(256), 0, st, (const ST*)qs,
                         (const ST*)ks, K, renorm, idx, bias, D);
    else
      hipLaunchKernelGGL((topk_lane_kernel<DS, ST, 32>), grid, dim3(256), 0, st, (const ST*)qs,
                         (const ST*)ks, K, renorm, idx, bias, D);
    return hipGetLastError();
  }
  // K >= 16: the radix-select kernel (same order and tie rule, frac = 0) costs
  // a few passes over a row's scores instead of K argmax rounds
  if (K >= 16 && topk_budget_supported(D, K))
    return launch_select_t<DS, ST>(qs, ks, K, 0.f, renorm, idx, bias, D, st);
  const size_t per = (size_t)(D.nb + K) * sizeof(float);
  int wpg = 4;
  while (wpg > 1 && per * wpg > 65536) wpg >>= 1;
  if (per * wpg > 65536) return hipErrorInvalidValue;
  const size_t nrows = (size_t)D.batch * D.hq * D.tq;
  const unsigned grid = (unsigned)((nrows + wpg - 1) / wpg);
  hipLaunchKernelGGL((topk_wave_kernel<DS, ST, DenseSel<ST>>), dim3(grid), dim3(64 * wpg),
                     per * wpg, st, (const ST*)qs, DenseSel<ST>{(const ST*)ks}, K, renorm, idx,
                     bias, D, wpg);
  return hipGetLastError();
}

template <int DS, typename ST>
static hipError_t launch_paged_topk_t(const void* qs, const void* ks_pool, const int* table,
                                      const int* lens, int pages, int K, int renorm, int* idx,
                                      float* bias, const Dims& D, hipStream_t st) {
  const size_t per = (size_t)(D.nb + K) * sizeof(float);
  int wpg = 4;
  while (wpg > 1 && per * wpg > 65536) wpg >>= 1;
  if (per * wpg > 65536) return hipErrorInvalidValue;
  const size_t nrows = (size_t)D.batch * D.hq;
  const unsigned grid = (unsigned)((nrows + wpg - 1) / wpg);
  hipLaunchKernelGGL((topk_wave_kernel<DS, ST, PagedSel<ST>>), dim3(grid), dim3(64 * wpg),
                     per * wpg, st, (const ST*)qs,
                     PagedSel<ST>{(const ST*)ks_pool, table, lens, pages}, K, renorm, idx, bias,
                     D, wpg);
  return hipGetLastError();
}

hipError_t launch_paged_topk(const void* qs, const void* ks_pool, const int* table,
                             const int* lens, int pages, int K, int renorm, int* idx, float* bias,
                             const Dims& D, bool sel_bf16, hipStream_t st) {
#define SAS_PTOPK_CASE(DSV)                                                                  \
  case DSV:                                                                                  \
    return sel_bf16 ? launch_paged_topk_t<DSV, bf16>(qs, ks_pool, table, lens, pages, K,     \
                                                     renorm, idx, bias, D, st)               \
                    : launch_paged_topk_t<DSV, float>(qs, ks_pool, table, lens, pages, K,    \
                                                      renorm, idx, bias, D, st);
  switch (D.ds) {
    SAS_PTOPK_CASE(16)
    SAS_PTOPK_CASE(32)
    SAS_PTOPK_CASE(64)
  }
#undef SAS_PTOPK_CASE
  return hipErrorInvalidValue;
}

bool topk_supported(const Dims& D, int K) {
  return use_lane_kernel(D, K) || (K >= 16 && topk_budget_supported(D, K)) ||
         (size_t)(D.nb + K) * sizeof(float) <= 65536;
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
