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
// Row path (decode, and any shape with units below 64 tokens): one workgroup
// per query row whose waves take the row's slots (the K listed blocks and the
// current block) and merge their online softmax states by log-sum-exp in LDS
// (sparse_row_kernel).  Entries of idx that are not blocks before c(t) are
// skipped, so no out-of-range block is ever read.
//
// Block-stationary path (prefill, tq >= 128, 64-token blocks): selection is
// per token, so the rows of a query tile pick nearly disjoint blocks and a
// per-tile union of blocks would stream almost all of K/V.  Instead the
// (row, slot) pairs are inverted into per-(batch, kv head, block) lists
// (count, scan, scatter); a chunk of up to 128 pairs of one list (or 128
// rows of one query block, for the current blocks) loads that block's K and
// V once, gathers the rows and runs S^T = K Q^T and O^T = V^T P^T on the MFMA
// units, writing a normalised partial and its log-sum-exp per pair; a merge
// kernel folds each row's partials by log-sum-exp.
#include "sas_device.h"
#include "sas_internal.h"
#include "select_device.h"

#include <algorithm>

namespace sas {

static size_t align256s(size_t x) { return (x + 255) & ~(size_t)255; }

// Where a row's keys live.  DenseKV: contiguous [B, Hkv, Tk, d] caches, row
// i of the query block at t = q_off + i.  PagedKV: pools [pages, Hkv, 64, d]
// (one 64-key block per page, 16 KB per head at d = 128), a sequence's block
// j on page table[b, j], its decode row at t = len[b] - 1.  A row whose length
// is out of range has no keys (t = -1); a block whose page id is out of range
// is never read.
template <int HD, typename T>
struct DenseKV {
  const T* k;
  const T* v;
  __device__ int t_of(const Dims& D, size_t row) const { return D.qoff + (int)(row % D.tq); }
  // element offset of block j of (b, kv head g) in k and v; -1: not readable
  __device__ long long block(const Dims& D, int b, int g, int j) const {
    return (long long)((((size_t)b * D.hkv + g) * D.tk + (size_t)j * D.blk) * HD);
  }
};

template <int HD, typename T>
struct PagedKV {
  const T* k;
  const T* v;
  const int* table;
  const int* lens;
  int pages;
  __device__ int t_of(const Dims& D, size_t row) const {
    const int len = lens[row / D.hq];
    return (len >= 1 && len <= D.nb * kBlock) ? len - 1 : -1;
  }
  __device__ long long block(const Dims& D, int b, int g, int j) const {
    const int pg = table[(size_t)b * D.nb + j];
    if (pg < 0 || pg >= pages) return -1;
    return (long long)(((size_t)pg * D.hkv + g) * kBlock * HD);
  }
};

// Row kernel (decode, and prefill with units below 64 tokens): one workgroup
// per query row, W = min(K + 1, 8) waves for K <= 8, else min(K + 1, 16);
// the last wave takes the current block (slot K) first, wave w the listed
// slots w, w + W, ...  K and V rows are read with 16-byte loads,
// LPK lanes per key row (a key row of d elements is LPK * 16 bytes), so one
// load instruction covers KPI = 64 / LPK whole consecutive rows.  A lane's
// partial dot product is summed over the key's LPK lanes; scores go through
// LDS for the softmax; each wave keeps an online (max, sum, P V) over its
// slots, and the waves' results are merged by their log-sum-exp in LDS.
constexpr int kRowWaves = 16;

// Slots of a row read from the idx / bias arrays.
struct GlobalSlots {
  const int* idx;
  const float* bias;
  __device__ void get(size_t row, int K, int slot, int* j, float* add) const {
    *j = idx[row * K + slot];
    *add = bias[row * K + slot];
  }
};

// LDS used by attend_row.
template <int HD>
struct RowLds {
  float ps[kRowWaves][64];
  float ow[kRowWaves][HD];
  float mw[kRowWaves], lw[kRowWaves];
};

// One whole 64-key block of a row by one wave, the online softmax state
// (m_w, l_w, acc) updated in place.  Every load of the block is issued
// without a branch (a whole block has no key past its end): the NIN load
// instructions of K, then those of V, so a wave waits for memory about
// twice per block instead of once per instruction.  Lane l holds keys
// it * KPI + l / LPK (it < NIN) of K and of V alike; after the sum over a
// key's LPK lanes (an all-reduce, so each of them holds the score) the
// lane's probabilities are exactly the ones its V rows need, and the scores
// never go through LDS.
template <int HD, typename T, typename Src>
__device__ __forceinline__ void attend_block64(const Src& S, long long boff, const float* qv,
                                               int kl, int d0, int j, int t, float add,
                                               float sm_scale, float& m_w, float& l_w,
                                               float* acc) {
  constexpr int EPL = 16 / (int)sizeof(T);
  constexpr int LPK = HD / EPL;
  constexpr int KPI = 64 / LPK;
  constexpr int NIN = kBlock / KPI;
  typedef T vec_t __attribute__((ext_vector_type(EPL)));
  const T* kb = S.k + boff + (size_t)kl * HD + d0;
  const T* vb = S.v + boff + (size_t)kl * HD + d0;
  vec_t kx[NIN];
#pragma unroll
  for (int it = 0; it < NIN; ++it) kx[it] = *(const vec_t*)(kb + (size_t)it * KPI * HD);
  float sc[NIN];
#pragma unroll
  for (int it = 0; it < NIN; ++it) {
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) a = fmaf(qv[e], to_f32(kx[it][e]), a);
    sc[it] = a;
  }
  vec_t vx[NIN];
#pragma unroll
  for (int it = 0; it < NIN; ++it) vx[it] = *(const vec_t*)(vb + (size_t)it * KPI * HD);
  float mloc = -INFINITY;
#pragma unroll
  for (int it = 0; it < NIN; ++it) {
    const float a = group_sum<LPK>(sc[it]);
    sc[it] = (j * kBlock + it * KPI + kl > t) ? -INFINITY : a * sm_scale + add;
    mloc = fmaxf(mloc, sc[it]);
  }
  // the lanes of a key group hold equal values, so the wave max is the
  // block's and a sum over lanes l ^ LPK, l ^ 2 LPK, ... counts each key once
  const float ms = wave_max(mloc);
  if (ms == -INFINITY) return;  // every key masked (a bias of -inf)
  const float m_new = fmaxf(m_w, ms);
  const float alpha = exp2f((m_w - m_new) * kLog2e);
  float ls = 0.f;
#pragma unroll
  for (int it = 0; it < NIN; ++it) {
    sc[it] = exp2f((sc[it] - m_new) * kLog2e);
    ls += sc[it];
  }
  l_w = l_w * alpha + stride_sum<LPK>(ls);
  m_w = m_new;
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
#pragma unroll
  for (int it = 0; it < NIN; ++it)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = fmaf(sc[it], to_f32(vx[it][e]), acc[e]);
}

// Whether rows of HD elements of T take attend_block64 for whole 64-key
// blocks: bf16 rows (at most 16 load instructions per block and tensor; fp32
// rows would spill).
template <int HD, typename T>
constexpr bool whole_blocks_fit() {
  return sizeof(T) == 2 && kBlock / (64 / (HD / (16 / (int)sizeof(T)))) <= 16;
}

// Attention of one query row over its K slots and its current block (slot
// K), W waves per row; every thread of the workgroup calls it.  WHOLE: every
// unit is a whole 64-key block (D.blk == 64), taken by attend_block64; the
// launch picks it, so the kernel for smaller units keeps its own (smaller)
// register budget.
template <int HD, typename T, bool WHOLE, typename Src, typename Slots>
__device__ __forceinline__ void attend_row(const T* __restrict__ q, const Src& S,
                                           const Slots& SL, T* __restrict__ o,
                                           float* __restrict__ lse, const Dims& D, int K,
                                           size_t row, int W, RowLds<HD>& L, bool early) {
  constexpr int EPL = 16 / (int)sizeof(T);  // elements per lane and load
  constexpr int LPK = HD / EPL;             // lanes per key row
  constexpr int KPI = 64 / LPK;             // key rows per load instruction
  typedef T vec_t __attribute__((ext_vector_type(EPL)));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = (int)((row / D.tq) % D.hq);
  const int b = (int)(row / ((size_t)D.tq * D.hq));
  const int t = S.t_of(D, row);
  const int B = D.blk;  // keys per block
  const int c = t < 0 ? -1 : t / B;
  const int g = h / D.hpg;
  const int kl = lane / LPK;          // key of this lane within a load instruction
  const int d0 = (lane % LPK) * EPL;  // its first column
  float qv[EPL];
  {
    const vec_t x = *(const vec_t*)(q + row * HD + d0);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[e] = to_f32(x[e]);
  }
  const int nin = (B + KPI - 1) / KPI;  // load instructions per block
  float m_w = -INFINITY, l_w = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  float* const pw = L.ps[wave];
  // The last wave takes the current block (slot K) first; historical slot s
  // goes to wave s % W, in ascending order.  early (fused selection): the
  // slots are published by a barrier that each wave passes exactly once,
  // before its first historical slot or after its last slot, so the wave of
  // the current block attends it while wave 0 is still selecting.
  const bool has_cur = wave == W - 1;
  const int n_hist = wave < K ? (K - 1 - wave) / W + 1 : 0;
  const int n_slots = t >= 0 ? n_hist + (has_cur ? 1 : 0) : 0;
  bool synced = !early;
  for (int n = 0; n < n_slots; ++n) {
    const bool cur = has_cur && n == 0;
    int j;
    float add;
    if (!cur) {
      if (!synced) {  // wave-uniform
        __syncthreads();
        synced = true;
      }
      SL.get(row, K, wave + (n - (has_cur ? 1 : 0)) * W, &j, &add);
      if (j < 0 || j >= c) continue;  // not a historical block: skipped, never read
    } else {
      j = c;
      add = 0.f;
    }
    const long long boff = S.block(D, b, g, j);
    if (boff < 0) continue;
    if constexpr (WHOLE) {  // whole 64-key blocks: every load of the block in flight
      static_assert(whole_blocks_fit<HD, T>(), "bf16 rows of at most 16 loads per block");
      attend_block64<HD, T>(S, boff, qv, kl, d0, j, t, add, D.sm_scale, m_w, l_w, acc);
      continue;
    }
    for (int it = 0; it < nin; ++it) {
      const int u = it * KPI + kl;
      float a = 0.f;
      if (u < B) {
        const vec_t x = *(const vec_t*)(S.k + boff + (size_t)u * HD + d0);
#pragma unroll
        for (int e = 0; e < EPL; ++e) a = fmaf(qv[e], to_f32(x[e]), a);
      }
      a = group_sum<LPK>(a);
      if (lane % LPK == 0 && u < B) pw[u] = (j * B + u > t) ? -INFINITY : a * D.sm_scale + add;
    }
    __builtin_amdgcn_wave_barrier();
    const float sc = lane < B ? pw[lane] : -INFINITY;
    const float ms = group_max<64>(sc);
    if (ms == -INFINITY) continue;  // every key masked (a bias of -inf)
    const float m_new = fmaxf(m_w, ms);
    const float alpha = exp2f((m_w - m_new) * kLog2e);
    const float pl = exp2f((sc - m_new) * kLog2e);
    l_w = l_w * alpha + group_sum<64>(pl);
    m_w = m_new;
    __builtin_amdgcn_wave_barrier();
    if (lane < B) pw[lane] = pl;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
    for (int it = 0; it < nin; ++it) {
      const int u = it * KPI + kl;
      if (u < B) {
        const float pu = pw[u];
        const vec_t x = *(const vec_t*)(S.v + boff + (size_t)u * HD + d0);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pu, to_f32(x[e]), acc[e]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  if (!synced) __syncthreads();
  // sum this wave's P V over its key groups, then merge the waves
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = stride_sum<LPK>(acc[e]);
  if (lane < LPK) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) L.ow[wave][d0 + e] = acc[e];
  }
  if (lane == 0) {
    L.mw[wave] = m_w;
    L.lw[wave] = l_w;
  }
  __syncthreads();
  if (wave != 0) return;
  float M = -INFINITY;
  for (int w = 0; w < W; ++w) M = fmaxf(M, L.mw[w]);
  if (M == -INFINITY) {  // no readable key: zeros, lse -inf
    if (lane < LPK) {
      vec_t z;
#pragma unroll
      for (int e = 0; e < EPL; ++e) z[e] = from_f32<T>(0.f);
      *(vec_t*)(o + row * HD + d0) = z;
    }
    if (lane == 0 && lse) lse[row] = -INFINITY;
    return;
  }
  float Ls = 0.f, out[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) out[e] = 0.f;
  for (int w = 0; w < W; ++w) {
    if (L.mw[w] == -INFINITY) continue;
    const float sw = exp2f((L.mw[w] - M) * kLog2e);
    Ls += L.lw[w] * sw;
    if (lane < LPK) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) out[e] = fmaf(sw, L.ow[w][d0 + e], out[e]);
    }
  }
  if (lane < LPK) {
    const float inv = 1.f / Ls;
    vec_t r;
#pragma unroll
    for (int e = 0; e < EPL; ++e) r[e] = from_f32<T>(out[e] * inv);
    *(vec_t*)(o + row * HD + d0) = r;
  }
  if (lane == 0 && lse) lse[row] = M + logf(Ls);
}


// Row of workgroup L of n (one row per workgroup).  Consecutive workgroups
// run on different XCDs (workgroup L on XCD L % 8); with n % 8 == 0 XCD x is
// given the contiguous rows x n / 8 .. (x + 1) n / 8 - 1, i.e. whole
// sequences, so each XCD's address translation caches and L2 hold the K / V
// pages of a few sequences instead of all of them.
__device__ __forceinline__ size_t xcd_row(size_t L, size_t n) {
  return n % 8 ? L : (L % 8) * (n / 8) + L / 8;
}

template <int HD, typename T, typename Src, bool WHOLE>
__global__ __launch_bounds__(64 * kRowWaves) void sparse_row_kernel(
    const T* __restrict__ q, Src S, const int* __restrict__ idx, const float* __restrict__ bias,
    T* __restrict__ o, float* __restrict__ lse, Dims D, int K) {
  __shared__ RowLds<HD> L;
  attend_row<HD, T, WHOLE>(q, S, GlobalSlots{idx, bias}, o, lse, D, K,
                           xcd_row(blockIdx.x, gridDim.x), blockDim.x >> 6, L, false);
}

// Slots of a row chosen in the same workgroup (LDS).
struct LdsSlots {
  const int* j;
  const float* b;
  __device__ void get(size_t, int, int slot, int* jj, float* add) const {
    *jj = j[slot];
    *add = b[slot];
  }
};

// Selection and attention of a row in one workgroup (decode): wave 0 picks
// the row's K <= KM blocks (wave_best_entry, the routine sas_topk_blocks and
// sas_paged_topk use for few rows) into LDS and optionally writes idx / bias;
// then every wave attends its slots as the row kernel does, the wave of the
// current block (which needs no selection) starting on it while wave 0
// selects.  One launch, and no round trip of the selection through global
// memory.  (Splitting the
// scoring over all the row's waves and merging their lists in LDS was
// slower: the selection is not what bounds this kernel.)
template <int HD, typename T, int DS, int KM, typename Sel, typename Src, bool WHOLE>
__global__ __launch_bounds__(64 * kRowWaves) void topk_row_kernel(
    const T* __restrict__ q, Src S, const T* __restrict__ qs, Sel SS, int K, int renorm,
    int* __restrict__ idx, float* __restrict__ bias, T* __restrict__ o, float* __restrict__ lse,
    Dims D) {
  __shared__ RowLds<HD> L;
  __shared__ int sj[KM];
  __shared__ float sb[KM];
  const size_t row = xcd_row(blockIdx.x, gridDim.x);
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    int j;
    float bs;
    // two selector rows in flight per lane: the attention waves' registers
    // allow five waves per SIMD, so two rows' workgroups share a compute unit
    wave_best_entry<DS, T, Sel, KM, 2>(qs, SS, D, row, K, renorm, lane, &j, &bs);
    if (lane < K) {
      sj[lane] = j;
      sb[lane] = bs;
      if (idx) idx[row * K + lane] = j;
      if (bias) bias[row * K + lane] = bs;
    }
  }
  // attend_row's first barrier publishes the selection
  attend_row<HD, T, WHOLE>(q, S, LdsSlots{sj, sb}, o, lse, D, K, row, blockDim.x >> 6, L, true);
}

// ---------------------------------------------------------------------------
// Block-stationary prefill.
// ---------------------------------------------------------------------------
constexpr int kChunk = 128;  // pairs per chunk of the partial kernel (32 per wave)

__global__ void sp_zero_kernel(int* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// Where the (row, block) pairs of a sparse forward come from.  FixedSel: idx
// and bias [rows, K], pair p = row * K + slot.  CsrSel: a row's pairs are
// p = row_ptr[row] .. row_ptr[row + 1] - 1 of col / bias [nnz]; rowof[p] is
// the row whose segment holds p (-1 if none), built from row_ptr, so even an
// inconsistent row_ptr never sends a pair outside [0, nnz) or to two rows.
struct FixedSel {
  const int* idx;
  const float* bias;
  int K;
  __device__ size_t lo(const Dims& D, int bh) const { return (size_t)bh * D.tq * K; }
  __device__ size_t hi(const Dims& D, int bh) const { return (size_t)(bh + 1) * D.tq * K; }
  __device__ int j_of(size_t p) const { return idx[p]; }
  __device__ long long row_of(size_t p) const { return (long long)(p / K); }
  __device__ float bias_of(size_t p) const { return bias[p]; }
  __device__ size_t seg_lo(size_t row) const { return row * K; }
  __device__ size_t seg_hi(size_t row) const { return (row + 1) * K; }
};

struct CsrSel {
  const long long* row_ptr;
  const int* col;
  const float* bias;
  const int* rowof;
  long long nnz;
  __device__ size_t cl(long long v) const { return (size_t)min(max(v, 0LL), nnz); }
  __device__ size_t lo(const Dims& D, int bh) const { return cl(row_ptr[(size_t)bh * D.tq]); }
  __device__ size_t hi(const Dims& D, int bh) const {
    return max(lo(D, bh), cl(row_ptr[(size_t)(bh + 1) * D.tq]));
  }
  __device__ int j_of(size_t p) const { return col[p]; }
  __device__ long long row_of(size_t p) const { return rowof[p]; }
  __device__ float bias_of(size_t p) const { return bias[p]; }
  __device__ size_t seg_lo(size_t row) const { return cl(row_ptr[row]); }
  __device__ size_t seg_hi(size_t row) const { return max(seg_lo(row), cl(row_ptr[row + 1])); }
};

// rowof for CsrSel: -1 everywhere, then each row stamps its segment.
__global__ __launch_bounds__(256) void sp_fill_value_kernel(int* __restrict__ p, size_t n,
                                                            int value) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = value;
}

__global__ __launch_bounds__(256) void sp_rowof_kernel(CsrSel S, int* __restrict__ rowof,
                                                       size_t nrows) {
  const size_t r = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= nrows) return;
  const size_t a = S.seg_lo(r), e = S.seg_hi(r);
  for (size_t p = a; p < e; ++p) rowof[p] = (int)r;
}

// A pair is listed when its row lies in the (batch, query head) being
// scanned and its block is historical for that row.
template <typename Src>
__device__ __forceinline__ int listed_block(const Src& S, const Dims& D, int bh, size_t p) {
  const long long row = S.row_of(p);
  if (row < 0 || row / D.tq != bh) return -1;
  const int j = S.j_of(p);
  const int c = (D.qoff + (int)(row % D.tq)) / D.blk;
  return (j >= 0 && j < c) ? j : -1;
}

// Inversion of the (row, slot) pairs into per-(batch, kv head, block) lists.
// The workgroups of one (batch, query head) share its pairs (grid-strided),
// so every pair a workgroup sees falls in the nb buckets of one (batch, kv
// head): it histograms them in LDS and touches each global counter once.
constexpr int kInvWGs = 64;  // workgroups per (batch, query head)

template <typename Src>
__global__ __launch_bounds__(256) void sp_count_kernel(Src S, int* __restrict__ count, Dims D) {
  extern __shared__ int hist[];  // nb counters
  const int bh = blockIdx.y, b = bh / D.hq, h = bh % D.hq;
  const size_t p1 = S.hi(D, bh);
  for (int x = threadIdx.x; x < D.nb; x += 256) hist[x] = 0;
  __syncthreads();
  for (size_t p = S.lo(D, bh) + (size_t)blockIdx.x * 256 + threadIdx.x; p < p1;
       p += (size_t)gridDim.x * 256) {
    const int j = listed_block(S, D, bh, p);
    if (j >= 0) atomicAdd(&hist[j], 1);
  }
  __syncthreads();
  int* cb = count + (size_t)(b * D.hkv + h / D.hpg) * D.nb;
  for (int x = threadIdx.x; x < D.nb; x += 256)
    if (hist[x]) atomicAdd(&cb[x], hist[x]);
}

// Exclusive scans of count (-> start) and of ceil(count / kChunk) (-> cstart,
// with cstart[n] = number of chunks), one workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void sp_scan_kernel(const int* __restrict__ count,
                                                       int* __restrict__ start,
                                                       int* __restrict__ cstart, int n) {
  __shared__ int s1[1024], s2[1024];
  const int tid = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int a = 0, c = 0;
  for (int i = lo; i < hi; ++i) {
    a += count[i];
    c += (count[i] + kChunk - 1) / kChunk;
  }
  s1[tid] = a;
  s2[tid] = c;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int x1 = tid >= off ? s1[tid - off] : 0;
    const int x2 = tid >= off ? s2[tid - off] : 0;
    __syncthreads();
    s1[tid] += x1;
    s2[tid] += x2;
    __syncthreads();
  }
  a = s1[tid] - a;  // exclusive prefix of this thread's range
  c = s2[tid] - c;
  for (int i = lo; i < hi; ++i) {
    start[i] = a;
    cstart[i] = c;
    a += count[i];
    c += (count[i] + kChunk - 1) / kChunk;
  }
  if (tid == 1023) cstart[n] = s2[1023];
}

// Same decomposition as sp_count_kernel: local histogram, one global
// reservation per (workgroup, block), then each pair takes a local rank.
// list[x] = pair, inv[pair] = x.
template <typename Src>
__global__ __launch_bounds__(256) void sp_fill_kernel(Src S, const int* __restrict__ start,
                                                      int* __restrict__ cursor,
                                                      int* __restrict__ list,
                                                      int* __restrict__ inv, Dims D) {
  extern __shared__ int sh[];  // hist[nb] then base[nb]
  int* hist = sh;
  int* base = sh + D.nb;
  const int bh = blockIdx.y, b = bh / D.hq, h = bh % D.hq;
  const size_t p0 = S.lo(D, bh) + (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t p1 = S.hi(D, bh), step = (size_t)gridDim.x * 256;
  for (int x = threadIdx.x; x < D.nb; x += 256) hist[x] = 0;
  __syncthreads();
  for (size_t p = p0; p < p1; p += step) {
    const int j = listed_block(S, D, bh, p);
    if (j >= 0) atomicAdd(&hist[j], 1);
  }
  __syncthreads();
  const size_t bucket0 = (size_t)(b * D.hkv + h / D.hpg) * D.nb;
  for (int x = threadIdx.x; x < D.nb; x += 256) {
    const int n = hist[x];
    base[x] = n ? start[bucket0 + x] + atomicAdd(&cursor[bucket0 + x], n) : 0;
    hist[x] = 0;
  }
  __syncthreads();
  for (size_t p = p0; p < p1; p += step) {
    const int j = listed_block(S, D, bh, p);
    if (j >= 0) {
      const int x = base[j] + atomicAdd(&hist[j], 1);
      list[x] = (int)p;
      inv[p] = x;
    }
  }
}

// Historical chunk -> bucket map (chunks are numbered bucket by bucket).
__global__ __launch_bounds__(256) void sp_chunkmap_kernel(const int* __restrict__ cstart,
                                                          int* __restrict__ cbk, int nbk) {
  const int bk = blockIdx.x * 256 + threadIdx.x;
  if (bk >= nbk) return;
  for (int x = cstart[bk]; x < cstart[bk + 1]; ++x) cbk[x] = bk;
}

// Partials of one (row, block) pair per lane-query.  The chunk sequence is
// [current-block chunks | historical chunks]: a current-block chunk holds 128
// (head, token) rows of one (batch, kv head, query block) and attends that
// block causally with bias 0; a historical chunk holds up to 128 listed pairs
// of one (batch, kv head, block) with their bias.  Partials are stored in
// chunk order (position = chunk * 128 + pair in chunk), so every chunk writes
// one contiguous 32 KB run; the merge finds a listed pair's partial through
// the inverse of the list.  A workgroup walks kChunksPerWG consecutive chunks and
// restages K and V only when the block changes (consecutive chunks mostly
// share it).  Wave w takes pairs 32w .. 32w+31 of a chunk; K row-major and V
// transposed in LDS; S^T = K Q^T and O^T = V^T P^T on 32x32x16 MFMA, so each
// lane owns one query.
constexpr int kChunksPerWG = 8;

template <int HD, typename Src>
__global__ __launch_bounds__(256, 2) void sp_partial_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    Src S, const int* __restrict__ list, const int* __restrict__ start,
    const int* __restrict__ count, const int* __restrict__ cstart, const int* __restrict__ cbk,
    float* __restrict__ plse, bf16* __restrict__ po, Dims D, int nbk, int nqb, int dcpb) {
  constexpr int KP = HD + 8, VP = kBlock + 4, KS = HD / 16, DM = HD / 32;
  constexpr int OP = 72;  // pitch (bf16) of the per-wave output staging rows: 16-byte aligned
  __shared__ __align__(16) bf16 Ks[kBlock * KP];
  __shared__ __align__(16) bf16 Vt[HD * VP];
  __shared__ __align__(16) bf16 Os[4 * 32 * OP];  // per wave: 32 queries x 64 columns
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  bf16* ow = Os + wave * 32 * OP;
  const int ndiag = D.batch * D.hkv * nqb * dcpb;
  const int total = ndiag + cstart[nbk];
  const int ch0 = blockIdx.x * kChunksPerWG;
  if (ch0 >= total) return;
  const int ch1 = min(total, ch0 + kChunksPerWG);
  const float c1 = D.sm_scale * kLog2e;
  const int B = D.blk;              // keys per gate unit (a 64-key tile holds 64 / B)
  const int qb0 = D.qoff / B;       // first unit holding a query row
  const int ntl = D.tk / kBlock;    // 64-key tiles per (batch, kv head)
  const int pi = wave * 32 + l32;   // this lane's pair within a chunk
  int cur = -1;                     // tile staged in LDS
  for (int ch = ch0; ch < ch1; ++ch) {
    int kv, tmax, pos;  // pos: where the partial goes (chunk order)
    size_t row;
    float bv;
    bool valid;
    if (ch < ndiag) {
      const int db = ch / dcpb, dc = ch - db * dcpb;
      const int bg = db / nqb, j = qb0 + db % nqb;
      kv = bg * D.nb + j;
      const int p = dc * kChunk + pi;
      const int hl = p / B, tok = j * B + p % B;
      valid = hl < D.hpg && tok >= D.qoff && tok < D.tk;
      const int b = bg / D.hkv, g = bg - b * D.hkv;
      const int h = g * D.hpg + (valid ? hl : 0);
      row = ((size_t)b * D.hq + h) * D.tq + (valid ? tok - D.qoff : 0);
      pos = ch * kChunk + pi;
      bv = 0.f;
      tmax = tok;
    } else {
      const int hc = ch - ndiag;
      const int bk = cbk[hc];
      kv = bk;
      const int ci = hc - cstart[bk];
      const int n = min(kChunk, count[bk] - ci * kChunk);
      valid = pi < n;
      const int pair = list[start[bk] + ci * kChunk + (valid ? pi : 0)];
      row = (size_t)S.row_of(pair);  // a listed pair has a valid row
      pos = ndiag * kChunk + start[bk] + ci * kChunk + pi;
      bv = S.bias_of(pair);
      tmax = 0x7fffffff;  // a historical block lies wholly before the query
    }
    bf16x8 qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *(const bf16x8*)(q + row * HD + 16 * s + 8 * hh);
    kv = __builtin_amdgcn_readfirstlane(kv);
    const int ulo = (kv % D.nb) * B;  // the unit's keys ulo .. ulo + B - 1
    const int tile = (kv / D.nb) * ntl + ulo / kBlock;
    if (tile != cur) {
      __syncthreads();  // every wave is done with the previous tile
      const int jt = tile % ntl, bg = tile / ntl;
      const bf16* kb = k + ((size_t)bg * D.tk + (size_t)jt * kBlock) * HD;
      const bf16* vb = v + ((size_t)bg * D.tk + (size_t)jt * kBlock) * HD;
      for (int x = tid; x < kBlock * HD / 8; x += 256) {
        const int r = x / (HD / 8), cc = x % (HD / 8);
        *(bf16x8*)&Ks[r * KP + cc * 8] = *(const bf16x8*)(kb + (size_t)r * HD + cc * 8);
      }
      for (int x = tid; x < 16 * (HD / 8); x += 256) {
        const int kg = x % 16, dcol = x / 16;
        bf16x8 rv[4];
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2)
          rv[i2] = *(const bf16x8*)(vb + (size_t)(kg * 4 + i2) * HD + dcol * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bf16x4 wv = {rv[0][e], rv[1][e], rv[2][e], rv[3][e]};
          *(bf16x4*)&Vt[(dcol * 8 + e) * VP + kg * 4] = wv;
        }
      }
      __syncthreads();
      cur = tile;
    }
    if (!__any(valid)) continue;  // wave-uniform: no pair of this chunk for this wave
    const float bias2 = bv * kLog2e;
    const int u0 = (ulo / kBlock) * kBlock;  // first key of the staged tile
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 a = *(const bf16x8*)&Ks[(32 * mt + l32) * KP + 16 * s + 8 * hh];
        sacc[mt] = mfma32(a, qf[s], sacc[mt]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int u = u0 + 32 * mt + (r / 4) * 8 + 4 * hh + (r % 4);
        if (u > tmax || u < ulo || u >= ulo + B) sacc[mt][r] = -INFINITY;  // causal, unit
        mx = fmaxf(mx, sacc[mt][r]);
      }
    mx = halves_max(mx);
    const float m2 = fmaf(mx, c1, bias2);  // row max in log2 units (-inf only if bias is -inf)
    const float off = bias2 - (m2 == -INFINITY ? 0.f : m2);
    float l = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = exp2_raw(fmaf(sacc[mt][r], c1, off));
        sacc[mt][r] = pv;
        l += pv;
      }
    l = halves_sum(l);
    f32x16 oacc[DM];
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) oacc[dm] = f32x16{};
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (bf16)sacc[mt][8 * pp + e];
#pragma unroll
        for (int dm = 0; dm < DM; ++dm) {
          const bf16* vp = &Vt[(32 * dm + l32) * VP + 32 * mt + 16 * pp + 4 * hh];
          const bf16x4 lo4 = *(const bf16x4*)vp;
          const bf16x4 hi4 = *(const bf16x4*)(vp + 8);
          oacc[dm] = mfma32(__builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7), pb, oacc[dm]);
        }
      }
    }
    const bool live = l > 0.f && m2 != -INFINITY;
    const float inv = live ? 1.f / l : 0.f;
    const int ps = valid ? pos : -1;
    if (valid && hh == 0) plse[ps] = live ? (m2 + log2f(l)) * kLn2 : -INFINITY;
    // Normalised partial rows go out through LDS, 64 columns at a time, so that
    // eight lanes write one contiguous 128-byte run of a row.
    const int rq = lane >> 3, c8 = (lane & 7) * 8;
#pragma unroll
    for (int hf = 0; hf < DM / 2; ++hf) {
#pragma unroll
      for (int d2 = 0; d2 < 2; ++d2) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          bf16x4 wv;
#pragma unroll
          for (int e = 0; e < 4; ++e) wv[e] = (bf16)(oacc[2 * hf + d2][4 * rr + e] * inv);
          *(bf16x4*)&ow[l32 * OP + 32 * d2 + 8 * rr + 4 * hh] = wv;
        }
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int r = rq + 8 * it;
        const int pr = __shfl(ps, r);
        const bf16x8 ov = *(const bf16x8*)&ow[r * OP + c8];
        if (pr >= 0) *(bf16x8*)(po + (size_t)pr * HD + 64 * hf + c8) = ov;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// Merge of a row's partials: its current block (always present) and every
// slot s < K whose block idx[row, s] lies before c(t).  L = log sum exp(lse_s),
// O = sum_s exp(lse_s - L) O_s.  One wavefront per row; a partial row is read
// by HD/8 lanes, 16 bytes each, so one load instruction covers 64/(HD/8) slots.
template <int HD, typename Src>
__global__ __launch_bounds__(256) void sp_merge_kernel(Src S, const int* __restrict__ inv,
                                                       const float* __restrict__ plse,
                                                       const bf16* __restrict__ po,
                                                       bf16* __restrict__ o,
                                                       float* __restrict__ lse, Dims D, int nqb,
                                                       int dcpb) {
  constexpr int LPP = HD / 8, SPW = 64 / LPP;
  const int lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const size_t nrows = (size_t)D.batch * D.hq * D.tq;
  if (row >= nrows) return;
  const int i = (int)(row % D.tq), t = D.qoff + i, c = t / D.blk;
  const int h = (int)((row / D.tq) % D.hq), b = (int)(row / ((size_t)D.tq * D.hq));
  const int g = h / D.hpg, hl = h - g * D.hpg;
  // chunk-order position of the current block's partial and of the listed ones
  const int dpos = ((b * D.hkv + g) * nqb + (c - D.qoff / D.blk)) * dcpb * kChunk +
                   hl * D.blk + t % D.blk;
  const int hbase = D.batch * D.hkv * nqb * dcpb * kChunk;
  const size_t a0 = S.seg_lo(row);
  const int len = (int)(S.seg_hi(row) - a0);
  const int grp = lane / LPP, col = (lane % LPP) * 8;
  const bf16* pr = po + col;
  // online merge in log2 units: m running max, sm = sum of 2^(lse - m),
  // acc = sum of 2^(lse - m) O (group g of lanes holds the slots it loaded)
  float m = plse[dpos] * kLog2e, sm = 1.f;
  float acc[8];
  {
    const bf16x8 cv = *(const bf16x8*)(pr + (size_t)dpos * HD);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = grp == 0 ? to_f32(cv[e]) : 0.f;
  }
  // the listed slots, 64 at a time: each lane reads one slot's block, position and lse
  for (int w0 = 0; w0 < len; w0 += 64) {
    const int x = w0 + lane;
    const int j = x < len ? S.j_of(a0 + x) : -1;
    const bool ok = j >= 0 && j < c && S.row_of(a0 + x) == (long long)row;
    const int px = ok ? hbase + inv[a0 + x] : dpos;
    const float lx = ok ? plse[px] * kLog2e : -INFINITY;
    const unsigned long long bal = __ballot(ok);
    if (bal == 0) continue;
    const float m_new = fmaxf(m, group_max<64>(lx));
    const float alpha = exp2_raw(m - m_new);
    m = m_new;
    const float pw = ok ? exp2_raw(lx - m) : 0.f;
    sm = sm * alpha + group_sum<64>(pw);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
    const int nval = 64 - __builtin_clzll(bal);  // slots past the last valid one are skipped
#pragma unroll 4
    for (int q0 = 0; q0 < nval; q0 += SPW) {
      const int sl = q0 + grp;
      const float w = __shfl(pw, sl);
      const int pp = __shfl(px, sl);
      const bf16x8 pv = *(const bf16x8*)(pr + (size_t)pp * HD);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, w != 0.f ? to_f32(pv[e]) : 0.f, acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = stride_sum<LPP>(acc[e]);
  if (grp == 0) {
    const float inv_s = 1.f / sm;
    bf16x8 ov;
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[e] = (bf16)(acc[e] * inv_s);
    *(bf16x8*)(o + row * HD + col) = ov;
  }
  if (lane == 0 && lse) lse[row] = (m + log2f(sm)) * kLn2;
}

// d = 128: the same merge with a 16-lane group per row, four rows per wave.
// A partial row is exactly 16 lanes x 16 bytes, so a group reads one of its
// row's partials per load while the other groups read theirs; the chain of
// dependent loads (slot list, inverse position, lse, partial rows) is paid
// once per four rows instead of once per row.  Group-local max and sum by
// DPP inside the 16-lane row; slots 16 at a time.
__device__ __forceinline__ float max16_dpp(float x) {
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false)));
  return x;
}
__device__ __forceinline__ float sum16_dpp(float x) {
  x = sum8_dpp(x);  // pairs, quads, halves of 8
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  return x;
}

template <typename Src>
__global__ __launch_bounds__(256) void sp_merge16_kernel(Src S, const int* __restrict__ inv,
                                                         const float* __restrict__ plse,
                                                         const bf16* __restrict__ po,
                                                         bf16* __restrict__ o,
                                                         float* __restrict__ lse, Dims D, int nqb,
                                                         int dcpb) {
  constexpr int HD = 128;
  const int lane = threadIdx.x & 63, grp = lane >> 4, sl = lane & 15;
  const size_t nrows = (size_t)D.batch * D.hq * D.tq;
  const size_t row = (size_t)blockIdx.x * 16 + (threadIdx.x >> 6) * 4 + grp;
  if (__builtin_amdgcn_readfirstlane((size_t)blockIdx.x * 16 + (threadIdx.x >> 6) * 4) >= nrows)
    return;  // whole wave past the end
  const bool live = row < nrows;  // uniform over the group
  const size_t rw = live ? row : nrows - 1;
  const int i = (int)(rw % D.tq), t = D.qoff + i, c = t / D.blk;
  const int h = (int)((rw / D.tq) % D.hq), b = (int)(rw / ((size_t)D.tq * D.hq));
  const int g = h / D.hpg, hl = h - g * D.hpg;
  const int dpos = ((b * D.hkv + g) * nqb + (c - D.qoff / D.blk)) * dcpb * kChunk +
                   hl * D.blk + t % D.blk;
  const int hbase = D.batch * D.hkv * nqb * dcpb * kChunk;
  const size_t a0 = S.seg_lo(rw);
  const int len = live ? (int)(S.seg_hi(rw) - a0) : 0;
  const bf16* pr = po + sl * 8;
  // online merge in log2 units, as in sp_merge_kernel; lane sl of a group
  // holds columns 8 sl .. 8 sl + 7 of its row
  float m = plse[dpos] * kLog2e, sm = 1.f;
  float acc[8];
  {
    const bf16x8 cv = *(const bf16x8*)(pr + (size_t)dpos * HD);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = to_f32(cv[e]);
  }
  for (int w0 = 0; w0 < len; w0 += 16) {
    const int x = w0 + sl;
    const int j = x < len ? S.j_of(a0 + x) : -1;
    const bool ok = j >= 0 && j < c && S.row_of(a0 + x) == (long long)rw;
    const int px = ok ? hbase + inv[a0 + x] : dpos;
    const float lx = ok ? plse[px] * kLog2e : -INFINITY;
    const unsigned gb = (unsigned)(__ballot(ok) >> (16 * grp)) & 0xFFFFu;
    if (gb == 0) continue;
    const float m_new = fmaxf(m, max16_dpp(lx));
    const float alpha = exp2_raw(m - m_new);
    m = m_new;
    const float pw = ok ? exp2_raw(lx - m) : 0.f;
    sm = sm * alpha + sum16_dpp(pw);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
    const int nval = 32 - __builtin_clz(gb);  // slots past the group's last valid one skipped
#pragma unroll 4
    for (int q = 0; q < nval; ++q) {
      const float w = __shfl(pw, q, 16);
      const int pp = __shfl(px, q, 16);
      const bf16x8 pv = *(const bf16x8*)(pr + (size_t)pp * HD);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, w != 0.f ? to_f32(pv[e]) : 0.f, acc[e]);
    }
  }
  if (!live) return;
  const float inv_s = 1.f / sm;
  bf16x8 ov;
#pragma unroll
  for (int e = 0; e < 8; ++e) ov[e] = (bf16)(acc[e] * inv_s);
  *(bf16x8*)(o + row * HD + sl * 8) = ov;
  if (sl == 0 && lse) lse[row] = (m + log2f(sm)) * kLn2;
}

// ---------------------------------------------------------------------------
// Dense selections (prefill whose rows keep a large share of their history,
// e.g. a quarter of it): the query-stationary dense kernel runs with the
// selection as a bias matrix, -inf where a row does not attend a block.  The
// matrix is tiled by 8-row chunks, bt [b * hq][tq / 8][nb][8]: a chunk's
// biases of one block are one 32-byte run (a wave's 32 rows read four), and a
// chunk's whole matrix is one contiguous run.  Built per (batch x head,
// 8-row chunk, 512-block range) in LDS: every slot of the chunk's rows lands
// in its LDS cell, then the cells of the blocks some row of the chunk can see
// (j < c of the chunk's last row) go out contiguously.  Entries that are not
// historical blocks of their row are skipped, as in the other paths.
constexpr int kBtRows = 8, kBtBlocks = 512;

__global__ __launch_bounds__(256) void sp_bias_matrix_kernel(const int* __restrict__ idx,
                                                             const float* __restrict__ bias,
                                                             int K, float* __restrict__ bt,
                                                             Dims D) {
  __shared__ __align__(16) float cell[kBtBlocks][kBtRows];
  const int i0 = blockIdx.x * kBtRows, j0 = blockIdx.y * kBtBlocks;
  const size_t bh = blockIdx.z;
  const int nrow = min(kBtRows, D.tq - i0);
  // blocks visible to some row of the chunk: j < c(last row)
  const int jend = min(min(j0 + kBtBlocks, D.nb), (D.qoff + i0 + nrow - 1) / kBlock);
  if (jend <= j0) return;  // uniform: no row of the chunk sees these blocks
  const f32x4 ninf = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  for (int x = threadIdx.x; x < kBtBlocks * kBtRows / 4; x += 256)
    *(f32x4*)&cell[x / (kBtRows / 4)][4 * (x % (kBtRows / 4))] = ninf;
  __syncthreads();
  const size_t r0 = bh * D.tq + i0;
  for (int x = threadIdx.x; x < nrow * K; x += 256) {
    const int r = x / K;  // slot fastest: the chunk's idx / bias are one contiguous run
    const int j = idx[r0 * K + x];
    const int c = (D.qoff + i0 + r) / kBlock;
    if (j >= j0 && j < jend && j < c) cell[j - j0][r] = bias[r0 * K + x];
  }
  __syncthreads();
  const int nch = (D.tq + kBtRows - 1) / kBtRows;
  float* dst = bt + ((bh * nch + blockIdx.x) * (size_t)D.nb + j0) * kBtRows;
  for (int x = threadIdx.x; x < (jend - j0) * (kBtRows / 4); x += 256)
    *(f32x4*)&dst[4 * x] = *(const f32x4*)&cell[x / (kBtRows / 4)][4 * (x % (kBtRows / 4))];
}

// The dense-kernel path pays every block of the causal triangle; the
// block-stationary path pays per selected pair (gather, partial, merge), about
// six times the cost of a dense pair on MI355X (top-16 at 32k: 3.1 ms for
// 1.09e9 pairs; dense: 9.0 ms for 1.72e10).  Selections keeping at least
// 3/16 of the average row's history take the dense kernel.
static bool use_given_bias_path(const Dims& D, int K) {
  if (D.blk != kBlock || D.tq < 256 || (D.d != 128 && D.d != 64)) return false;
  const double avg_keys = (double)D.qoff + 0.5 * (double)(D.tq + 1);
  return 16.0 * (double)K * kBlock >= 3.0 * avg_keys;
}
static size_t given_bias_workspace(const Dims& D) {
  const size_t nch = (D.tq + kBtRows - 1) / kBtRows;
  return align256s((size_t)D.batch * D.hq * nch * kBtRows * D.nb * sizeof(float));
}

static int diag_chunks_per_block(const Dims& D) { return (D.hpg * D.blk + kChunk - 1) / kChunk; }
static int query_blocks(const Dims& D) { return D.nb - D.qoff / D.blk; }
// Partial slots of the block path: current-block chunks, then one per pair.
static size_t block_path_slots(const Dims& D, size_t npairs) {
  return (size_t)D.batch * D.hkv * query_blocks(D) * diag_chunks_per_block(D) * kChunk + npairs;
}

// The block path stages the 64-key tile that holds a gate unit (keys outside
// the unit masked), histograms units in LDS: nb <= 8192 (64 KB for the
// fill); partial positions are int.
static bool block_path_fits(const Dims& D, size_t npairs) {
  return D.nb <= 8192 && block_path_slots(D, npairs) < ((size_t)1 << 31);
}
// units below 16 tokens would waste most of each 64-key tile: the row path
static bool use_block_path(const Dims& D, int K) {
  return D.tq >= 128 && D.blk >= 16 && block_path_fits(D, (size_t)D.batch * D.hq * D.tq * K);
}

// Block path workspace: [count | cursor | start | cstart | cbk | list | inv |
// plse (slots) | po (slots x d)], then rowof (npairs) for a CSR selection.
static size_t block_path_workspace(const Dims& D, size_t npairs, bool csr) {
  const size_t nbk = (size_t)D.batch * D.hkv * D.nb;
  const size_t slots = block_path_slots(D, npairs);
  const size_t max_chunks = npairs / kChunk + nbk;
  return 3 * align256s(nbk * 4) + align256s((nbk + 1) * 4) + align256s(max_chunks * 4) +
         2 * align256s(npairs * 4) + align256s(slots * 4) + align256s(slots * D.d * 2) +
         (csr ? align256s(npairs * 4) : 0);
}

// Workspace: pair path  [plse (rows x (K+1)) | po (rows x (K+1) x d)]; block path above.
size_t sparse_workspace(const Dims& D, int K) {
  const size_t rows = (size_t)D.batch * D.hq * D.tq;
  if (use_given_bias_path(D, K)) return given_bias_workspace(D);
  if (use_block_path(D, K)) return block_path_workspace(D, rows * K, false);
  return 256;  // the row kernel needs none
}

bool sparse_csr_supported(const Dims& D, long long nnz) {
  return nnz >= 0 && block_path_fits(D, (size_t)nnz);
}
size_t sparse_csr_workspace(const Dims& D, long long nnz) {
  return block_path_workspace(D, (size_t)nnz, true);
}

template <int HD, typename Src>
static hipError_t launch_block_path(const void* q, const void* k, const void* v, const Src& S,
                                    size_t npairs, size_t per_bh, void* o, float* lse, char* ws,
                                    const Dims& D, const StageEvents& E, hipStream_t st) {
  const size_t rows = (size_t)D.batch * D.hq * D.tq;
  const size_t slots = block_path_slots(D, npairs);
  const int nbk = D.batch * D.hkv * D.nb;
  const size_t max_chunks = npairs / kChunk + (size_t)nbk;
  char* p = ws;
  int* count = (int*)p;  p += align256s((size_t)nbk * 4);
  int* cursor = (int*)p; p += align256s((size_t)nbk * 4);
  int* start = (int*)p;  p += align256s((size_t)nbk * 4);
  int* cstart = (int*)p; p += align256s((size_t)(nbk + 1) * 4);
  int* cbk = (int*)p;    p += align256s(max_chunks * 4);
  int* list = (int*)p;   p += align256s(npairs * 4);
  int* inv = (int*)p;    p += align256s(npairs * 4);
  float* plse = (float*)p; p += align256s(slots * 4);
  bf16* po = (bf16*)p;
  const unsigned zg = (unsigned)std::min<size_t>((2 * (size_t)nbk + 255) / 256, 4096);
  hipLaunchKernelGGL(sp_zero_kernel, dim3(zg), dim3(256), 0, st, count, (size_t)nbk);
  hipLaunchKernelGGL(sp_zero_kernel, dim3(zg), dim3(256), 0, st, cursor, (size_t)nbk);
  // workgroups per (batch, query head): one per 4096 pairs, at most kInvWGs
  const unsigned gx = (unsigned)std::max<size_t>(1, std::min<size_t>(kInvWGs,
                                                                     (per_bh + 4095) / 4096));
  const dim3 ig(gx, D.batch * D.hq);
  hipLaunchKernelGGL((sp_count_kernel<Src>), ig, dim3(256), (size_t)D.nb * 4, st, S, count, D);
  hipLaunchKernelGGL(sp_scan_kernel, dim3(1), dim3(1024), 0, st, (const int*)count, start, cstart,
                     nbk);
  hipLaunchKernelGGL((sp_fill_kernel<Src>), ig, dim3(256), (size_t)D.nb * 8, st, S,
                     (const int*)start, cursor, list, inv, D);
  hipLaunchKernelGGL(sp_chunkmap_kernel, dim3((unsigned)((nbk + 255) / 256)), dim3(256), 0, st,
                     (const int*)cstart, cbk, nbk);
  // upper bound on the number of chunks; workgroups past the real count exit
  const int nqb = query_blocks(D), dcpb = diag_chunks_per_block(D);
  const size_t ndiag = (size_t)D.batch * D.hkv * nqb * dcpb;
  const size_t wgs = (ndiag + max_chunks + kChunksPerWG - 1) / kChunksPerWG;
  hipLaunchKernelGGL((sp_partial_kernel<HD, Src>), dim3((unsigned)wgs), dim3(256), 0, st,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, S, (const int*)list,
                     (const int*)start, (const int*)count, (const int*)cstart, (const int*)cbk,
                     plse, po, D, nbk, nqb, dcpb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  E.record(0, st);
  // grouped merge while rows list 16 slots or fewer on average; a wave per
  // row (64 slots per pass) for larger selections
  if (HD == 128 && npairs <= 16 * rows)
    hipLaunchKernelGGL((sp_merge16_kernel<Src>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0,
                       st, S, (const int*)inv, (const float*)plse, (const bf16*)po, (bf16*)o, lse,
                       D, nqb, dcpb);
  else
    hipLaunchKernelGGL((sp_merge_kernel<HD, Src>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                       st, S, (const int*)inv, (const float*)plse, (const bf16*)po, (bf16*)o, lse,
                       D, nqb, dcpb);
  return hipGetLastError();
}

template <int HD>
static hipError_t launch_fixed_block_path(const void* q, const void* k, const void* v,
                                          const int* idx, const float* bias, void* o, float* lse,
                                          char* ws, int K, const Dims& D, const StageEvents& E,
                                          hipStream_t st) {
  const size_t rows = (size_t)D.batch * D.hq * D.tq;
  return launch_block_path<HD, FixedSel>(q, k, v, FixedSel{idx, bias, K}, rows * K,
                                         (size_t)D.tq * K, o, lse, ws, D, E, st);
}

template <int HD>
static hipError_t launch_csr_t(const void* q, const void* k, const void* v,
                               const long long* row_ptr, const int* col, const float* bias,
                               long long nnz, void* o, float* lse, char* ws, const Dims& D,
                               const StageEvents& E, hipStream_t st) {
  const size_t rows = (size_t)D.batch * D.hq * D.tq;
  int* rowof = (int*)(ws + block_path_workspace(D, (size_t)nnz, false));
  const CsrSel S{row_ptr, col, bias, rowof, nnz};
  if (nnz > 0) {
    const unsigned g = (unsigned)std::min<size_t>(((size_t)nnz + 255) / 256, 8192);
    hipLaunchKernelGGL(sp_fill_value_kernel, dim3(g), dim3(256), 0, st, rowof, (size_t)nnz, -1);
    hipLaunchKernelGGL(sp_rowof_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, S,
                       rowof, rows);
  }
  const size_t per_bh = ((size_t)nnz + (size_t)D.batch * D.hq - 1) / ((size_t)D.batch * D.hq);
  return launch_block_path<HD, CsrSel>(q, k, v, S, (size_t)nnz, per_bh, o, lse, ws, D, E, st);
}

hipError_t launch_sparse_csr(const void* q, const void* k, const void* v, const long long* row_ptr,
                             const int* col, const float* bias, long long nnz, void* o,
                             float* lse, char* ws, const Dims& D, const StageEvents& E,
                             hipStream_t st) {
  if (D.d == 128) return launch_csr_t<128>(q, k, v, row_ptr, col, bias, nnz, o, lse, ws, D, E, st);
  if (D.d == 64) return launch_csr_t<64>(q, k, v, row_ptr, col, bias, nnz, o, lse, ws, D, E, st);
  return hipErrorInvalidValue;
}

// Waves per row of the row kernels: one per slot, at most 8 for K <= 8 and
// 16 beyond.  The fused selection + decode kernel's registers (about 100 per
// lane) allow four waves per SIMD, so two rows of eight waves share a compute
// unit where two rows of nine would not (the wave that takes a second slot
// costs less than rows waiting for a free unit); the separate decode uses the
// same count, so that both merge the same partial states in the same order
// and give identical results.
static int row_waves(int K) {
  return K <= 8 ? std::min(K + 1, 8) : std::min(K + 1, kRowWaves);
}

template <int HD, typename T>
static hipError_t launch_sparse_t(const void* q, const void* k, const void* v, const int* idx,
                                  const float* bias, void* o, float* lse, int K, const Dims& D,
                                  const StageEvents& E, hipStream_t st) {
  const size_t rows = (size_t)D.batch * D.hq * D.tq;
  const DenseKV<HD, T> S{(const T*)k, (const T*)v};
  const dim3 grid((unsigned)rows), blk(64 * row_waves(K));
  bool whole = false;
  if constexpr (whole_blocks_fit<HD, T>()) whole = D.blk == kBlock;
  if (whole)
    hipLaunchKernelGGL((sparse_row_kernel<HD, T, DenseKV<HD, T>, whole_blocks_fit<HD, T>()>),
                       grid, blk, 0, st, (const T*)q, S, idx, bias, (T*)o, lse, D, K);
  else
    hipLaunchKernelGGL((sparse_row_kernel<HD, T, DenseKV<HD, T>, false>), grid, blk, 0, st,
                       (const T*)q, S, idx, bias, (T*)o, lse, D, K);
  E.record(0, st);
  return hipGetLastError();
}

hipError_t launch_sparse(const void* q, const void* k, const void* v, const int* idx,
                         const float* bias, void* o, float* lse, char* ws, size_t ws_bytes,
                         int K, const Dims& D, bool bf16_io, const StageEvents& E,
                         hipStream_t st) {
  (void)ws_bytes;
  if (bf16_io && use_given_bias_path(D, K)) {
    float* bt = (float*)ws;
    const dim3 grid((unsigned)((D.tq + kBtRows - 1) / kBtRows),
                    (unsigned)((D.nb + kBtBlocks - 1) / kBtBlocks), (unsigned)(D.batch * D.hq));
    hipLaunchKernelGGL(sp_bias_matrix_kernel, grid, dim3(256), 0, st, idx, bias, K, bt, D);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    E.record(0, st);
    return launch_fwd_given_bias(q, k, v, bt, o, lse, D, st);
  }
  if (bf16_io && use_block_path(D, K)) {
    if (D.d == 128)
      return launch_fixed_block_path<128>(q, k, v, idx, bias, o, lse, ws, K, D, E, st);
    if (D.d == 64) return launch_fixed_block_path<64>(q, k, v, idx, bias, o, lse, ws, K, D, E, st);
  }
  if (D.d == 128)
    return bf16_io ? launch_sparse_t<128, bf16>(q, k, v, idx, bias, o, lse, K, D, E, st)
                   : launch_sparse_t<128, float>(q, k, v, idx, bias, o, lse, K, D, E, st);
  if (D.d == 64)
    return bf16_io ? launch_sparse_t<64, bf16>(q, k, v, idx, bias, o, lse, K, D, E, st)
                   : launch_sparse_t<64, float>(q, k, v, idx, bias, o, lse, K, D, E, st);
  return hipErrorInvalidValue;
}

// Paged decode: one row per (sequence, query head), the pair path over the
// page pools.  Workspace as for the pair path with tq = 1.
template <int HD, typename T>
static hipError_t launch_paged_t(const void* q, const void* k_pool, const void* v_pool,
                                 const int* table, const int* lens, int pages, const int* idx,
                                 const float* bias, void* o, float* lse, int K, const Dims& D,
                                 hipStream_t st) {
  const size_t rows = (size_t)D.batch * D.hq;
  // pages hold whole 64-key blocks
  hipLaunchKernelGGL((sparse_row_kernel<HD, T, PagedKV<HD, T>, whole_blocks_fit<HD, T>()>),
                     dim3((unsigned)rows),
                     dim3(64 * row_waves(K)), 0, st, (const T*)q,
                     PagedKV<HD, T>{(const T*)k_pool, (const T*)v_pool, table, lens, pages}, idx,
                     bias, (T*)o, lse, D, K);
  return hipGetLastError();
}

// The row kernel needs no workspace; the size query still answers.
size_t paged_workspace(const Dims& D, int K) {
  (void)D;
  (void)K;
  return 256;
}

hipError_t launch_paged_decode(const void* q, const void* k_pool, const void* v_pool,
                               const int* table, const int* lens, int pages, const int* idx,
                               const float* bias, void* o, float* lse, char* ws, int K,
                               const Dims& D, bool bf16_io, hipStream_t st) {
  (void)ws;
  if (D.d == 128)
    return bf16_io ? launch_paged_t<128, bf16>(q, k_pool, v_pool, table, lens, pages, idx, bias,
                                               o, lse, K, D, st)
                   : launch_paged_t<128, float>(q, k_pool, v_pool, table, lens, pages, idx,
                                                bias, o, lse, K, D, st);
  if (D.d == 64)
    return bf16_io ? launch_paged_t<64, bf16>(q, k_pool, v_pool, table, lens, pages, idx, bias,
                                              o, lse, K, D, st)
                   : launch_paged_t<64, float>(q, k_pool, v_pool, table, lens, pages, idx, bias,
                                               o, lse, K, D, st);
  return hipErrorInvalidValue;
}

// Fused selection + decode (K <= 16), contiguous and paged caches.
template <int HD, typename T, int DS, typename Sel, typename Src>
static hipError_t launch_topk_row_t(const void* q, Src S, const void* qs, Sel SS, int K,
                                    int renorm, int* idx, float* bias, void* o, float* lse,
                                    const Dims& D, size_t rows, hipStream_t st) {
  const dim3 grid((unsigned)rows), blk(64 * row_waves(K));
  constexpr bool W = whole_blocks_fit<HD, T>();
  const bool whole = W && D.blk == kBlock;
  if (K <= 8 && whole)
    hipLaunchKernelGGL((topk_row_kernel<HD, T, DS, 8, Sel, Src, W>), grid, blk, 0, st,
                       (const T*)q, S, (const T*)qs, SS, K, renorm, idx, bias, (T*)o, lse, D);
  else if (K <= 8)
    hipLaunchKernelGGL((topk_row_kernel<HD, T, DS, 8, Sel, Src, false>), grid, blk, 0, st,
                       (const T*)q, S, (const T*)qs, SS, K, renorm, idx, bias, (T*)o, lse, D);
  else if (whole)
    hipLaunchKernelGGL((topk_row_kernel<HD, T, DS, 16, Sel, Src, W>), grid, blk, 0, st,
                       (const T*)q, S, (const T*)qs, SS, K, renorm, idx, bias, (T*)o, lse, D);
  else
    hipLaunchKernelGGL((topk_row_kernel<HD, T, DS, 16, Sel, Src, false>), grid, blk, 0, st,
                       (const T*)q, S, (const T*)qs, SS, K, renorm, idx, bias, (T*)o, lse, D);
  return hipGetLastError();
}

template <int HD, typename T>
static hipError_t launch_topk_decode_d(const void* q, const void* k, const void* v,
                                       const void* qs, const void* ks, int K, int renorm,
                                       int* idx, float* bias, void* o, float* lse, const Dims& D,
                                       hipStream_t st) {
  const size_t rows = (size_t)D.batch * D.hq * D.tq;
  const DenseKV<HD, T> S{(const T*)k, (const T*)v};
  const DenseSel<T> SS{(const T*)ks};
  switch (D.ds) {
    case 16: return launch_topk_row_t<HD, T, 16>(q, S, qs, SS, K, renorm, idx, bias, o, lse, D, rows, st);
    case 32: return launch_topk_row_t<HD, T, 32>(q, S, qs, SS, K, renorm, idx, bias, o, lse, D, rows, st);
    case 64: return launch_topk_row_t<HD, T, 64>(q, S, qs, SS, K, renorm, idx, bias, o, lse, D, rows, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_topk_decode(const void* q, const void* k, const void* v, const void* qs,
                              const void* ks, int K, int renorm, int* idx, float* bias, void* o,
                              float* lse, const Dims& D, bool bf16_io, hipStream_t st) {
  if (K < 1 || K > 16) return hipErrorInvalidValue;
  if (bf16_io) {
    if (D.d == 128)
      return launch_topk_decode_d<128, bf16>(q, k, v, qs, ks, K, renorm, idx, bias, o, lse, D, st);
    if (D.d == 64)
      return launch_topk_decode_d<64, bf16>(q, k, v, qs, ks, K, renorm, idx, bias, o, lse, D, st);
  } else if (D.d == 64) {
    return launch_topk_decode_d<64, float>(q, k, v, qs, ks, K, renorm, idx, bias, o, lse, D, st);
  }
  return hipErrorInvalidValue;
}

template <int HD, typename T>
static hipError_t launch_paged_topk_decode_d(const void* q, const void* k_pool,
                                             const void* v_pool, const void* qs,
                                             const void* ks_pool, const int* table,
                                             const int* lens, int pages, int K, int renorm,
                                             int* idx, float* bias, void* o, float* lse,
                                             const Dims& D, hipStream_t st) {
  const size_t rows = (size_t)D.batch * D.hq;
  const PagedKV<HD, T> S{(const T*)k_pool, (const T*)v_pool, table, lens, pages};
  const PagedSel<T> SS{(const T*)ks_pool, table, lens, pages};
  switch (D.ds) {
    case 16: return launch_topk_row_t<HD, T, 16>(q, S, qs, SS, K, renorm, idx, bias, o, lse, D, rows, st);
    case 32: return launch_topk_row_t<HD, T, 32>(q, S, qs, SS, K, renorm, idx, bias, o, lse, D, rows, st);
    case 64: return launch_topk_row_t<HD, T, 64>(q, S, qs, SS, K, renorm, idx, bias, o, lse, D, rows, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_paged_topk_decode(const void* q, const void* k_pool, const void* v_pool,
                                    const void* qs, const void* ks_pool, const int* table,
                                    const int* lens, int pages, int K, int renorm, int* idx,
                                    float* bias, void* o, float* lse, const Dims& D,
                                    bool bf16_io, hipStream_t st) {
  if (K < 1 || K > 16) return hipErrorInvalidValue;
  if (bf16_io) {
    if (D.d == 128)
      return launch_paged_topk_decode_d<128, bf16>(q, k_pool, v_pool, qs, ks_pool, table, lens,
                                                   pages, K, renorm, idx, bias, o, lse, D, st);
    if (D.d == 64)
      return launch_paged_topk_decode_d<64, bf16>(q, k_pool, v_pool, qs, ks_pool, table, lens,
                                                  pages, K, renorm, idx, bias, o, lse, D, st);
  } else if (D.d == 64) {
    return launch_paged_topk_decode_d<64, float>(q, k_pool, v_pool, qs, ks_pool, table, lens,
                                                 pages, K, renorm, idx, bias, o, lse, D, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace sas
