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
// rank on (score descending, block ascending); the scores are fp32 sums of
// the exact bf16 products, from packed dot products (SelQ) or from MFMA
// tiles, so kernels agree on every row whose scores are apart by more than
// the last bits of fp32, and within one kernel exactly equal scores (ties)
// always go to the smaller block.
//
// Wave per row: the row's scores are computed once into LDS (lane j % 64
// owns block j), lam comes from a wave max + sum, then K rounds each pick the
// best remaining block with a 64-lane argmax on (z, -j): round r takes the
// best candidate strictly after round r-1's winner in that total order, so
// no "already taken" set is needed.
#include "sas_device.h"
#include "sas_internal.h"
#include "select_device.h"

namespace sas {

__device__ __forceinline__ bool better(float za, int ja, float zb, int jb) {
  return za > zb || (za == zb && ja < jb);
}

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

// Lane-per-row variant for many rows and K <= 32: the 64 rows of a wave are
// consecutive positions of one (batch, head) and share the ks rows they
// score.  Each lane keeps its best KMAX (>= K) blocks in registers as 64-bit
// keys (ord_key of z above, the complement of the block below), so that one
// unsigned comparison gives the selection order (z descending, block
// ascending) and no two candidates tie.  Candidates come 16 at a time and
// are folded in batches of 8: the batch is sorted by a 19-comparator
// network, each of the last 8 list entries keeps the larger of itself and
// its mirror in the batch (the list then holds the best KMAX of both, in
// bitonic order), and a bitonic merge sorts it again; every step is
// branch-free, so the lanes of a wave never wait on each other's insertions.
//
// Scores.  bf16 selectors: the wave's 64 x 16 score tile is a small matrix
// product on the matrix cores (lane_tile_scores below: exact bf16 products,
// fp32 sums in the MFMA's order, so a score may differ in its last bits from
// the packed-dot SelQ score of the other kernels; equal selector vectors
// still give equal scores, and the order on ties is unchanged).  f32
// selectors: SelQ, lane by lane.
template <int DS>
struct LaneTile {
  static constexpr int NK = (DS + 31) / 32;  // 16x16x32 products per 16 rows
  bf16x8 qb[4][NK];                          // B operands: rows 16 r + lane % 16

  // qs rows first .. first + 63 of the (batch, head) whose rows start at q0
  // (rows past tq - 1 repeat it).  16x16x32 operand layout: lane l holds
  // row / column l % 16 and k = 8 (l / 16) .. + 7 of each 32-wide k slice.
  __device__ __forceinline__ void load(const bf16* q0, int first, int tq, int lane) {
    const int kg = 8 * (lane >> 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bf16* p = q0 + (size_t)min(first + 16 * r + (lane & 15), tq - 1) * DS;
#pragma unroll
      for (int s = 0; s < NK; ++s)
        qb[r][s] = 32 * s + kg < DS ? *(const bf16x8*)(p + 32 * s + kg) : bf16x8{};
    }
  }

  // Unscaled scores of blocks j0 .. j0 + 15 (rows of ksb past nb - 1 repeat
  // it) for this lane's row: z[4 g + v] for block j0 + 4 g + v.  Product r
  // leaves lane l with row 16 r + l % 16, blocks j0 + 4 (l / 16) + v; the 4 x 4
  // transpose of (product, 16-lane row) that gives lane l its own row is two
  // rounds of register swaps, v_permlane32_swap (rows g, g ^ 2) and then
  // v_permlane16_swap (rows g, g ^ 1).  The whole wave must be active.
  __device__ __forceinline__ void score(const bf16* ksb, int j0, int nb, int lane,
                                        float (&z)[16]) const {
    const int kg = 8 * (lane >> 4);
    const bf16* kp = ksb + (size_t)min(j0 + (lane & 15), nb - 1) * DS;
    bf16x8 a[NK];
#pragma unroll
    for (int s = 0; s < NK; ++s)
      a[s] = 32 * s + kg < DS ? *(const bf16x8*)(kp + 32 * s + kg) : bf16x8{};
    f32x4 t[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      t[r] = mfma16(a[0], qb[r][0], f32x4{});
#pragma unroll
      for (int s = 1; s < NK; ++s) t[r] = mfma16(a[s], qb[r][s], t[r]);
    }
    unsigned u[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int v = 0; v < 4; ++v) u[r][v] = __float_as_uint(t[r][v]);
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const auto x = __builtin_amdgcn_permlane32_swap(u[r][v], u[r + 2][v], false, false);
        u[r][v] = x[0];
        u[r + 2][v] = x[1];
      }
#pragma unroll
    for (int r = 0; r < 4; r += 2)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const auto x = __builtin_amdgcn_permlane16_swap(u[r][v], u[r + 1][v], false, false);
        u[r][v] = x[0];
        u[r + 1][v] = x[1];
      }
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int v = 0; v < 4; ++v) z[4 * g + v] = __uint_as_float(u[g][v]);
  }
};

// One batch of 8 scores zz (blocks j0 .. j0 + 7, -inf at or after c) into
// the running log-sum-exp (log2 domain: m, s) and the list tk.
template <int KMAX>
__device__ __forceinline__ void lane_fold8(const float (&zz)[8], int j0, float& m,
                                           float& s, unsigned long long (&tk)[KMAX]) {
  float mc = zz[0];
#pragma unroll
  for (int kk = 1; kk < 8; ++kk) mc = fmaxf(mc, zz[kk]);
  const float mn = fmaxf(m, mc * kLog2e);
  if (mn != -INFINITY) {
    float acc = s * exp2_raw(m - mn);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) acc += exp2_raw(zz[kk] * kLog2e - mn);
    s = acc;
    m = mn;
  }
  // the batch as keys, sorted.  Blocks at or after c score -inf, whose key
  // lies below that of every finite score: they fill only list entries at or
  // past c, which are never output.
  unsigned long long bk[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    bk[kk] = ((unsigned long long)ord_key(zz[kk]) << 32) | (unsigned)~(j0 + kk);
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

template <int DS, typename ST, int KMAX>
__global__ __launch_bounds__(256) void topk_lane_kernel(const ST* __restrict__ qs,
                                                        const ST* __restrict__ ks, int K,
                                                        int renorm, int* __restrict__ idx,
                                                        float* __restrict__ bias, Dims D) {
  static_assert(KMAX >= 8 && (KMAX & (KMAX - 1)) == 0, "KMAX: a power of two >= 8");
  constexpr bool kTile = std::is_same<ST, bf16>::value;
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int wave_first = __builtin_amdgcn_readfirstlane(blockIdx.x * 256 + (threadIdx.x & ~63));
  if (wave_first >= D.tq) return;
  const int ic = min(i, D.tq - 1);
  const int c = (D.qoff + ic) / D.blk;
  const int cw = (D.qoff + min(wave_first + 63, D.tq - 1)) / D.blk;  // wave max of c
  const size_t row0 = ((size_t)b * D.hq + h) * D.tq, row = row0 + ic;
  const ST* ksb = ks + ((size_t)b * D.hks + h / D.hps) * (size_t)D.nb * DS;
  LaneTile<DS> tile;
  SelQ<DS, ST> qsv;
  if constexpr (kTile)
    tile.load((const bf16*)qs + row0 * DS, wave_first, D.tq, lane);
  else
    qsv.load(qs + row * DS);
  unsigned long long tk[KMAX];  // best blocks, key descending; 0 = empty
#pragma unroll
  for (int r = 0; r < KMAX; ++r) tk[r] = 0ull;
  float m = -INFINITY, s = 0.f;  // log2-domain running log-sum-exp of z
  for (int j0 = 0; j0 < cw; j0 += 16) {
    float z[16];
    if constexpr (kTile) {
      tile.score((const bf16*)ksb, j0, D.nb, lane, z);
    } else {
#pragma unroll
      for (int kk = 0; kk < 16; ++kk)
        z[kk] = j0 + kk < cw ? qsv.dot(ksb + (size_t)(j0 + kk) * DS) : 0.f;
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      if (hf == 1 && j0 + 8 >= cw) break;  // wave-uniform
      float zz[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        zz[kk] = j0 + 8 * hf + kk < c ? D.sel_scale * z[8 * hf + kk] : -INFINITY;
      lane_fold8<KMAX>(zz, j0 + 8 * hf, m, s, tk);
    }
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

// Wave per row for few rows and K <= KM (decode, paged decode, small calls):
// wave_best (select_device.h) leaves every lane with the row's best KM keys
// and its log-sum-exp; lane r < K writes entry r.
template <int DS, typename ST, typename Sel, int KM>
__global__ __launch_bounds__(256) void topk_merge_kernel(const ST* __restrict__ qs, Sel S, int K,
                                                         int renorm, int* __restrict__ idx,
                                                         float* __restrict__ bias, Dims D) {
  const int lane = threadIdx.x & 63;
  const size_t nrows = (size_t)D.batch * D.hq * D.tq;
  const size_t row = (size_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= nrows) return;  // whole wave (no workgroup barrier below)
  int j;
  float bs;
  wave_best_entry<DS, ST, Sel, KM>(qs, S, D, row, K, renorm, lane, &j, &bs);
  if (lane < K) {
    idx[row * K + lane] = j;
    bias[row * K + lane] = bs;
  }
}

// Budgeted / large-K variant: one wavefront per query row keeps the
// n_t = min(kmax, c(t), ceil(num c(t) / den)) best blocks (num <= 0: no
// fraction; the ceiling in exact integer arithmetic).  Scores go to LDS (same SelQ dot product as above) and become
// order-preserving 32-bit keys; a radix select (8 bits per pass, LDS
// histogram) narrows down the n_t-th largest key, stopping early once the bin
// that holds it is needed whole; keys tied with it are taken in block order;
// the n_t winners are then sorted (bitonic network in LDS) by key
// descending, block ascending — the same order as the other kernels.

// Register bitonic sort of a row's winners (partners by lane_xor).
// One bitonic step at lane distance S over the E keys of each lane (key e of
// lane l is element x = 64 e + l): x keeps the larger of itself and x ^ S
// when x is the lower of the two in a block sorted descending ((x & size) ==
// 0), or the higher in an ascending one; else the smaller.
template <int S, int E>
__device__ __forceinline__ void bitonic_lanes(unsigned long long (&v)[E], int lane, int size) {
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const unsigned lo = lane_xor<S>((unsigned)v[e], lane);
    const unsigned hi = lane_xor<S>((unsigned)(v[e] >> 32), lane);
    const unsigned long long o = ((unsigned long long)hi << 32) | lo;
    const int x = 64 * e + lane;
    const bool keep_max = ((x & S) == 0) == ((x & size) == 0);
    v[e] = (keep_max ? o > v[e] : o < v[e]) ? o : v[e];
  }
}

// Sorts the n winning blocks sj [0, n) (their keys: zk [block]) into
// selection order (z descending, block ascending), p2 = the power of two
// >= n, p2 <= 64 E: 64-bit keys (ord_key << 32 | ~block) held E per lane
// (position 64 e + lane in v [e]), padding 0 (below every real key), and
// writes the row's kmax outputs from the sorted registers: block and score
// minus the normaliser (lam, or with renorm the log-sum-exp of the winners'
// scores), -1 and -inf past n.
template <int E>
__device__ __forceinline__ void sort_emit(const unsigned* zk, const int* sj, int n, int p2,
                                          int lane, int kmax, int renorm, float lam, size_t row,
                                          int* __restrict__ idx, float* __restrict__ bias) {
  unsigned long long v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int x = 64 * e + lane;
    const int j = x < n ? sj[x] : 0;
    v[e] = x < n ? ((unsigned long long)zk[j] << 32) | (unsigned)~j : 0ull;
  }
  for (int size = 2; size <= p2; size <<= 1) {
    // distances of 64 elements and more: within the lane
    if constexpr (E >= 4) {
      if (size >= 256) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const bool desc = ((64 * e + lane) & size) == 0;
          const bool sw = desc ? v[e + 2] > v[e] : v[e + 2] < v[e];
          const unsigned long long a = v[e], b = v[e + 2];
          v[e] = sw ? b : a;
          v[e + 2] = sw ? a : b;
        }
      }
    }
    if constexpr (E >= 2) {
      if (size >= 128) {
#pragma unroll
        for (int e = 0; e < E; e += 2) {
          const bool desc = ((64 * e + lane) & size) == 0;
          const bool sw = desc ? v[e + 1] > v[e] : v[e + 1] < v[e];
          const unsigned long long a = v[e], b = v[e + 1];
          v[e] = sw ? b : a;
          v[e + 1] = sw ? a : b;
        }
      }
    }
    if (size > 32) bitonic_lanes<32>(v, lane, size);
    if (size > 16) bitonic_lanes<16>(v, lane, size);
    if (size > 8) bitonic_lanes<8>(v, lane, size);
    if (size > 4) bitonic_lanes<4>(v, lane, size);
    if (size > 2) bitonic_lanes<2>(v, lane, size);
    bitonic_lanes<1>(v, lane, size);
  }
  float norm = lam;
  if (renorm) {
    // the best winner sits at position 0
    const float mm = key_value((unsigned)__builtin_amdgcn_readlane((int)(unsigned)(v[0] >> 32), 0));
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (64 * e + lane < n) ss += exp2f((key_value((unsigned)(v[e] >> 32)) - mm) * kLog2e);
    ss = wave_sum(ss);
    norm = n == 0 ? -INFINITY : mm + log2f(ss) * kLn2;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int x = 64 * e + lane;
    if (x < kmax) {
      idx[row * kmax + x] = x < n ? (int)~(unsigned)v[e] : -1;
      bias[row * kmax + x] = x < n ? key_value((unsigned)(v[e] >> 32)) - norm : -INFINITY;
    }
  }
  for (int x = 64 * E + lane; x < kmax; x += 64) {  // n <= 64 E: padding only
    idx[row * kmax + x] = -1;
    bias[row * kmax + x] = -INFINITY;
  }
}

// The selection of one query row (row) from its scores zc [0, c) in LDS
// (m: their maximum, or -inf with c = 0), by one wavefront.  One pass over
// the scores gives the gate normaliser lam, turns each score into its
// ord_key in place (zk; a score comes back from its key exactly, up to the
// sign of a zero) and counts the first radix digit: key bits 31..20 (8
// values per octave of the score), over the 256 values at and below the
// top key's only.  (A digit of the top 8 bits alone would put most scores
// of a row into a handful of bins, whose LDS atomics serialise.)  When the
// bin holding the n-th best key has at most 64 keys, one more pass writes
// the blocks above that bin to sj and the bin's blocks after them, and each
// of those candidates ranks itself among the others on the unique 64-bit
// order (key, ~block) to settle which are taken.  Otherwise (a larger bin,
// or a window holding fewer than n keys) radix passes over all keys resolve
// the remaining bits and a gather takes the keys above the resulting
// prefix, then the first keys on it by block.  The n winners are then sorted
// and written out.  hist: 256 words, sj: kp2 + 64 words, this wave's own.
__device__ __forceinline__ void select_row(float* zc, float m, int c, int n, int kmax,
                                           int renorm, unsigned* hist, int* sj, size_t row,
                                           int* __restrict__ idx, float* __restrict__ bias,
                                           int lane) {
  unsigned* zk = (unsigned*)zc;
  const unsigned long long lt = lane == 0 ? 0ull : ~0ull >> (64 - lane);  // lanes below
  const unsigned top = c > 0 ? ord_key(m) >> 20 : 0u;
  if (n > 0)
    for (int x = lane; x < 256; x += 64) hist[x] = 0;
  float sum = 0.f;
  for (int j = lane; j < c; j += 64) {  // c > 0: m finite
    const float z = zc[j];
    sum += exp2_raw((z - m) * kLog2e);
    const unsigned k = ord_key(z);
    zk[j] = k;
    const unsigned d = top - (k >> 20);  // keys never exceed the top one
    if (n > 0 && d < 256u) atomicAdd(&hist[d], 1u);
  }
  sum = wave_sum(sum);
  const float lam = c == 0 ? -INFINITY : m + log2f(sum) * kLn2;
  int need = n;
  unsigned prefix = 0, pmask = 0;
  // The counts in hist ranked from the top (rank r = 4 l + u on lane l, at
  // hist [dmax - r] or, !rev, hist [r]; ranks past dmax count 0): the rank
  // where the count from the top first reaches need, the count above it and
  // in it; -1 when all of them together hold fewer than need.
  auto pick = [&](bool rev, int dmax, unsigned& above, unsigned& inbin) -> int {
    unsigned cnt[4], tot = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = 4 * lane + u;
      cnt[u] = r <= dmax ? hist[rev ? dmax - r : r] : 0u;
      tot += cnt[u];
    }
    const unsigned inc = wave_incl_scan(tot, lane), exc = inc - tot;
    int rsel = -1;
    unsigned ab = 0, ib = 0;
    if (exc < (unsigned)need && inc >= (unsigned)need) {
      unsigned run = exc;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (rsel < 0 && run + cnt[u] >= (unsigned)need) {
          rsel = 4 * lane + u;
          ab = run;
          ib = cnt[u];
        }
        run += cnt[u];
      }
    }
    const unsigned long long bal = __ballot(rsel >= 0);
    if (bal == 0ull) return -1;
    const int src = __ffsll((long long)bal) - 1;  // one lane, wave-uniform
    above = (unsigned)__builtin_amdgcn_readlane((int)ab, src);
    inbin = (unsigned)__builtin_amdgcn_readlane((int)ib, src);
    return __builtin_amdgcn_readlane(rsel, src);
  };
  // One radix pass over the digit (key >> shift) & (2^bits - 1) of the keys
  // on the prefix; true once every key of the chosen digit is needed.
  auto pass = [&](int shift, int bits) -> bool {
    const unsigned dmask = (1u << bits) - 1u;
    for (int x = lane; x < 256; x += 64) hist[x] = 0;
    for (int j = lane; j < c; j += 64) {
      const unsigned kk = zk[j];
      if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & dmask], 1u);
    }
    unsigned above = 0, inbin = 0;
    const int r = pick(true, (int)dmask, above, inbin);
    need -= (int)above;
    prefix |= (dmask - (unsigned)r) << shift;
    pmask |= dmask << shift;
    return (int)inbin == need;
  };
  if (n > 0) {
    unsigned above = 0, inbin = 0;
    const int r = pick(false, 255, above, inbin);
    if (r >= 0 && inbin <= 64u) {
      int nw = 0, nc = 0;
      for (int j0 = 0; j0 < c; j0 += 64) {
        const int j = j0 + lane;
        const unsigned d = j < c ? top - (zk[j] >> 20) : ~0u;
        const bool w = d < (unsigned)r, cd = d == (unsigned)r;
        const unsigned long long bw = __ballot(w), bc = __ballot(cd);
        if (w) sj[nw + __popcll(bw & lt)] = j;
        if (cd) sj[(int)above + nc + __popcll(bc & lt)] = j;
        nw += __popcll(bw);
        nc += __popcll(bc);
      }
      need -= (int)above;
      if ((int)inbin > need) {
        const bool has = lane < (int)inbin;
        const int jt = has ? sj[(int)above + lane] : 0;
        const unsigned kh = has ? zk[jt] : 0u, kl = ~(unsigned)jt;
        const unsigned long long kt = ((unsigned long long)kh << 32) | kl;
        int rank = 0;
        for (int u = 0; u < (int)inbin; ++u) {
          const unsigned long long ku =
              ((unsigned long long)(unsigned)__builtin_amdgcn_readlane((int)kh, u) << 32) |
              (unsigned)__builtin_amdgcn_readlane((int)kl, u);
          rank += ku > kt;
        }
        const bool take = has && rank < need;
        const unsigned long long bt = __ballot(take);
        if (take) sj[(int)above + __popcll(bt & lt)] = jt;
      }
    } else {
      if (r >= 0) {
        need -= (int)above;
        prefix = (top - (unsigned)r) << 20;
        pmask = 0xFFF00000u;
        if ((int)inbin != need && !pass(12, 8) && !pass(4, 8)) pass(0, 4);
      } else {
        if (!pass(24, 8) && !pass(16, 8) && !pass(8, 8)) pass(0, 8);
      }
      // gather: keys whose resolved bits lie above the prefix, then the
      // first `need` keys on it by block (all of them when the passes
      // stopped early)
      int cnt_sel = 0, ties_left = need;
      for (int j0 = 0; j0 < c; j0 += 64) {
        const int j = j0 + lane;
        const unsigned kk = j < c ? zk[j] & pmask : 0u;
        const bool abv = j < c && kk > prefix;
        const bool tie = j < c && kk == prefix;
        const unsigned long long bt = __ballot(tie);
        const int trank = __popcll(bt & lt);
        const bool take = abv || (tie && trank < ties_left);
        const unsigned long long bs = __ballot(take);
        if (take) sj[cnt_sel + __popcll(bs & lt)] = j;
        cnt_sel += __popcll(bs);
        ties_left -= min(ties_left, (int)__popcll(bt));
      }
    }
  }
  // bitonic sort of the n winners (padded to a power of two with the worst
  // key): in registers up to 256 of them, in LDS beyond (padding block -1,
  // key 0)
  int p2 = 1;
  while (p2 < n) p2 <<= 1;
  if (p2 <= 64) {
    sort_emit<1>(zk, sj, n, p2, lane, kmax, renorm, lam, row, idx, bias);
    return;
  } else if (p2 == 128) {
    sort_emit<2>(zk, sj, n, p2, lane, kmax, renorm, lam, row, idx, bias);
    return;
  } else if (p2 == 256) {
    sort_emit<4>(zk, sj, n, p2, lane, kmax, renorm, lam, row, idx, bias);
    return;
  } else {
    for (int x = n + lane; x < p2; x += 64) sj[x] = -1;
    for (int size = 2; size <= p2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int pr = lane; pr < (p2 >> 1); pr += 64) {
          const int lo = 2 * stride * (pr / stride) + (pr % stride), hi = lo + stride;
          const int ja = sj[lo], jb = sj[hi];
          const unsigned ka = ja < 0 ? 0u : zk[ja], kb2 = jb < 0 ? 0u : zk[jb];
          const bool first_better = key_before(ka, ja, kb2, jb);
          const bool want_better_first = (lo & size) == 0;
          if (first_better != want_better_first) {
            sj[lo] = jb;
            sj[hi] = ja;
          }
        }
      }
    }
  }
  // outputs
  float norm = lam;
  if (renorm) {
    float mm = -INFINITY;
    for (int r = lane; r < n; r += 64) mm = fmaxf(mm, key_value(zk[sj[r]]));
    mm = wave_max(mm);
    float ss = 0.f;
    for (int r = lane; r < n; r += 64) ss += exp2f((key_value(zk[sj[r]]) - mm) * kLog2e);
    ss = wave_sum(ss);
    norm = n == 0 ? -INFINITY : mm + log2f(ss) * kLn2;
  }
  for (int r = lane; r < kmax; r += 64) {
    if (r < n) {
      const int j = sj[r];
      idx[row * kmax + r] = j;
      bias[row * kmax + r] = key_value(zk[j]) - norm;
    } else {
      idx[row * kmax + r] = -1;
      bias[row * kmax + r] = -INFINITY;
    }
  }
}

template <int DS, typename ST>
__global__ __launch_bounds__(256) void topk_select_kernel(const ST* __restrict__ qs,
                                                          const ST* __restrict__ ks, int kmax,
                                                          int fnum, int fden, int renorm,
                                                          int* __restrict__ idx,
                                                          float* __restrict__ bias, Dims D,
                                                          int kp2, int wpg) {
  extern __shared__ unsigned tsm[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int per = D.nb + 256 + kp2 + 64;
  float* zc = (float*)(tsm + (size_t)wave * per);  // scores of this row's blocks
  unsigned* hist = tsm + (size_t)wave * per + D.nb;  // radix histogram
  int* sj = (int*)(hist + 256);                      // selected blocks
  const size_t nrows = (size_t)D.batch * D.hq * D.tq;
  const size_t row = (size_t)blockIdx.x * wpg + wave;
  if (row >= nrows) return;  // whole wave (no workgroup barrier below)
  const int i = (int)(row % D.tq);
  const int h = (int)((row / D.tq) % D.hq);
  const int b = (int)(row / ((size_t)D.tq * D.hq));
  const int c = (D.qoff + i) / D.blk;
  int n = min(kmax, c);
  if (fnum > 0) n = (int)min((long long)n, ((long long)fnum * c + fden - 1) / fden);
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
  select_row(zc, m, c, n, kmax, renorm, hist, sj, row, idx, bias, lane);
}

// The same selection for bf16 selectors, RW consecutive query rows of one
// (batch, head) per workgroup of four waves.  The rows share their ks
// history, so the workgroup reads it once: wave w scores the 16-block tiles
// w, w + 4, ... for all RW rows with one 16x16x32 matrix product per k slice
// (A = the tile's 16 ks rows, B = the RW qs rows, padded to 16 columns; exact
// bf16 products summed by the MFMA, as in the lane kernel) into LDS, and
// after one barrier each wave runs select_row on RW / 4 of the rows.
template <int DS, int RW>
__global__ __launch_bounds__(256) void topk_select_tile_kernel(
    const bf16* __restrict__ qs, const bf16* __restrict__ ks, int kmax, int fnum, int fden,
    int renorm, int* __restrict__ idx, float* __restrict__ bias, Dims D, int kp2, int nbp) {
  static_assert(RW == 4 || RW == 8 || RW == 16, "RW: 4, 8 or 16 rows");
  constexpr int NK = (DS + 31) / 32;  // k slices of 32
  extern __shared__ unsigned tsm[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  float* zs = (float*)tsm;  // RW rows of nbp scores
  unsigned* hist = tsm + (size_t)RW * nbp + (size_t)wave * (256 + kp2 + 64);
  int* sj = (int*)(hist + 256);
  const int tiles = (D.tq + RW - 1) / RW;
  const int bh = blockIdx.x / tiles;  // b * hq + h
  const int i0 = (blockIdx.x - bh * tiles) * RW;
  const int h = bh % D.hq, b = bh / D.hq;
  const int ilast = min(i0 + RW, D.tq) - 1;
  const int cmax = (D.qoff + ilast) / D.blk;
  const size_t row0 = (size_t)bh * D.tq;
  const bf16* ksb = ks + ((size_t)b * D.hks + h / D.hps) * (size_t)D.nb * DS;
  // 16x16x32 operands: lane l holds row / column l % 16, k = 8 (l / 16) .. + 7
  const int kg = 8 * (lane >> 4), r16 = lane & 15;
  bf16x8 qb[NK];
  {
    const bf16* p = qs + (row0 + min(i0 + r16, ilast)) * DS;
#pragma unroll
    for (int s = 0; s < NK; ++s)
      qb[s] = 32 * s + kg < DS ? *(const bf16x8*)(p + 32 * s + kg) : bf16x8{};
  }
  // four tiles per round (their loads in flight together); a tile past cmax
  // reads clamped rows and is not stored
  for (int j00 = 16 * wave; j00 < cmax; j00 += 256) {
    bf16x8 a[4][NK];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bf16* kp = ksb + (size_t)min(j00 + 64 * u + r16, D.nb - 1) * DS;
#pragma unroll
      for (int s = 0; s < NK; ++s)
        a[u][s] = 32 * s + kg < DS ? *(const bf16x8*)(kp + 32 * s + kg) : bf16x8{};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j0 = j00 + 64 * u;
      f32x4 t = f32x4{};
#pragma unroll
      for (int s = 0; s < NK; ++s) t = mfma16(a[u][s], qb[s], t);
      // lane: row i0 + r16, blocks j0 + 4 (lane / 16) .. + 3 (those at or
      // past the row's c are never read)
      if (r16 < RW && j0 < cmax)
        *(f32x4*)(zs + (size_t)r16 * nbp + j0 + 4 * (lane >> 4)) = D.sel_scale * t;
    }
  }
  __syncthreads();
  for (int q = 0; q < RW / 4; ++q) {
    const int i = i0 + wave * (RW / 4) + q;
    if (i > ilast) break;  // whole wave (no workgroup barrier below)
    const int c = (D.qoff + i) / D.blk;
    int n = min(kmax, c);
    if (fnum > 0) n = (int)min((long long)n, ((long long)fnum * c + fden - 1) / fden);
    float* zc = zs + (size_t)(i - i0) * nbp;
    float m = -INFINITY;
    for (int j = lane; j < c; j += 64) m = fmaxf(m, zc[j]);
    m = wave_max(m);
    select_row(zc, m, c, n, kmax, renorm, hist, sj, row0 + i, idx, bias, lane);
  }
}

// LDS bytes of the tiled selection with RW rows per workgroup.
static size_t select_tile_bytes(const Dims& D, int kp2, int RW, int* nbp) {
  *nbp = (D.nb + 15) / 16 * 16 + 4;  // whole 16-block tiles, rows 16 B apart off the banks
  return ((size_t)RW * *nbp + 4 * (size_t)(256 + kp2 + 64)) * sizeof(unsigned);
}

template <int DS, typename ST>
static hipError_t launch_select_t(const void* qs, const void* ks, int kmax, int fnum, int fden,
                                  int renorm,
                                  int* idx, float* bias, const Dims& D, hipStream_t st) {
  int kp2 = 1;
  while (kp2 < kmax) kp2 <<= 1;
  if constexpr (std::is_same<ST, bf16>::value) {
    // 16 or 8 rows per workgroup while eight workgroups (32 waves) still fit
    // a CU's 160 KiB of LDS, else 4 rows (at most 64 KiB): the selection
    // phase needs the waves more than the scoring needs the shared reads
    int nbp = 0;
    const unsigned tiles16 = (unsigned)((D.tq + 15) / 16), tiles8 = (unsigned)((D.tq + 7) / 8),
                   tiles4 = (unsigned)((D.tq + 3) / 4), bh = (unsigned)(D.batch * D.hq);
#define SAS_TILE_LAUNCH(RWV, TILES, CAP)                                                       \
  if (select_tile_bytes(D, kp2, RWV, &nbp) <= CAP) {                                          \
    hipLaunchKernelGGL((topk_select_tile_kernel<DS, RWV>), dim3(bh * TILES), dim3(256),       \
                       select_tile_bytes(D, kp2, RWV, &nbp), st, (const bf16*)qs,             \
                       (const bf16*)ks, kmax, fnum, fden, renorm, idx, bias, D, kp2, nbp);    \
    return hipGetLastError();                                                                 \
  }
    SAS_TILE_LAUNCH(16, tiles16, 20480)
    SAS_TILE_LAUNCH(8, tiles8, 20480)
    SAS_TILE_LAUNCH(4, tiles4, 65536)
#undef SAS_TILE_LAUNCH
  }
  const size_t per = (size_t)(D.nb + 256 + kp2 + 64) * sizeof(unsigned);
  int wpg = 4;  // rows (waves) per workgroup, as many as 64 KiB of LDS holds
  while (wpg > 1 && per * wpg > 65536) wpg >>= 1;
  const size_t nrows = (size_t)D.batch * D.hq * D.tq;
  hipLaunchKernelGGL((topk_select_kernel<DS, ST>), dim3((unsigned)((nrows + wpg - 1) / wpg)),
                     dim3(64 * wpg), per * wpg, st, (const ST*)qs, (const ST*)ks, kmax, fnum,
                     fden, renorm, idx, bias, D, kp2, wpg);
  return hipGetLastError();
}

bool topk_budget_supported(const Dims& D, int kmax) {
  int kp2 = 1;
  while (kp2 < kmax) kp2 <<= 1;
  return kmax <= 1024 && (size_t)(D.nb + 256 + kp2 + 64) * sizeof(unsigned) <= 65536;
}

hipError_t launch_topk_budget(const void* qs, const void* ks, int kmax, int fnum, int fden,
                              int renorm,
                              int* idx, float* bias, const Dims& D, bool sel_bf16,
                              hipStream_t st) {
#define SAS_SEL_CASE(DSV)                                                                     \
  case DSV:                                                                                   \
    return sel_bf16                                                                           \
               ? launch_select_t<DSV, bf16>(qs, ks, kmax, fnum, fden, renorm, idx, bias, D, st) \
               : launch_select_t<DSV, float>(qs, ks, kmax, fnum, fden, renorm, idx, bias, D, st);
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
    return launch_select_t<DS, ST>(qs, ks, K, 0, 1, renorm, idx, bias, D, st);
  const size_t nrows = (size_t)D.batch * D.hq * D.tq;
  if (K <= 16) {
    const unsigned grid = (unsigned)((nrows + 3) / 4);
    if (K <= 8)
      hipLaunchKernelGGL((topk_merge_kernel<DS, ST, DenseSel<ST>, 8>), dim3(grid), dim3(256), 0,
                         st, (const ST*)qs, DenseSel<ST>{(const ST*)ks}, K, renorm, idx, bias, D);
    else
      hipLaunchKernelGGL((topk_merge_kernel<DS, ST, DenseSel<ST>, 16>), dim3(grid), dim3(256), 0,
                         st, (const ST*)qs, DenseSel<ST>{(const ST*)ks}, K, renorm, idx, bias, D);
    return hipGetLastError();
  }
  const size_t per = (size_t)(D.nb + K) * sizeof(float);
  int wpg = 4;
  while (wpg > 1 && per * wpg > 65536) wpg >>= 1;
  if (per * wpg > 65536) return hipErrorInvalidValue;
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
  if (K <= 16) {
    const unsigned grid = (unsigned)(((size_t)D.batch * D.hq + 3) / 4);
    const PagedSel<ST> sel{(const ST*)ks_pool, table, lens, pages};
    if (K <= 8)
      hipLaunchKernelGGL((topk_merge_kernel<DS, ST, PagedSel<ST>, 8>), dim3(grid), dim3(256), 0,
                         st, (const ST*)qs, sel, K, renorm, idx, bias, D);
    else
      hipLaunchKernelGGL((topk_merge_kernel<DS, ST, PagedSel<ST>, 16>), dim3(grid), dim3(256), 0,
                         st, (const ST*)qs, sel, K, renorm, idx, bias, D);
    return hipGetLastError();
  }
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
  return use_lane_kernel(D, K) || K <= 16 || (K >= 16 && topk_budget_supported(D, K)) ||
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
