// threshold.hip -- dynamic-threshold block selection with CSR output.
//
// Blog "SAS Learns Token Importance for Sparse Attention", "Implementation
// and Efficiency": attention is computed only for the blocks whose selector
// score clears a threshold that moves with the query.  Here the threshold
// applies to the normalised gate g_j = exp(z_j - lam) (lam = log sum over the
// query's historical blocks of exp z): block j < c(t) is kept when
// z_j - lam >= log(theta) (theta <= 0 keeps every historical block).  The
// number kept varies per row, so the result is CSR: row_ptr [rows + 1]
// (int64), then col / bias [nnz] with each row's blocks in ascending order.
//
// Two calls: a count pass writes every row's count into row_ptr[r + 1] and
// scans it in place (row_ptr[0] = 0, row_ptr[rows] = nnz); after the caller
// has sized col / bias, a fill pass writes them.  Both passes run the same
// kernel (one `fill` flag, uniform per launch), so the predicate is evaluated
// by the same instructions and the counts always match the entries.
//
// bf16 selectors (thr_mfma_kernel): the scores of 32 rows x 64 units come
// from matrix products, as in the gate kernel, recomputed per pass: the
// normaliser in one online pass, then the count, or the (renormalised) bias
// and the entries.  fp32 selectors (thr_kernel): one lane per row, the 64
// rows of a wave consecutive positions of one (batch, head), every ks row a
// wave-uniform load, the same passes with per-lane dot products.
#include "sas_device.h"
#include "sas_internal.h"

#include <algorithm>
#include <type_traits>

namespace sas {

template <int DS, typename ST>
__global__ __launch_bounds__(256) void thr_kernel(const ST* __restrict__ qs,
                                                  const ST* __restrict__ ks, float theta,
                                                  int renorm, int fill,
                                                  long long* __restrict__ row_ptr,
                                                  int* __restrict__ col, float* __restrict__ bias,
                                                  long long nnz, Dims D) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int wave_first = __builtin_amdgcn_readfirstlane(blockIdx.x * 256 + (threadIdx.x & ~63));
  if (wave_first >= D.tq) return;
  const bool active = i < D.tq;
  const int ic = min(i, D.tq - 1);
  const int c = active ? (D.qoff + ic) / D.blk : 0;
  const int cw = (D.qoff + min(wave_first + 63, D.tq - 1)) / D.blk;  // wave max of c
  const size_t row = ((size_t)b * D.hq + h) * D.tq + ic;
  SelQ<DS, ST> qsv;  // bf16 rows: packed bf16 dot products
  qsv.load(qs + row * DS);
  const ST* ksb = ks + ((size_t)b * D.hks + h / D.hps) * (size_t)D.nb * DS;
  const float zs = D.sel_scale * kLog2e;  // scores in log2 units
  auto z2 = [&](int j) __attribute__((always_inline)) {
    return zs * qsv.dot(ksb + (size_t)j * DS);
  };
  // lam2 = m + log2 sum 2^(z2 - m) over j < c, online in chunks of 8 blocks
  float m = -INFINITY, s = 0.f;
  for (int j0 = 0; j0 < cw; j0 += 8) {
    float zz[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = j0 + k;
      zz[k] = -INFINITY;
      if (j < cw) {
        const float z = z2(j);
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
  const float lam2 = c > 0 ? m + log2f(s) : -INFINITY;
  const float lt2 = theta > 0.f ? log2f(theta) : -INFINITY;
  auto keep = [&](int j, float z) __attribute__((always_inline)) {
    return j < c && (theta <= 0.f || z - lam2 >= lt2);
  };
  if (!fill) {
    long long n = 0;
    for (int j = 0; j < cw; ++j) n += keep(j, z2(j)) ? 1 : 0;
    if (active) {
      row_ptr[row + 1] = n;
      if (row == 0) row_ptr[0] = 0;
    }
    return;
  }
  float norm2 = lam2;
  if (renorm) {
    float sk = 0.f;
    for (int j = 0; j < cw; ++j) {
      const float z = z2(j);
      if (keep(j, z)) sk += exp2f(z - m);
    }
    norm2 = sk > 0.f ? m + log2f(sk) : -INFINITY;
  }
  if (!active) return;
  // this row's entries: [row_ptr[row], row_ptr[row + 1]) clamped to [0, nnz)
  long long p = min(max(row_ptr[row], 0LL), nnz);
  const long long e = max(p, min(row_ptr[row + 1], nnz));
  for (int j = 0; j < c && p < e; ++j) {
    const float z = z2(j);
    if (keep(j, z)) {
      col[p] = j;
      bias[p] = (z - norm2) * kLn2;
      ++p;
    }
  }
}

// bf16 selectors: the same passes with the scores on the matrix cores, as
// the gate kernel forms lam.  A workgroup of 8 waves takes 256 consecutive
// rows of one (b, h), 32 rows per wave; tiles of 64 ks rows go global ->
// registers -> LDS one tile ahead; Z^T = KS QS^T on 32x32x16 MFMA leaves 32
// units of a row's tile in each lane (the other 32 in lane l ^ 32).  Pass 1:
// lam, an online log-sum-exp whose running max moves only when it grows by
// more than 8 (log2 units).  Then the count, or (renorm: one more pass for
// the kept units' log-sum-exp) the entries: each tile's kept units form a
// 64-bit mask that the two lane halves share, and a lane writes a kept unit
// at the row's running position plus the unit's rank in the mask.  Every
// pass runs the same products in the same order, so the count and fill
// launches take the same decisions.
constexpr int kThrRows = 256;

// (Four waves per SIMD, i.e. two workgroups per compute unit, for ds <= 32:
// 126 registers and no spills; ds = 64 would spill and keeps three.)
template <int DS>
__global__ __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(DS <= 32 ? 4 : 3))) void thr_mfma_kernel(
    const bf16* __restrict__ qs, const bf16* __restrict__ ks, float theta, int renorm, int fill,
    long long* __restrict__ row_ptr, int* __restrict__ col, float* __restrict__ bias,
    long long nnz, Dims D) {
  constexpr int XP = DS + 8;  // LDS row pitch (elements)
  constexpr int CH = DS / 8;  // 16-byte chunks per ks row
  constexpr int NL = 64 * CH; // chunks per tile (<= 512 threads)
  __shared__ __align__(16) bf16 X0[64 * XP];
  __shared__ __align__(16) bf16 X1[64 * XP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int r0 = blockIdx.x * kThrRows;
  const int qi = r0 + wave * 32 + l32;
  const bool valid = qi < D.tq;
  const int qc = min(qi, D.tq - 1);
  const int c = (D.qoff + qc) / D.blk;  // historical units of the row
  const int cw = (D.qoff + min(r0 + wave * 32 + 31, D.tq - 1)) / D.blk;  // wave max of c
  const int cg = (D.qoff + min(r0 + kThrRows - 1, D.tq - 1)) / D.blk;    // workgroup max
  const int ntiles = (cg + 63) / 64;
  const size_t row = ((size_t)b * D.hq + h) * D.tq + qc;
  bf16x8 qf[DS / 16];
#pragma unroll
  for (int s = 0; s < DS / 16; ++s) qf[s] = *(const bf16x8*)(qs + row * DS + 16 * s + 8 * hh);
  const bf16* ksb = ks + ((size_t)b * D.hks + h / D.hps) * (size_t)D.nb * DS;
  const float zs = D.sel_scale * kLog2e;  // scores in log2 units
  bf16x8 reg = bf16x8{};
  auto gload = [&](int j) {
    const int u = 64 * j + tid / CH;
    if (tid < NL) reg = u < D.nb ? *(const bf16x8*)(ksb + (size_t)u * DS + (tid % CH) * 8)
                                 : bf16x8{};
  };
  auto sstore = [&](bf16* Xd) {
    if (tid < NL) *(bf16x8*)&Xd[(tid / CH) * XP + (tid % CH) * 8] = reg;
  };
  // unit of register r of M-tile mt in tile j, this lane half
  auto unit = [&](int j, int mt, int r) {
    return 64 * j + 32 * mt + 8 * (r / 4) + 4 * hh + (r % 4);
  };
  // One pass over the workgroup's tiles: fn(j, z) with z the log2-domain
  // scores of this lane's units of tile j (waves whose rows have no unit in
  // the tile skip it; every wave meets every barrier)
  auto pass = [&](auto&& fn) {
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
                *(const bf16x8*)&Xs[(32 * mt + l32) * XP + 16 * s + 8 * hh], qf[s], z[mt], 0, 0,
                0);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) z[mt][r] *= zs;
        fn(j, z);
      }
      if (j + 1 < ntiles) sstore((j & 1) ? X0 : X1);
      __syncthreads();
    }
  };
  // pass 1: lam2 = m + log2 sum 2^(z - m) over the row's units u < c
  float m_run = -INFINITY, s_run = 0.f;
  pass([&](int j, const f32x16 (&z)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (unit(j, mt, r) < c) mx = fmaxf(mx, z[mt][r]);
    mx = halves_max(mx);
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
      for (int r = 0; r < 16; ++r)
        if (unit(j, mt, r) < c) ps += exp2_raw(z[mt][r] - m_run);
    s_run += m_run > -INFINITY ? ps : 0.f;
  });
  s_run = halves_sum(s_run);
  const float lam2 = c > 0 ? m_run + log2f(s_run) : -INFINITY;
  const float lt2 = theta > 0.f ? log2f(theta) : -INFINITY;
  auto keep = [&](int u, float z) __attribute__((always_inline)) {
    return u < c && (theta <= 0.f || z - lam2 >= lt2);
  };
  if (!fill) {
    float n = 0.f;  // exact: at most nb < 2^24
    pass([&](int j, const f32x16 (&z)[2]) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) n += keep(unit(j, mt, r), z[mt][r]) ? 1.f : 0.f;
    });
    n = halves_sum(n);
    if (valid && hh == 0) {
      row_ptr[row + 1] = (long long)n;
      if (row == 0) row_ptr[0] = 0;
    }
    return;
  }
  float norm2 = lam2;
  if (renorm) {
    float sk = 0.f;
    pass([&](int j, const f32x16 (&z)[2]) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (keep(unit(j, mt, r), z[mt][r])) sk += exp2_raw(z[mt][r] - m_run);
    });
    sk = halves_sum(sk);
    norm2 = sk > 0.f ? m_run + log2f(sk) : -INFINITY;
  }
  // this row's entries: [row_ptr[row], row_ptr[row + 1]) clamped to [0, nnz)
  // (at most nb of them); padding rows write nothing
  const long long p0 = min(max(row_ptr[row], 0LL), nnz);
  const long long e = valid ? max(p0, min(row_ptr[row + 1], nnz)) : p0;
  int* cp = col + p0;
  float* bp = bias + p0;
  int room = (int)min(e - p0, (long long)D.nb);
  pass([&](int j, const f32x16 (&z)[2]) {
    // keep bits in register order (bit 4 n + i: register 4 (n % 4) + i of
    // M-tile n / 4, unit 8 n + 4 hh + i of the tile), then in unit order:
    // nibble n moves to bits 8 n .. 8 n + 3, and up by 4 in the upper half
    unsigned kb = 0u;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        kb |= keep(unit(j, mt, r), z[mt][r]) ? 1u << (16 * mt + r) : 0u;
    unsigned long long y = kb;
    y = (y | (y << 16)) & 0x0000FFFF0000FFFFull;
    y = (y | (y << 8)) & 0x00FF00FF00FF00FFull;
    y = (y | (y << 4)) & 0x0F0F0F0F0F0F0F0Full;
    const unsigned long long mine = hh ? y << 4 : y;
    const unsigned long long all = mine | lane_xor_u64<32>(mine, lane);
    // a kept unit's entry: the row's running position plus its rank in the
    // tile (the units of the bytes below, the lower half's nibble of its own
    // byte when hh = 1, its own nibble's bits below it)
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const unsigned nib = (kb >> (4 * n)) & 15u;
      const int base = __builtin_popcountll(all & ((1ull << (8 * n)) - 1ull)) +
                       (hh ? __builtin_popcount((unsigned)(all >> (8 * n)) & 15u) : 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int off = base + __builtin_popcount(nib & ((1u << i) - 1u));
        if (((nib >> i) & 1u) && off < room) {
          cp[off] = 64 * j + 8 * n + 4 * hh + i;
          bp[off] = (z[n / 4][4 * (n % 4) + i] - norm2) * kLn2;
        }
      }
    }
    const int nt = __builtin_popcountll(all);
    cp += nt;
    bp += nt;
    room -= nt;
  });
}

// In-place inclusive scan of a[0 .. n-1] (int64): per-workgroup scans of
// kScanTile elements, an exclusive scan of the tile totals, then the offsets.
constexpr int kScanTile = 4096;  // 1024 threads x 4

__global__ __launch_bounds__(1024) void thr_scan_tile_kernel(long long* __restrict__ a, size_t n,
                                                             long long* __restrict__ tot) {
  __shared__ long long sh[1024];
  const int tid = threadIdx.x;
  const size_t base = (size_t)blockIdx.x * kScanTile + (size_t)tid * 4;
  long long v[4], run = 0;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    v[x] = base + x < n ? a[base + x] : 0;
    run += v[x];
    v[x] = run;
  }
  sh[tid] = run;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const long long y = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += y;
    __syncthreads();
  }
  const long long before = sh[tid] - run;
#pragma unroll
  for (int x = 0; x < 4; ++x)
    if (base + x < n) a[base + x] = v[x] + before;
  if (tid == 1023) tot[blockIdx.x] = sh[1023];
}

__global__ __launch_bounds__(1024) void thr_scan_totals_kernel(long long* __restrict__ tot,
                                                               int nt) {
  __shared__ long long sh[1024];
  const int tid = threadIdx.x;
  const int per = (nt + 1023) / 1024;
  const int lo = min(nt, tid * per), hi = min(nt, lo + per);
  long long a = 0;
  for (int x = lo; x < hi; ++x) a += tot[x];
  sh[tid] = a;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const long long y = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += y;
    __syncthreads();
  }
  long long run = sh[tid] - a;  // exclusive prefix of this thread's range
  for (int x = lo; x < hi; ++x) {
    const long long t = tot[x];
    tot[x] = run;
    run += t;
  }
}

__global__ __launch_bounds__(1024) void thr_scan_add_kernel(long long* __restrict__ a, size_t n,
                                                            const long long* __restrict__ tot) {
  const long long off = tot[blockIdx.x];
  const size_t base = (size_t)blockIdx.x * kScanTile;
  for (int x = threadIdx.x; x < kScanTile; x += 1024)
    if (base + x < n) a[base + x] += off;
}

size_t threshold_workspace(const Dims& D) {
  const size_t rows = (size_t)D.batch * D.hq * D.tq;
  return ((rows + kScanTile - 1) / kScanTile) * sizeof(long long);
}

template <int DS, typename ST>
static hipError_t launch_thr_t(const void* qs, const void* ks, float theta, int renorm, int fill,
                               long long* row_ptr, int* col, float* bias, long long nnz,
                               char* ws, const Dims& D, hipStream_t st) {
  if (std::is_same<ST, bf16>::value)
    hipLaunchKernelGGL((thr_mfma_kernel<DS>),
                       dim3((D.tq + kThrRows - 1) / kThrRows, D.hq, D.batch), dim3(512), 0, st,
                       (const bf16*)qs, (const bf16*)ks, theta, renorm, fill, row_ptr, col, bias,
                       nnz, D);
  else
    hipLaunchKernelGGL((thr_kernel<DS, ST>), dim3((D.tq + 255) / 256, D.hq, D.batch), dim3(256), 0,
                       st, (const ST*)qs, (const ST*)ks, theta, renorm, fill, row_ptr, col, bias,
                       nnz, D);
  if (fill) return hipGetLastError();
  const size_t rows = (size_t)D.batch * D.hq * D.tq;
  const int nt = (int)((rows + kScanTile - 1) / kScanTile);
  long long* tot = (long long*)ws;
  hipLaunchKernelGGL(thr_scan_tile_kernel, dim3(nt), dim3(1024), 0, st, row_ptr + 1, rows, tot);
  hipLaunchKernelGGL(thr_scan_totals_kernel, dim3(1), dim3(1024), 0, st, tot, nt);
  hipLaunchKernelGGL(thr_scan_add_kernel, dim3(nt), dim3(1024), 0, st, row_ptr + 1, rows,
                     (const long long*)tot);
  return hipGetLastError();
}

hipError_t launch_threshold(const void* qs, const void* ks, float theta, int renorm, int fill,
                            long long* row_ptr, int* col, float* bias, long long nnz, char* ws,
                            const Dims& D, bool sel_bf16, hipStream_t st) {
#define SAS_THR_CASE(DSV)                                                                      \
  case DSV:                                                                                    \
    return sel_bf16 ? launch_thr_t<DSV, bf16>(qs, ks, theta, renorm, fill, row_ptr, col, bias, \
                                              nnz, ws, D, st)                                  \
                    : launch_thr_t<DSV, float>(qs, ks, theta, renorm, fill, row_ptr, col,      \
                                               bias, nnz, ws, D, st);
  switch (D.ds) {
    SAS_THR_CASE(16)
    SAS_THR_CASE(32)
    SAS_THR_CASE(64)
  }
#undef SAS_THR_CASE
  return hipErrorInvalidValue;
}

}  // namespace sas
