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
// One lane per row, the 64 rows of a wave consecutive positions of one
// (batch, head) as in the gate kernel: every ks row is a wave-uniform load,
// scores (packed bf16 dot products, log2 units) are recomputed per pass: the
// normaliser in one online pass, then the count, or the (renormalised) bias
// and the entries.
#include "sas_device.h"
#include "sas_internal.h"

#include <algorithm>

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
  const dim3 grid((D.tq + 255) / 256, D.hq, D.batch);
  hipLaunchKernelGGL((thr_kernel<DS, ST>), grid, dim3(256), 0, st, (const ST*)qs, (const ST*)ks,
                     theta, renorm, fill, row_ptr, col, bias, nnz, D);
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
