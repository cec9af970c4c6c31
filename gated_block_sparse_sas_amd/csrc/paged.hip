// paged.hip -- upkeep of a block-paged decode cache.
//
// A page holds one 64-key block of one sequence for every kv head
// ([pages, hkv, 64, d] for K and V) plus that block's selector key
// ([pages, hks, ds]).  Appending a token writes its K and V rows into the
// page of its block; when the token completes the block, the block's
// selector key is stored with it.  Only complete blocks are historical
// (c(t) = t / 64 counts the blocks strictly before the query's own), so a
// block's selector key is needed from the first query after it completes,
// which is exactly when it is written.  The attention and selection over the
// pools reuse the top-K and pair-path kernels through their paged sources
// (topk.hip, sparse.hip).
#include "sas_device.h"
#include "sas_internal.h"

namespace sas {

// One workgroup per sequence.
template <typename T, typename ST>
__global__ __launch_bounds__(256) void paged_append_kernel(
    const int* __restrict__ pos, const int* __restrict__ table, const T* __restrict__ k_new,
    const T* __restrict__ v_new, const ST* __restrict__ ks_new, T* __restrict__ k_pool,
    T* __restrict__ v_pool, ST* __restrict__ ks_pool, Dims D, int pages) {
  const int b = blockIdx.x;
  const int p = pos[b];
  if (p < 0 || p >= D.nb * kBlock) return;
  const int pg = table[(size_t)b * D.nb + p / kBlock];
  if (pg < 0 || pg >= pages) return;
  const int r = p % kBlock;
  const size_t src0 = (size_t)b * D.hkv * D.d;
  for (int x = threadIdx.x; x < D.hkv * D.d; x += blockDim.x) {
    const int g = x / D.d, e = x - g * D.d;
    const size_t dst = (((size_t)pg * D.hkv + g) * kBlock + r) * D.d + e;
    k_pool[dst] = k_new[src0 + x];
    v_pool[dst] = v_new[src0 + x];
  }
  if (ks_new != nullptr && r == kBlock - 1) {
    const size_t n = (size_t)D.hks * D.ds;
    for (int x = threadIdx.x; x < (int)n; x += blockDim.x)
      ks_pool[(size_t)pg * n + x] = ks_new[(size_t)b * n + x];
  }
}

hipError_t launch_paged_append(const int* pos, const int* table, const void* k_new,
                               const void* v_new, const void* ks_new, void* k_pool, void* v_pool,
                               void* ks_pool, const Dims& D, int pages, bool is_bf16,
                               hipStream_t st) {
  if (is_bf16)
    hipLaunchKernelGGL((paged_append_kernel<bf16, bf16>), dim3(D.batch), dim3(256), 0, st, pos,
                       table, (const bf16*)k_new, (const bf16*)v_new, (const bf16*)ks_new,
                       (bf16*)k_pool, (bf16*)v_pool, (bf16*)ks_pool, D, pages);
  else
    hipLaunchKernelGGL((paged_append_kernel<float, float>), dim3(D.batch), dim3(256), 0, st, pos,
                       table, (const float*)k_new, (const float*)v_new, (const float*)ks_new,
                       (float*)k_pool, (float*)v_pool, (float*)ks_pool, D, pages);
  return hipGetLastError();
}

}  // namespace sas
