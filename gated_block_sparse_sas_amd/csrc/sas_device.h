// sas_device.h -- device-side types and helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sas {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBlock = 64;  // keys per gate block == keys per LDS tile

// Resolved problem description passed by value to every kernel.
struct Dims {
  int batch, hq, hkv, hks;
  int tq, tk, d, ds, nb, qoff;
  int hpg;   // query heads per kv head   (hq / hkv)
  int hps;   // query heads per selector head (hq / hks)
  float sm_scale, sel_scale;
};

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Selector score dot product <qs, ks> over ds elements, accumulated in fp32
// in index order with fused multiply-adds.  Every kernel that ranks or
// normalises scores uses this one routine so that they agree bit for bit.
template <int DS, typename ST>
__device__ __forceinline__ float sel_dot(const float* qsv, const ST* ksrow) {
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < DS; ++e) acc = fmaf(qsv[e], to_f32(ksrow[e]), acc);
  return acc;
}

// Query-tile scheduling for the causal kernels.  Tiles are issued longest
// first (the last query tile attends the most keys).  When the (batch, kv
// head) groups divide evenly over the 8 XCDs, linear workgroup id L runs on
// XCD L % 8 and every XCD is given whole kv groups, so the query heads of a
// group stream the same K/V tiles through one L2 at about the same time.
struct QTile {
  int b, h, qt;
};
__device__ __forceinline__ QTile map_q_tile(int L, int nqt, const Dims& D, int xcd_groups) {
  QTile r;
  if (xcd_groups > 0) {
    const int xcd = L & 7, s = L >> 3;
    const int per_rank = xcd_groups * D.hpg;
    const int qrank = s / per_rank, rem = s - qrank * per_rank;
    const int G = (rem / D.hpg) * 8 + xcd;
    r.b = G / D.hkv;
    r.h = (G % D.hkv) * D.hpg + rem % D.hpg;
    r.qt = nqt - 1 - qrank;
  } else {
    const int bh = D.batch * D.hq;
    const int qrank = L / bh, rem = L - qrank * bh;
    r.b = rem / D.hq;
    r.h = rem % D.hq;
    r.qt = nqt - 1 - qrank;
  }
  return r;
}

}  // namespace sas
