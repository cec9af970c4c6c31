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
constexpr int kBlock = 64;  // keys per LDS tile; the gate block size of the MFMA kernels

// Resolved problem description passed by value to every kernel.
struct Dims {
  int batch, hq, hkv, hks;
  int tq, tk, d, ds, nb, qoff;
  int blk;   // gate block (context unit) size: 1, 2, 4, ..., 64; nb = tk / blk
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
// 16x16x32: A lane l = row l%16, k 8(l/16)..+7; B lane l = column l%16, same k;
// D lane l = column l%16, rows 4(l/16)..+3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Row-major bf16 tiles in LDS with 256-byte rows (d = 128) use an XOR swizzle
// of the 16-byte chunks: logical chunk c of row r sits at physical chunk
// c ^ swz(r).  swz permutes the bits of r % 16 so that (a) 16 consecutive
// rows read at one logical chunk hit 16 distinct chunks (the 16-byte MFMA
// operand reads) and (b) 4 consecutive rows (aligned to 4) read at an even
// chunk pair hit 8 distinct chunks (the transposing 8-byte reads).
__device__ __forceinline__ int swz16(int r) { return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8); }
__device__ __forceinline__ int swz_off(int row, int col) {  // element offset of (row, col)
  return row * 128 + ((((col >> 3) ^ swz16(row)) << 3) | (col & 7));
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// i receives element i % 4 of the 8-byte vectors read by lanes i/4 + 4k,
// k = 0..3.  If lane 4k + a of a group points at row R0 + k, columns
// C0 + 4a .. C0 + 4a + 3, lane i ends up with column C0 + i of rows R0..R0+3.
__device__ __forceinline__ bf16x4 ds_read_tr(const bf16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(bf16x4, v);
}

// LDS layout of 128-wide bf16 tiles that are read both as 16-byte MFMA row
// operands (16 consecutive rows per instruction) and by transposing 8-byte
// reads (16 rows, 32 lanes = 8 rows per pass): rows 144 elements (72 dwords)
// apart.  Measured with SQ_LDS_BANK_CONFLICT on gfx950, this pitch gives no
// bank conflicts for either kind of read, where 68 and 76 dwords conflict on
// both.  Direct global -> LDS loads fill it 18 slots of 16 bytes per row: 16
// data slots and 2 padding slots.
__device__ __forceinline__ constexpr int trow(int r) { return 144 * r; }
// Element offset, within a row-major [rows][128] global tile, of the data the
// direct load of LDS slot s carries (padding slots reload chunk 0 of their row).
__device__ __forceinline__ unsigned tslot_src(int s) {
  const int r = s / 18, ch = s % 18;
  return (unsigned)(r * 128 + (ch < 16 ? ch : 0) * 8);
}

// Sum over each aligned group of 8 lanes, every lane of the group receiving it
// (DPP: swap neighbours, swap pairs within a quad, then mirror within 8 lanes).
__device__ __forceinline__ float sum8_dpp(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  return x;
}

// s_waitcnt vmcnt(0) (all of this wave's global loads, including the
// global-to-LDS ones, have landed); other counters untouched.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 2^x with the hardware exponential (v_exp_f32): no range reduction, so
// arguments below -126 give 0 or denormals; used on softmax exponents of at
// most 16 (the forward's running max lags the true one by less than that).
__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum / max of x over lanes l and l ^ 32 (the two 32-lane halves of a wave),
// every lane receiving it.  v_permlane32_swap trades lanes 32..63 of its first
// register with lanes 0..31 of its second; with x in both, one result holds
// the low half's x in every lane and the other the high half's, so the
// exchange needs no LDS round trip (as a lane shuffle would).  The whole wave
// must be active.
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Reductions over aligned groups of N lanes (N = 2, 4, ..., 64), every lane
// of a group receiving the result, with no LDS round trip: DPP quad
// permutes (neighbours, then pairs), DPP mirrors within 8 and within 16
// lanes (once the quads are reduced, a lane's mirror holds the other half's
// value), then the swaps of 16-lane rows and of the wave halves.  Each step
// combines a lane's value with its partner's, the same two numbers on both
// lanes, so every lane of a group ends with the same bits.  The whole wave
// must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int N, bool MAX>
__device__ __forceinline__ float group_reduce(float x) {
  static_assert(N >= 2 && N <= 64 && (N & (N - 1)) == 0, "group of 2 .. 64 lanes");
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  x = op(x, dpp_f<0xB1>(x));                         // lane ^ 1
  if constexpr (N >= 4) x = op(x, dpp_f<0x4E>(x));   // lane ^ 2
  if constexpr (N >= 8) x = op(x, dpp_f<0x141>(x));  // mirror within 8
  if constexpr (N >= 16) x = op(x, dpp_f<0x140>(x)); // mirror within 16
  if constexpr (N >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  if constexpr (N >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return x;
}
template <int N>
__device__ __forceinline__ float group_sum(float x) { return group_reduce<N, false>(x); }
template <int N>
__device__ __forceinline__ float group_max(float x) { return group_reduce<N, true>(x); }

// Sum of x over the lanes that share lane % G (G = 8, 16 or 32): lanes l ^ G,
// l ^ 2 G, ...; distance 8 by DPP row shifts (up and down by 8 within a row
// of 16), 16 and 32 by the row and half swaps.  Same bits in every lane of a
// set; the whole wave must be active.
template <int G>
__device__ __forceinline__ float stride_sum(float x) {
  static_assert(G == 8 || G == 16 || G == 32, "stride of 8, 16 or 32 lanes");
  if constexpr (G == 8) {
    const int lane = __lane_id();
    const float up = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x108, 0xF, 0xF, true));
    const float dn = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x118, 0xF, 0xF, true));
    x = (lane & 8) ? dn + x : x + up;  // (the lower lane's value first on both)
  }
  if constexpr (G <= 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Inclusive prefix sum over the lanes of a wave (lane 0 first): within each
// 16-lane row by DPP row shifts of 1, 2, 4 and 8 (a lane shifted in from
// outside the row adds 0), then the totals of the rows below (lanes 15, 31,
// 47 after the first step) read into scalars and added.  No LDS round trip;
// the whole wave must be active.
__device__ __forceinline__ unsigned wave_incl_scan(unsigned x, int lane) {
  x += (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x118, 0xF, 0xF, true);  // row_shr:8
  const unsigned t0 = (unsigned)__builtin_amdgcn_readlane((int)x, 15);
  const unsigned t1 = (unsigned)__builtin_amdgcn_readlane((int)x, 31);
  const unsigned t2 = (unsigned)__builtin_amdgcn_readlane((int)x, 47);
  const int row = lane >> 4;
  return x + (row >= 1 ? t0 : 0u) + (row >= 2 ? t1 : 0u) + (row >= 3 ? t2 : 0u);
}

// The value of lane l ^ S (S = 1, 2, ..., 32) for lane l, without an LDS
// round trip: DPP quad permutes (S = 1, 2), row shifts up and down by S
// (4, 8: the row of 16 lanes holds both), and the swaps of 16-lane rows and
// 32-lane halves (v_permlane16_swap / v_permlane32_swap with both operands x:
// one result holds the even row (lower half) of each pair, the other the odd
// one).  The whole wave must be active.
template <int S>
__device__ __forceinline__ unsigned lane_xor(unsigned x, int lane) {
  if constexpr (S == 1) {
    return (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
  } else if constexpr (S == 2) {
    return (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);
  } else if constexpr (S == 4 || S == 8) {
    const unsigned up = (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x100 + S, 0xF, 0xF, true);
    const unsigned dn = (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x110 + S, 0xF, 0xF, true);
    return (lane & S) ? dn : up;  // lane + S below, lane - S above
  } else if constexpr (S == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16) ? r[0] : r[1];
  } else {
    static_assert(S == 32, "lane distance");
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
}
template <int S>
__device__ __forceinline__ unsigned long long lane_xor_u64(unsigned long long v, int lane) {
  const unsigned lo = lane_xor<S>((unsigned)v, lane), hi = lane_xor<S>((unsigned)(v >> 32), lane);
  return ((unsigned long long)hi << 32) | lo;
}

// Whole-wave max / sum, every lane receiving it (group_reduce over 64 lanes).
__device__ __forceinline__ float wave_max(float x) { return group_max<64>(x); }
__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }

// Selector score dot product <qs, ks> over ds elements, accumulated in fp32
// in index order with fused multiply-adds.
template <int DS, typename ST>
__device__ __forceinline__ float sel_dot(const float* qsv, const ST* ksrow) {
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < DS; ++e) acc = fmaf(qsv[e], to_f32(ksrow[e]), acc);
  return acc;
}

// A query's selector row held in registers for scoring many ks rows: bf16
// rows as bf16 pairs, scored with packed bf16 dot products (each pair of
// products exact, the chain summed in fp32 in index order); f32 rows with
// sel_dot.  The row-wise selection kernels (the wave-per-row top-K and the
// fused decode) and the fp32 paths score with it; the matrix-core kernels
// (the bf16 gate normaliser, threshold selection and tiled top-K) sum the
// same exact bf16 products on MFMA in an order of their own, so their fp32
// scores may differ from these in the last bits.
template <int DS, typename ST>
struct SelQ {
  float v[DS];
  __device__ __forceinline__ void load(const ST* p) {
#pragma unroll
    for (int e = 0; e < DS; ++e) v[e] = to_f32(p[e]);
  }
  __device__ __forceinline__ float dot(const ST* kr) const { return sel_dot<DS>(v, kr); }
};
template <int DS>
struct SelQ<DS, bf16> {
  typedef __bf16 pair_t __attribute__((ext_vector_type(2)));
  pair_t v[DS / 2];
  __device__ __forceinline__ void load(const bf16* p) {
#pragma unroll
    for (int e = 0; e < DS / 2; ++e) v[e] = *(const pair_t*)(p + 2 * e);
  }
  __device__ __forceinline__ float dot(const bf16* kr) const {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < DS / 2; ++e)
      acc = __builtin_amdgcn_fdot2_f32_bf16(v[e], *(const pair_t*)(kr + 2 * e), acc, false);
    return acc;
  }
};

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
