// hils_common.h -- device helpers shared by the HiLS kernels (gfx950 / CDNA4, wave64).
//
// MFMA fragment convention (v_mfma_f32_16x16x32_bf16; for fp32 operands eight
// v_mfma_f32_16x16x4f32 steps cover the same 32-wide reduction):
//   A (16 x 32): lane l holds row l%16, reduction elements 8*(l/16) .. 8*(l/16)+7
//   B (32 x 16): lane l holds column l%16, the same 8 reduction elements
//   C (16 x 16): lane l holds column l%16, rows 4*(l/16) .. 4*(l/16)+3
// The reduction index may be permuted as long as A and B use the same order;
// the attention kernels use that to feed P straight from the score tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hils {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // bf16 storage

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Hardware 2^x and log2(x) (v_exp_f32, v_log_f32): about 1 ulp, no range handling
// beyond the instruction's own (2^-inf = 0); callers pass finite or -inf inputs.
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float bf2f(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T> __device__ __forceinline__ float to_f(T x);
template <> __device__ __forceinline__ float to_f<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t x) { return bf2f(x); }

template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float x) { return f2bf(x); }

// 8 reduction elements of one lane.
template <typename T> struct Frag;
template <> struct Frag<bf16_t> {
  bf16x8_t v;
};
template <> struct Frag<float> {
  float v[8];
};

__device__ __forceinline__ void mma(f32x4_t& c, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4_t& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], c, 0, 0, 0);
}

// Load 8 contiguous elements (16 B for bf16, 32 B for fp32); p must be 16-byte aligned.
__device__ __forceinline__ void load_frag(Frag<bf16_t>& f, const bf16_t* p) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  f.v = __builtin_bit_cast(bf16x8_t, u);
}
__device__ __forceinline__ void load_frag(Frag<float>& f, const float* p) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
// Two runs of 4 contiguous elements (8 B each for bf16, 16 B for fp32).
__device__ __forceinline__ void load_frag2x4(Frag<bf16_t>& f, const bf16_t* p0, const bf16_t* p1) {
  uint2 a = *reinterpret_cast<const uint2*>(p0);
  uint2 b = *reinterpret_cast<const uint2*>(p1);
  uint4 u = make_uint4(a.x, a.y, b.x, b.y);
  f.v = __builtin_bit_cast(bf16x8_t, u);
}
__device__ __forceinline__ void load_frag2x4(Frag<float>& f, const float* p0, const float* p1) {
  float4 a = *reinterpret_cast<const float4*>(p0);
  float4 b = *reinterpret_cast<const float4*>(p1);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
__device__ __forceinline__ void zero_frag(Frag<bf16_t>& f) {
  f.v = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
}
__device__ __forceinline__ void zero_frag(Frag<float>& f) {
#pragma unroll
  for (int s = 0; s < 8; ++s) f.v[s] = 0.f;
}
// Build a fragment from 8 floats (P tiles); bf16 rounds to nearest even.
__device__ __forceinline__ void set_frag(Frag<bf16_t>& f, const float* x) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
  f.v = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
}
__device__ __forceinline__ void set_frag(Frag<float>& f, const float* x) {
#pragma unroll
  for (int s = 0; s < 8; ++s) f.v[s] = x[s];
}

// Dot product of two contiguous D-vectors held by one lane (16-byte loads, fp32 sums).
template <typename T, int D>
__device__ __forceinline__ float dot_row(const T* a, const T* b) {
  constexpr int EPV = 16 / sizeof(T);
  float acc = 0.f;
#pragma unroll
  for (int e0 = 0; e0 < D; e0 += EPV) {
    const uint4 ua = *reinterpret_cast<const uint4*>(a + e0);
    const uint4 ub = *reinterpret_cast<const uint4*>(b + e0);
    const T* ta = reinterpret_cast<const T*>(&ua);
    const T* tb = reinterpret_cast<const T*>(&ub);
#pragma unroll
    for (int t = 0; t < EPV; ++t) acc = fmaf(to_f<T>(ta[t]), to_f<T>(tb[t]), acc);
  }
  return acc;
}

// LDS tiles of one chunk: K as [kS][D] and V^T as [D][kS], unpadded, with the
// 16-byte pieces of each row XOR-swizzled so that the 16 rows an MFMA operand
// read touches at one logical column land in distinct banks (rows of >= 256
// bytes: swizzle by row mod 16; rows of 128 bytes: by (row / 2) mod 8, since two
// consecutive rows already split the banks).
template <int PPR>
__device__ __forceinline__ int swz(int r, int p) {
  return r * PPR + (p ^ (PPR >= 16 ? (r & 15) : ((r >> 1) & 7)));
}

// Operand fragment of 8 consecutive elements (logical column col, a multiple of
// 8) of row `row` of a swizzled tile.
template <int PPR>
__device__ __forceinline__ void load_frag_swz(Frag<bf16_t>& f, const bf16_t* tile, int row, int col) {
  f.v = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(tile + swz<PPR>(row, col / 8) * 8));
}
template <int PPR>
__device__ __forceinline__ void load_frag_swz(Frag<float>& f, const float* tile, int row, int col) {
  const float4 x = *reinterpret_cast<const float4*>(tile + swz<PPR>(row, col / 4) * 4);
  const float4 y = *reinterpret_cast<const float4*>(tile + swz<PPR>(row, col / 4 + 1) * 4);
  f.v[0] = x.x; f.v[1] = x.y; f.v[2] = x.z; f.v[3] = x.w;
  f.v[4] = y.x; f.v[5] = y.y; f.v[6] = y.z; f.v[7] = y.w;
}
// Wave-wide reductions (64 lanes).
// x from lane (lane ^ M).  Masks below 16 stay inside a 16-lane row and use DPP
// moves (quad permutes for 1 and 2, a row rotation by 8 for 8, and the two row
// shifts by 4 selected by lane bit 2 for 4); wider masks use a permute.
template <int M>
__device__ __forceinline__ float xor_lane(float x) {
  const int v = __float_as_int(x);
  if constexpr (M == 1) {
    return __int_as_float(__builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  } else if constexpr (M == 2) {
    return __int_as_float(__builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  } else if constexpr (M == 4) {
    const int up = __builtin_amdgcn_update_dpp(v, v, 0x104, 0xF, 0xF, false);   // row_shl 4: from lane + 4
    const int dn = __builtin_amdgcn_update_dpp(v, v, 0x114, 0xF, 0xF, false);   // row_shr 4: from lane - 4
    return __int_as_float((threadIdx.x & 4) ? dn : up);
  } else if constexpr (M == 8) {
    return __int_as_float(__builtin_amdgcn_update_dpp(v, v, 0x128, 0xF, 0xF, false));  // row_ror 8
  } else {
    return __shfl_xor(x, M, kWave);
  }
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, xor_lane<32>(x));
  x = fmaxf(x, xor_lane<16>(x));
  x = fmaxf(x, xor_lane<8>(x));
  x = fmaxf(x, xor_lane<4>(x));
  x = fmaxf(x, xor_lane<2>(x));
  return fmaxf(x, xor_lane<1>(x));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += xor_lane<32>(x);
  x += xor_lane<16>(x);
  x += xor_lane<8>(x);
  x += xor_lane<4>(x);
  x += xor_lane<2>(x);
  return x + xor_lane<1>(x);
}
__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

// Aligned window left edge l_i = max(0, S*floor((i-W+1)/S)) and |C_i| = l_i / S.
__host__ __device__ __forceinline__ int64_t window_left(int64_t i, int S, int W) {
  int64_t a = i - (int64_t)W + 1;
  if (a <= 0) return 0;
  return (a / S) * S;
}
__host__ __device__ __forceinline__ int64_t num_candidates(int64_t i, int S, int W) {
  return window_left(i, S, W) / S;
}

// Orderable key of a float: larger float -> larger unsigned key (-0 folded to +0).
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

}  // namespace hils
