// attend_tiles.h -- MFMA tile helpers shared by the attention kernels
// (forward and backward) for one 64-token chunk (gfx950, wave64).
//
// Score tiles are computed transposed, S^T = K Q^T (tokens x rows), so each lane
// holds one row's scores for 16 tokens; the same registers, cast to the operand
// type, are the B operand of O^T = V^T P^T with the reduction order of the
// token axis permuted to match (V^T rows store their tokens in that order).
#pragma once

#include "hils_common.h"

namespace hils {

constexpr int kTileS = 64;  // tokens per chunk

// Token order inside a chunk's V^T row.  The P operand of O^T += V^T P^T comes
// straight from the S^T tile, whose lane holds tokens 16*mt + 4*grp + i
// (i < 4) for mt = 2*k2 and 2*k2 + 1 in the k2-th 32-token step; storing those
// eight tokens next to each other at 32*k2 + 8*grp makes each V^T operand one
// 16-byte read.
__device__ __forceinline__ int vt_token(int pos) {
  const int k2 = pos >> 5, grp = (pos >> 3) & 3, h = (pos >> 2) & 1, i = pos & 3;
  return 16 * (2 * k2 + h) + 4 * grp + i;
}


// Stage one chunk (K rows and V^T rows, already zero past the sequence end for
// V^T) into the swizzled LDS tiles with NT threads.
template <typename T, int D, int NT>
__device__ __forceinline__ void stage_chunk(const T* kc, const T* vtc, T* ks, T* vt, int64_t nvalid) {
  constexpr int EPV = 16 / sizeof(T);
  constexpr int PK = D / EPV, PV = kTileS / EPV;
  for (int e = threadIdx.x; e < kTileS * PK; e += NT) {
    const int row = e / PK, p = e % PK;
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (row < nvalid) u = *reinterpret_cast<const uint4*>(kc + (int64_t)row * D + p * EPV);
    *reinterpret_cast<uint4*>(ks + swz<PK>(row, p) * EPV) = u;
  }
  for (int e = threadIdx.x; e < D * PV; e += NT) {
    const int row = e / PV, p = e % PV;
    *reinterpret_cast<uint4*>(vt + swz<PV>(row, p) * EPV) =
        *reinterpret_cast<const uint4*>(vtc + (int64_t)row * kTileS + p * EPV);
  }
}

// S^T tile (64 tokens x 16 rows) for one row-fragment set bq[KS]; acc[mt][i] is the
// logit of token 16*mt + 4*grp + i for row lane%16.
template <typename T, int D>
__device__ __forceinline__ void score_tile(const T* ks, const Frag<T> (&bq)[D / 32], f32x4_t (&acc)[4],
                                           int r16, int grp) {
  constexpr int PK = D / (16 / (int)sizeof(T));
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kq = 0; kq < D / 32; ++kq) {
      Frag<T> af;
      load_frag_swz<PK>(af, ks, 16 * mt + r16, 8 * grp + 32 * kq);
      mma(acc[mt], af, bq[kq]);
    }
  }
}

// O^T += V^T P^T: o[md] (dims 16*md + 4*grp + i, row lane%16), p[mt][i] as from score_tile.
template <typename T, int D>
__device__ __forceinline__ void pv_tile(const T* vt, const float (&p)[4][4], f32x4_t (&o)[D / 16],
                                        int r16, int grp) {
  constexpr int PV = kTileS / (16 / (int)sizeof(T));
  Frag<T> pf[2];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = p[2 * k2][i];
      x[4 + i] = p[2 * k2 + 1][i];
    }
    set_frag(pf[k2], x);
  }
#pragma unroll
  for (int md = 0; md < D / 16; ++md) {
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      Frag<T> af;
      load_frag_swz<PV>(af, vt, 16 * md + r16, 32 * k2 + 8 * grp);
      mma(o[md], af, pf[k2]);
    }
  }
}

template <typename T>
__device__ __forceinline__ void store4(T* p, const f32x4_t& v, float w);
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, const f32x4_t& v, float w) {
  const uint32_t lo = pack_bf16x2(v[0] * w, v[1] * w);
  const uint32_t hi = pack_bf16x2(v[2] * w, v[3] * w);
  *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const f32x4_t& v, float w) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0] * w, v[1] * w, v[2] * w, v[3] * w);
}
template <typename T>
__device__ __forceinline__ void load4_add(f32x4_t& acc, const T* p);
template <>
__device__ __forceinline__ void load4_add<bf16_t>(f32x4_t& acc, const bf16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  acc[0] += __uint_as_float(u.x << 16);
  acc[1] += __uint_as_float(u.x & 0xffff0000u);
  acc[2] += __uint_as_float(u.y << 16);
  acc[3] += __uint_as_float(u.y & 0xffff0000u);
}
template <>
__device__ __forceinline__ void load4_add<float>(f32x4_t& acc, const float* p) {
  const float4 u = *reinterpret_cast<const float4*>(p);
  acc[0] += u.x; acc[1] += u.y; acc[2] += u.z; acc[3] += u.w;
}



}  // namespace hils
