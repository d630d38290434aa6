// qcal_tile.h -- the pieces of the low-rank query calibration shared by its own
// kernel and by the scoring pass that fuses it (paper-body page, implementation:
// Q-Cal; summary page, practical enhancements):
//     q_hat = q + W_up[h] z,   z = W_down h_t   (z kept in fp32, q_hat rounded once)
// The up-projection of 16 tokens for 16 output elements is one fp32 16x16x4 MFMA
// chain over the rank.  The contraction runs in the order j = RG grp + s (step s
// of the chain), so a lane's W_up operand is RG consecutive elements of one row
// and its z operand RG consecutive values of one token; every caller uses this
// same order, so every path stores the same bits.
#pragma once

#include "hils_common.h"

namespace hils {

// W_up[hd][row][RG grp .. RG grp + RG - 1] as fp32 (W_up is [Hq, D, R]).
template <typename T, int D, int R>
__device__ __forceinline__ void qcal_wup_piece(const T* wu, int hd, int row, int grp, float (&wa)[R / 4]) {
  constexpr int RG = R / 4;
  const T* wr = wu + ((int64_t)hd * D + row) * R + RG * grp;
  if constexpr (RG * sizeof(T) >= 16) {
#pragma unroll
    for (int s = 0; s < RG; s += 16 / (int)sizeof(T)) {
      const uint4 u = *reinterpret_cast<const uint4*>(wr + s);
      const T* x = reinterpret_cast<const T*>(&u);
#pragma unroll
      for (int e = 0; e < 16 / (int)sizeof(T); ++e) wa[s + e] = to_f<T>(x[e]);
    }
  } else {   // bf16 with r = 16: four elements, 8 bytes
    const uint2 u = *reinterpret_cast<const uint2*>(wr);
    const T* x = reinterpret_cast<const T*>(&u);
#pragma unroll
    for (int e = 0; e < RG; ++e) wa[e] = to_f<T>(x[e]);
  }
}

// (q_hat - q) for 16 tokens (MFMA columns, z operand zr of token r16) and the 16
// elements 16 md .. 16 md + 15 whose W_up pieces are wa (qcal_wup_piece of row
// 16 md + r16): acc[i] = element 16 md + 4 grp + i of token r16.
template <int R>
__device__ __forceinline__ f32x4_t qcal_chain(const float (&wa)[R / 4], const float (&zr)[R / 4]) {
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < R / 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[s], zr[s], acc, 0, 0, 0);
  return acc;
}

}  // namespace hils
