// qcal.hip -- low-rank query calibration of the retrieval query (paper-body
// page, implementation: Q-Cal; summary page, practical enhancements):
//     q_hat[b, h, t, :] = q[b, h, t, :] + W_up[h] (W_down h_t)
// with h_t the token's hidden state [dm], W_down [r, dm], W_up [Hq, d, r].
// One kernel does both low-rank products, the residual add and the single
// rounding to the stored dtype: a workgroup owns 64 tokens (16 per wave).
//   1. z = W_down h_t for the wave's 16 tokens: MFMA tiles (tokens x r) over dm,
//      operands read straight from HBM / L2 (h rows once, W_down shared by all);
//      z stays fp32.
//   2. each wave takes whole heads for the 64 tokens: (q_hat - q)^T = W_up z^T
//      with fp32 MFMA (16x16x4), so z is never rounded, W_up rows read straight
//      from L2; each lane adds its four q values, rounds once and stores them.
#include "attend_tiles.h"   // load4_add, store4
#include "hils_internal.h"

namespace hils {

namespace {

template <typename T, int D, int R>
__global__ __launch_bounds__(256) void qcal_kernel(QcalArgs a) {
  constexpr int KS = 32;          // contraction step of one fragment
  constexpr int NT = R / 16;      // r tiles of step 1
  constexpr int RG = R / 4;       // contraction elements per lane group in step 2
  constexpr int ZP = R + 4;       // padded LDS row of z (fp32 words)
  __shared__ __align__(16) float zl[64 * ZP];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r16 = lane % 16, grp = lane / 16;
  const int b = blockIdx.y;
  const int64_t T_ = a.T;
  const int64_t tb = (int64_t)blockIdx.x * 64;
  const int dm = a.dm;
  // 1. z (tokens x r) of this wave's 16 tokens: lane holds tokens 4 grp + i of
  //    column j = 16 nt + r16
  {
    const T* hg = static_cast<const T*>(a.h) + ((int64_t)b * T_ + min(tb + 16 * wave + r16, T_ - 1)) * dm;
    const T* wd = static_cast<const T*>(a.wd);
    f32x4_t zacc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) zacc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int m0 = 0; m0 < dm; m0 += KS) {
      Frag<T> ah, bw[NT];
      load_frag(ah, hg + m0 + 8 * grp);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) load_frag(bw[nt], wd + (int64_t)(16 * nt + r16) * dm + m0 + 8 * grp);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) mma(zacc[nt], ah, bw[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) zl[(16 * wave + 4 * grp + i) * ZP + 16 * nt + r16] = zacc[nt][i];
  }
  __syncthreads();
  // 2. every wave takes whole heads for all 64 tokens.  The contraction over j
  //    runs in the order j = RG grp + s (step s of the 16x16x4 products), so a
  //    lane's W_up operand is RG consecutive elements of one row and its z
  //    operand RG consecutive values of one token.
  float zr[4][RG];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int s = 0; s < RG; s += 4) {
      const float4 v = *reinterpret_cast<const float4*>(&zl[(16 * tt + r16) * ZP + RG * grp + s]);
      zr[tt][s] = v.x; zr[tt][s + 1] = v.y; zr[tt][s + 2] = v.z; zr[tt][s + 3] = v.w;
    }
  const T* wu = static_cast<const T*>(a.wu);
  for (int hd = wave; hd < a.Hq; hd += 4) {
    const int64_t rb = ((int64_t)b * a.Hq + hd) * T_;
#pragma unroll 1
    for (int md = 0; md < D / 16; ++md) {
      // W_up[hd][16 md + r16][RG grp .. RG grp + RG - 1]
      float wa[RG];
      const T* wr = wu + ((int64_t)hd * D + 16 * md + r16) * R + RG * grp;
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
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < RG; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[s], zr[tt][s], acc, 0, 0, 0);
        // acc[i]: element 16 md + 4 grp + i of token 16 tt + r16
        const int64_t tq = tb + 16 * tt + r16;
        if (tq < T_) {
          const int64_t o = (rb + tq) * D + 16 * md + 4 * grp;
          f32x4_t qv = f32x4_t{0.f, 0.f, 0.f, 0.f};
          load4_add<T>(qv, static_cast<const T*>(a.q) + o);
          store4<T>(static_cast<T*>(a.qh) + o, acc + qv, 1.f);
        }
      }
    }
  }
}

template <typename T, int D>
hipError_t launch_qcal_td(const QcalArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.T + 63) / 64), (unsigned)a.B);
  switch (a.r) {
    case 16: hipLaunchKernelGGL((qcal_kernel<T, D, 16>), grid, dim3(256), 0, st, a); break;
    case 32: hipLaunchKernelGGL((qcal_kernel<T, D, 32>), grid, dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL((qcal_kernel<T, D, 64>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((qcal_kernel<T, D, 128>), grid, dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qcal(const QcalArgs& a, hipStream_t st) {
  KTimer tm(K_QCAL, st);
  if (a.bf16) return a.D == 128 ? launch_qcal_td<bf16_t, 128>(a, st) : launch_qcal_td<bf16_t, 64>(a, st);
  return a.D == 128 ? launch_qcal_td<float, 128>(a, st) : launch_qcal_td<float, 64>(a, st);
}

}  // namespace hils
