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
//      with fp32 MFMA (16x16x4, qcal_tile.h), so z is never rounded, W_up rows
//      read straight from L2; each lane adds its four q values, rounds once and
//      stores them.
// zdown_kernel runs step 1 alone and stores z (fp32), for the selection pass
// that fuses step 2 into its scoring.
#include "attend_tiles.h"   // load4_add, store4
#include "hils_internal.h"
#include "qcal_tile.h"

namespace hils {

namespace {

// z (tokens x r) of 16 tokens 16 wave .. of the workgroup's 64: lane holds
// zacc[nt][i] = z of token 16 wave + 4 grp + i, column 16 nt + r16.
template <typename T, int R>
__device__ __forceinline__ void zdown_tile(const QcalArgs& a, int b, int64_t tb, int wave, int lane,
                                           f32x4_t (&zacc)[R / 16]) {
  constexpr int KS = 32;          // contraction step of one fragment
  constexpr int NT = R / 16;      // r tiles
  const int r16 = lane % 16, grp = lane / 16;
  const int64_t T_ = a.T;
  const int dm = a.dm;
  const T* hg = static_cast<const T*>(a.h) + ((int64_t)b * T_ + min(tb + 16 * wave + r16, T_ - 1)) * dm;
  const T* wd = static_cast<const T*>(a.wd);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) zacc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4   // four steps' loads in flight: the chain is latency-bound
  for (int m0 = 0; m0 < dm; m0 += KS) {
    Frag<T> ah, bw[NT];
    load_frag(ah, hg + m0 + 8 * grp);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) load_frag(bw[nt], wd + (int64_t)(16 * nt + r16) * dm + m0 + 8 * grp);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) mma(zacc[nt], ah, bw[nt]);
  }
}

template <typename T, int D, int R>
__global__ __launch_bounds__(256) void qcal_kernel(QcalArgs a) {
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
  {
    f32x4_t zacc[NT];
    zdown_tile<T, R>(a, b, tb, wave, lane, zacc);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) zl[(16 * wave + 4 * grp + i) * ZP + 16 * nt + r16] = zacc[nt][i];
  }
  __syncthreads();
  // 2. every wave takes whole heads for all 64 tokens
  float zr[4][RG];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int s = 0; s < RG; s += 4) {
      const float4 v = *reinterpret_cast<const float4*>(&zl[(16 * tt + r16) * ZP + RG * grp + s]);
      zr[tt][s] = v.x; zr[tt][s + 1] = v.y; zr[tt][s + 2] = v.z; zr[tt][s + 3] = v.w;
    }
  for (int hd = wave; hd < a.Hq; hd += 4) {
    const int64_t rb = ((int64_t)b * a.Hq + hd) * T_;
#pragma unroll 1
    for (int md = 0; md < D / 16; ++md) {
      float wa[RG];
      qcal_wup_piece<T, D, R>(static_cast<const T*>(a.wu), hd, 16 * md + r16, grp, wa);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const f32x4_t acc = qcal_chain<R>(wa, zr[tt]);
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

// Step 1 alone: z of 64 tokens per workgroup into zout [B, T, R] (fp32).
template <typename T, int R>
__global__ __launch_bounds__(256) void zdown_kernel(QcalArgs a, float* __restrict__ zout) {
  constexpr int NT = R / 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r16 = lane % 16, grp = lane / 16;
  const int b = blockIdx.y;
  const int64_t tb = (int64_t)blockIdx.x * 64;
  f32x4_t zacc[NT];
  zdown_tile<T, R>(a, b, tb, wave, lane, zacc);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = tb + 16 * wave + 4 * grp + i;
    if (t < a.T)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) zout[((int64_t)b * a.T + t) * R + 16 * nt + r16] = zacc[nt][i];
  }
}

template <typename T>
hipError_t launch_zdown_t(const QcalArgs& a, float* z, hipStream_t st) {
  const dim3 grid((unsigned)((a.T + 63) / 64), (unsigned)a.B);
  switch (a.r) {
    case 16: hipLaunchKernelGGL((zdown_kernel<T, 16>), grid, dim3(256), 0, st, a, z); break;
    case 32: hipLaunchKernelGGL((zdown_kernel<T, 32>), grid, dim3(256), 0, st, a, z); break;
    case 64: hipLaunchKernelGGL((zdown_kernel<T, 64>), grid, dim3(256), 0, st, a, z); break;
    default: hipLaunchKernelGGL((zdown_kernel<T, 128>), grid, dim3(256), 0, st, a, z); break;
  }
  return hipGetLastError();
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

hipError_t launch_zdown(const QcalArgs& a, float* z, hipStream_t st) {
  KTimer tm(K_QCAL_ZDOWN, st);
  return a.bf16 ? launch_zdown_t<bf16_t>(a, z, st) : launch_zdown_t<float>(a, z, st);
}

hipError_t launch_qcal(const QcalArgs& a, hipStream_t st) {
  KTimer tm(K_QCAL, st);
  if (a.bf16) return a.D == 128 ? launch_qcal_td<bf16_t, 128>(a, st) : launch_qcal_td<bf16_t, 64>(a, st);
  return a.D == 128 ? launch_qcal_td<float, 128>(a, st) : launch_qcal_td<float, 64>(a, st);
}

}  // namespace hils
