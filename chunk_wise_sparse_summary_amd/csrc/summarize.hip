// summarize.hip -- landmark chunk summaries (k', b').
//
// Summary page, Methodology 1, Eq. 8: with p = softmax_j(scale * q'_c . k_j) over
// the chunk's S keys, k'_c = sum_j p_j k_j and b'_c = -sum_j p_j log p_j (the
// entropy, evaluated as LSE(s) - sum_j p_j s_j).  Paper-body page, RQ1: the
// cost is O(S*d) per chunk and the landmark token of chunk c supplies q'_c.
//
// One workgroup per (b, KV head g, chunk c): the chunk's S x d keys are read from
// HBM once (16-byte loads, coalesced) into LDS as fp32, and each wave handles one
// query head of the group, so K is streamed exactly once for all G heads.
//   logits: lane j owns key row j (padded LDS rows make the column walk
//           conflict-free); softmax and entropy are wave reductions;
//   k':     lane l owns columns l, l+64; p_j is broadcast from LDS.
#include "hils_internal.h"

namespace hils {

template <typename T, int D>
__global__ __launch_bounds__(256) void summarize_kernel(const T* __restrict__ k,
                                                        const T* __restrict__ ql,
                                                        T* __restrict__ ksum,
                                                        float* __restrict__ bsum, int Hq, int Hkv,
                                                        int64_t kT, int64_t NCs, int64_t ql_sb,
                                                        int64_t ql_sh, int64_t ql_sc, int64_t c0,
                                                        float scale, SumList list) {
  constexpr int S = 64;
  constexpr int KP = D + 1;  // padded LDS row (floats)
  __shared__ float ks[S * KP];
  __shared__ float qs[4][D];
  __shared__ float ps[4][S];

  const int G = Hq / Hkv;
  const int g = blockIdx.y;
  int64_t c;
  int b;
  if (list.n > 0) {  // decode: one (sequence, chunk) pair per block row
    b = list.b[blockIdx.x];
    c = list.c[blockIdx.x];
  } else {
    b = blockIdx.z;
    c = c0 + blockIdx.x;
  }
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;

  // Stage the chunk's keys: S*D elements, 16 B per thread per step.
  constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte vector
  const T* kc = k + (((int64_t)b * Hkv + g) * kT + c * S) * D;
#pragma unroll
  for (int base = 0; base < S * D; base += 256 * EPV) {
    const int e = base + tid * EPV;
    const uint4 u = *reinterpret_cast<const uint4*>(kc + e);
    const T* tv = reinterpret_cast<const T*>(&u);
    const int row = e / D, col = e % D;
#pragma unroll
    for (int t = 0; t < EPV; ++t) ks[row * KP + col + t] = to_f<T>(tv[t]);
  }

  for (int hb = 0; hb < G; hb += 4) {
    const int hl = hb + wave;
    const bool active = hl < G;
    const int h = g * G + hl;
    if (active) {
      const T* q = ql + b * ql_sb + h * ql_sh + c * ql_sc;
      for (int t = lane; t < D; t += kWave) qs[wave][t] = to_f<T>(q[t]);
    }
    __syncthreads();
    if (active) {
      // logits of key row `lane`
      float acc = 0.f;
      const float* kr = ks + lane * KP;
#pragma unroll 16
      for (int t = 0; t < D; ++t) acc = fmaf(qs[wave][t], kr[t], acc);
      const float s2 = acc * (scale * kLog2e);  // log2 domain
      const float m2 = wave_max(s2);
      const float e = exp2f(s2 - m2);
      const float z = wave_sum(e);
      const float p = e / z;
      const float L2 = m2 + log2f(z);
      const float ps2 = wave_sum(p * s2);
      ps[wave][lane] = p;
      if (lane == 0) bsum[((int64_t)b * Hq + h) * NCs + c] = (L2 - ps2) * kLn2;
    }
    __syncthreads();
    if (active) {
      T* out = ksum + (((int64_t)b * Hq + h) * NCs + c) * D;
#pragma unroll
      for (int t0 = 0; t0 < D; t0 += kWave) {
        const int t = t0 + lane;
        float acc = 0.f;
#pragma unroll 16
        for (int j = 0; j < S; ++j) acc = fmaf(ps[wave][j], ks[j * KP + t], acc);
        out[t] = from_f<T>(acc);
      }
    }
    __syncthreads();
  }
}

template <typename T, int D>
static hipError_t launch_summarize_t(const SumArgs& a, hipStream_t st) {
  dim3 grid = a.list.n > 0 ? dim3((unsigned)a.list.n, (unsigned)a.Hkv, 1u)
                           : dim3((unsigned)a.n_chunks, (unsigned)a.Hkv, (unsigned)a.B);
  KTimer tm(a.list.n > 0 ? K_DEC_SUMMARIZE : K_SUMMARIZE, st);
  hipLaunchKernelGGL((summarize_kernel<T, D>), grid, dim3(256), 0, st,
                     static_cast<const T*>(a.k), static_cast<const T*>(a.ql),
                     static_cast<T*>(a.ksum), a.bsum, a.Hq, a.Hkv, a.kT, a.NCs, a.ql_sb, a.ql_sh,
                     a.ql_sc, a.c0, a.scale, a.list);
  return hipGetLastError();
}

hipError_t launch_summarize(const SumArgs& a, hipStream_t st) {
  if (a.list.n <= 0 && a.n_chunks <= 0) return hipSuccess;
  if (a.bf16) return a.D == 128 ? launch_summarize_t<bf16_t, 128>(a, st) : launch_summarize_t<bf16_t, 64>(a, st);
  return a.D == 128 ? launch_summarize_t<float, 128>(a, st) : launch_summarize_t<float, 64>(a, st);
}

}  // namespace hils
