// summarize.hip -- landmark chunk summaries (k', b').
//
// Summary page, Methodology 1, Eq. 8: with p = softmax_j(scale * q'_c . k_j) over
// the chunk's S keys, k'_c = sum_j p_j k_j and b'_c = -sum_j p_j log p_j (the
// entropy, evaluated as LSE(s) - sum_j p_j s_j).  Paper-body page, RQ1: the
// cost is O(S*d) per chunk and the landmark token of chunk c supplies q'_c.
//
// One wave per (b, KV head g, chunk c), all G query heads of the group at once,
// so every key of the chunk leaves HBM once, with whole-wave contiguous loads:
// PPR lanes cover one key row with 16-byte pieces, so one load instruction reads
// RPI = 64 / PPR consecutive rows, and lane (grp, p) holds piece p of rows
// grp + RPI*i (i < PPR).  Nothing is staged in LDS but the probabilities.
//   logits  per head, each lane's partial dot products with the matching piece
//           of q'_h (packed bf16 dot products with fp32 accumulation, or fp32
//           FMAs), then a reduce-scatter over the PPR lanes of a row group leaves
//           lane (grp, p) with the logit of row grp + RPI*p;
//   softmax per head over the 64 lanes with DPP wave reductions; p to LDS;
//   k'      each lane sums p_r,h k_r over its PPR rows for the elements of its
//           piece and every head, and a reduce-scatter over the RPI row groups
//           leaves lane (grp, p) with a run of (head, element) sums to store.
// Four waves per workgroup work on four consecutive chunks.
#include "hils_internal.h"
#include "topk.h"   // wave_lds_sync

namespace hils {

namespace {

constexpr int kSumWaves = 4;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// One reduce-scatter step over lane mask M on the first N entries of v: lanes
// with bit M set keep the upper half and send the lower, the others the
// reverse; each kept entry gains the partner's copy.  Steps run for masks M,
// M/2, ..., MLO, so the kept block's index is the lane's bits M .. MLO.
template <int M, int MLO, int N, int CAP>
__device__ __forceinline__ void reduce_scatter(float (&v)[CAP], int lane) {
  const bool up = (lane & M) != 0;
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    const float send = up ? v[k] : v[k + N / 2];
    const float keep = up ? v[k + N / 2] : v[k];
    v[k] = keep + xor_lane<M>(send);
  }
  if constexpr (M > MLO) reduce_scatter<M / 2, MLO, N / 2, CAP>(v, lane);
}

// n consecutive summary elements from fp32 sums (n * sizeof(T) a power of two).
template <typename T, int N>
__device__ __forceinline__ void store_run(T* dst, const float* x) {
  if constexpr (sizeof(T) == 2 && N >= 2) {
    uint32_t w[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    if constexpr (N == 8) *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    else if constexpr (N == 4) *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    else *reinterpret_cast<uint32_t*>(dst) = w[0];
  } else if constexpr (sizeof(T) == 4 && N == 4) {
    *reinterpret_cast<float4*>(dst) = make_float4(x[0], x[1], x[2], x[3]);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) dst[i] = from_f<T>(x[i]);
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(64 * kSumWaves) void summarize_kernel(SumArgs a) {
  constexpr int S = 64;
  constexpr int EPP = 16 / (int)sizeof(T);   // elements per 16-byte piece
  constexpr int PPR = D / EPP;               // pieces per row
  constexpr int RPI = kWave / PPR;           // rows per load instruction
  constexpr int NI = S / RPI;                // rows per lane (= PPR)
  constexpr int V = G * EPP;                 // k' partial sums per lane
  constexpr int VK = V / RPI;                // sums kept per lane after the reduction
  constexpr int RUN = VK < EPP ? VK : EPP;   // contiguous elements per store
  static_assert(NI == PPR && VK >= 1, "layout");
  __shared__ __align__(16) float pbuf[kSumWaves][S * G];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int p = lane % PPR, grp = lane / PPR;

  // work item of this wave: chunk c of (b, KV head g); grid (chunk groups, Hkv, B)
  const int g = blockIdx.y;
  int b;
  int64_t c;
  const int slot = blockIdx.x * kSumWaves + wave;
  if (a.list.n > 0) {   // decode: one list entry per wave
    if (slot >= a.list.n) return;
    b = __builtin_amdgcn_readfirstlane(a.list.b[slot]);
    c = __builtin_amdgcn_readfirstlane((int)a.list.c[slot]);
  } else {              // range: consecutive chunks
    if (slot >= a.n_chunks) return;
    b = blockIdx.z;
    c = a.c0 + slot;
  }

  // piece p of rows grp + RPI*i
  const T* kc = static_cast<const T*>(a.k) + (((int64_t)b * a.Hkv + g) * a.kT + c * S) * D + p * EPP;
  uint32_t kr[NI][4];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint4 u = *reinterpret_cast<const uint4*>(kc + (int64_t)(grp + RPI * i) * D);
    kr[i][0] = u.x; kr[i][1] = u.y; kr[i][2] = u.z; kr[i][3] = u.w;
  }
  // piece p of each head's landmark query
  uint32_t qp[G][4];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const T* q = static_cast<const T*>(a.ql) + b * a.ql_sb + (g * G + hh) * a.ql_sh + c * a.ql_sc + p * EPP;
    const uint4 u = *reinterpret_cast<const uint4*>(q);
    qp[hh][0] = u.x; qp[hh][1] = u.y; qp[hh][2] = u.z; qp[hh][3] = u.w;
  }

  // per head: logits (log2 domain), softmax and entropy; p to LDS
  const float sl2 = a.scale * kLog2e;
  float* pb = pbuf[wave];
  const int myrow = grp + RPI * p;   // the row whose logit this lane ends with
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float part[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if constexpr (sizeof(T) == 2)
          acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qp[hh][t]),
                                                __builtin_bit_cast(bf16x2_t, kr[i][t]), acc, false);
        else
          acc = fmaf(__uint_as_float(qp[hh][t]), __uint_as_float(kr[i][t]), acc);
      }
      part[i] = acc;
    }
    reduce_scatter<PPR / 2, 1, NI, NI>(part, lane);
    const float s2 = part[0] * sl2;
    const float m2 = wave_max(s2);
    const float e = hw_exp2(s2 - m2);
    const float z = wave_sum(e);
    const float pr = e / z;
    const float ps2 = wave_sum(pr * s2);
    pb[myrow * G + hh] = pr;
    if (lane == 0)
      a.bsum[((int64_t)b * a.Hq + g * G + hh) * a.NCs + c] = (m2 + hw_log2(z) - ps2) * kLn2;
  }
  wave_lds_sync();

  // k' partial sums over this lane's rows, v = hh * EPP + element
  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = grp + RPI * i;
    float kf[EPP];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        kf[2 * t] = __uint_as_float(kr[i][t] << 16);
        kf[2 * t + 1] = __uint_as_float(kr[i][t] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) kf[t] = __uint_as_float(kr[i][t]);
    }
    float pj[G];
    if constexpr (G % 4 == 0) {
#pragma unroll
      for (int q4 = 0; q4 < G; q4 += 4) {
        const float4 w = *reinterpret_cast<const float4*>(pb + r * G + q4);
        pj[q4] = w.x; pj[q4 + 1] = w.y; pj[q4 + 2] = w.z; pj[q4 + 3] = w.w;
      }
    } else {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) pj[hh] = pb[r * G + hh];
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < EPP; ++e) acc[hh * EPP + e] = fmaf(pj[hh], kf[e], acc[hh * EPP + e]);
  }
  reduce_scatter<kWave / 2, PPR, V, V>(acc, lane);

  // this lane keeps sums grp*VK .. grp*VK + VK - 1
#pragma unroll
  for (int u0 = 0; u0 < VK; u0 += RUN) {
    const int v0 = grp * VK + u0;
    const int hh = v0 / EPP, e0 = v0 % EPP;
    T* out = static_cast<T*>(a.ksum) + (((int64_t)b * a.Hq + g * G + hh) * a.NCs + c) * D + p * EPP + e0;
    store_run<T, RUN>(out, acc + u0);
  }
}

template <typename T, int D, int G>
hipError_t launch_g(const SumArgs& a, hipStream_t st) {
  const int64_t items = a.list.n > 0 ? a.list.n : a.n_chunks;
  const dim3 grid((unsigned)((items + kSumWaves - 1) / kSumWaves), (unsigned)a.Hkv,
                  a.list.n > 0 ? 1u : (unsigned)a.B);
  KTimer tm(a.list.n > 0 ? K_DEC_SUMMARIZE : K_SUMMARIZE, st);
  hipLaunchKernelGGL((summarize_kernel<T, D, G>), grid, dim3(64 * kSumWaves), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_t(const SumArgs& a, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_g<T, D, 1>(a, st);
    case 2: return launch_g<T, D, 2>(a, st);
    case 4: return launch_g<T, D, 4>(a, st);
    default: return launch_g<T, D, 8>(a, st);
  }
}

}  // namespace

hipError_t launch_summarize(const SumArgs& a, hipStream_t st) {
  if (a.list.n <= 0 && a.n_chunks <= 0) return hipSuccess;
  if (a.bf16) return a.D == 128 ? launch_t<bf16_t, 128>(a, st) : launch_t<bf16_t, 64>(a, st);
  return a.D == 128 ? launch_t<float, 128>(a, st) : launch_t<float, 64>(a, st);
}

}  // namespace hils
