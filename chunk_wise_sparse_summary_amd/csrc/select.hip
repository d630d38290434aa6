// select.hip -- retrieval scores and GQA-aware top-k chunk selection (prefill).
//
// Paper-body page, RQ1: each query scores every chunk summary with the linear
// surrogate of Eq. 7 and keeps the top-k ("the routing cost is the only
// quadratic term").  Summary page, Eq. 10: s_hat = q_hat . k' / sqrt(d) + b'.
// Paper-body page, GQA-aware chunk selection: per-head normalised chunk weights,
// max over the heads of a group, top-k per group.  The normalised weight is
// exp(s_hat - LSE_{C_i} s_hat), so ranking by max_h (s_hat_h - L_h) is ranking by
// the max weight; for a group of one head the rank key is s_hat itself.  Ties
// go to the lower chunk index.
//
// Two kernels:
//   score_lse   (G > 1 only) L_{h,i} = LSE_{c in C_i} s_hat_{h,i,c}: an MFMA score
//               tile (16 queries x 16 chunks per wave step) with an online
//               log-sum-exp epilogue.  One workgroup = one head x 64 queries.
//   rank_select persistent workgroups, each owning a scratch slot.  For a tile of
//               64 queries x one group it recomputes the score tiles for all G
//               heads (A fragments of q_hat stay in registers), forms the rank
//               key per (query, chunk), writes it to its slot, then each wave
//               selects the top-k of its 16 queries (below) and recomputes each
//               head's s_hat on the selected chunks.
//
// Wave-level top-k of n <= 64*J keys held J per lane (candidate c = lane + 64*j):
//   total order: (key desc, chunk asc), packed as key<<32 | ~c in 64 bits;
//   1. theta = the k-th largest of the 64 per-lane maxima: a lower bound of the
//      k-th largest key (the top-k lane maxima are k distinct candidates);
//   2. if at most 64 candidates reach theta, compact them into one per lane and
//      bitonic-sort the 64-bit keys across the wave; the k-th is the threshold;
//      otherwise find the k-th largest key exactly by bisection on the key bits
//      and take ties in ascending chunk order;
//   3. select every candidate whose 64-bit key reaches the threshold and write
//      the chosen ids in ascending order with a ballot prefix scan.
#include "hils_internal.h"
#include "topk.h"

namespace hils {

namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void score_lse_kernel(const T* __restrict__ qh,
                                                        const T* __restrict__ ksum,
                                                        const float* __restrict__ bsum,
                                                        float* __restrict__ Lout, int Hq,
                                                        int64_t T_, int64_t NCs, int S, int W,
                                                        float scale) {
  constexpr int KS = D / 32;
  const int h = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t q0 = (int64_t)blockIdx.x * 64 + wave * 16;
  if (q0 >= T_) return;
  const int r16 = lane % 16, grp = lane / 16;

  Frag<T> a[KS];
  {
    const int64_t qa = min(q0 + r16, T_ - 1);
    const T* qrow = qh + (((int64_t)b * Hq + h) * T_ + qa) * D + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) load_frag(a[ks], qrow + 32 * ks);
  }
  int64_t ncq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t qi = q0 + 4 * grp + i;
    ncq[i] = qi < T_ ? num_candidates(qi, S, W) : 0;
  }
  const int64_t ncmax = num_candidates(min(q0 + 15, T_ - 1), S, W);
  const float sl2 = scale * kLog2e;
  float m[4], s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m[i] = kNegInf; s[i] = 0.f; }

  const T* kb = ksum + ((int64_t)b * Hq + h) * NCs * D + 8 * grp;
  const float* bb = bsum + ((int64_t)b * Hq + h) * NCs;
  for (int64_t c0 = 0; c0 < ncmax; c0 += 16) {
    const int64_t c = c0 + r16;
    const int64_t cl = c < ncmax ? c : ncmax - 1;
    Frag<T> bf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) load_frag(bf[ks], kb + cl * D + 32 * ks);
    const float b2 = bb[cl] * kLog2e;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) mma(acc, a[ks], bf[ks]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (c < ncq[i]) {
        const float x = fmaf(acc[i], sl2, b2);
        const float mn = fmaxf(m[i], x);
        s[i] = (m[i] == mn ? s[i] : s[i] * exp2f(m[i] - mn)) + exp2f(x - mn);
        m[i] = mn;
      }
    }
  }
  // combine the 16 lanes of each row group
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float mo = __shfl_xor(m[i], o, kWave);
      const float so = __shfl_xor(s[i], o, kWave);
      const float mn = fmaxf(m[i], mo);
      if (mn != kNegInf) {
        s[i] = (m[i] == kNegInf ? 0.f : s[i] * exp2f(m[i] - mn)) +
               (mo == kNegInf ? 0.f : so * exp2f(mo - mn));
      }
      m[i] = mn;
    }
  }
  if (r16 == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t qi = q0 + 4 * grp + i;
      if (qi < T_)
        Lout[((int64_t)b * Hq + h) * T_ + qi] = ncq[i] > 0 ? (m[i] + log2f(s[i])) * kLn2 : kNegInf;
    }
  }
}

template <typename T, int D, int G, int J>
__global__ __launch_bounds__(256) void rank_select_kernel(SelArgs a) {
  constexpr int KS = D / 32;
  __shared__ uint64_t sbuf[4][64];
  __shared__ int32_t sidx[4][64];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r16 = lane % 16, grp = lane / 16;
  const T* qh = static_cast<const T*>(a.qh);
  const T* ksum = static_cast<const T*>(a.ksum);
  const int64_t T_ = a.T, NCs = a.NCs;
  const int Hq = a.Hq, Hkv = a.Hkv, S = a.S, W = a.W, topk = a.topk;
  const int64_t nqt = (T_ + 63) / 64;
  const int64_t ntiles = (int64_t)a.B * Hkv * nqt;
  float* slot = a.scratch + (int64_t)blockIdx.x * a.slot_stride;  // [64][64*J]
  constexpr int NCP = 64 * J;

  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t qt = tile % nqt;
    const int g = (int)((tile / nqt) % Hkv);
    const int b = (int)(tile / (nqt * Hkv));
    const int64_t q0 = qt * 64 + wave * 16;

    // ---------- phase 1: rank keys of every (query, candidate) of this wave
    if (q0 < T_) {
      Frag<T> af[G][KS];
      {
        const int64_t qa = min(q0 + r16, T_ - 1);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const T* qrow = qh + (((int64_t)b * Hq + g * G + hh) * T_ + qa) * D + 8 * grp;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) load_frag(af[hh][ks], qrow + 32 * ks);
        }
      }
      int64_t ncq[4];
      float Lr[G][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t qi = q0 + 4 * grp + i;
        ncq[i] = qi < T_ ? num_candidates(qi, S, W) : 0;
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
          Lr[hh][i] = (G > 1 && qi < T_) ? a.L[((int64_t)b * Hq + g * G + hh) * T_ + qi] : 0.f;
      }
      const int64_t ncmax = num_candidates(min(q0 + 15, T_ - 1), S, W);
      for (int64_t c0 = 0; c0 < ncmax; c0 += 16) {
        const int64_t c = c0 + r16;
        const int64_t cl = c < ncmax ? c : ncmax - 1;
        float r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = kNegInf;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const int h = g * G + hh;
          const T* krow = ksum + (((int64_t)b * Hq + h) * NCs + cl) * D + 8 * grp;
          Frag<T> bf[KS];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) load_frag(bf[ks], krow + 32 * ks);
          const float bv = a.bsum[((int64_t)b * Hq + h) * NCs + cl];
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) mma(acc, af[hh][ks], bf[ks]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float sh = fmaf(acc[i], a.scale, bv);
            const float x = G > 1 ? sh - Lr[hh][i] : sh;
            r[i] = fmaxf(r[i], x);
          }
        }
        if (c < NCP) {
#pragma unroll
          for (int i = 0; i < 4; ++i) slot[(wave * 16 + 4 * grp + i) * NCP + c] = r[i];
        }
      }
    }
    __threadfence_block();
    __syncthreads();

    // ---------- phase 2: top-k per query, then each head's s_hat on the selection
    if (q0 < T_) {
      for (int qq = 0; qq < 16; ++qq) {
        const int64_t i = q0 + qq;
        if (i >= T_) break;
        const int64_t nc = num_candidates(i, S, W);
        int32_t* orow = a.idx + (((int64_t)b * Hkv + g) * T_ + i) * topk;
        int nsel;
        if (nc <= topk) {
          nsel = (int)nc;
          if (lane < topk) sidx[wave][lane] = lane < nc ? lane : -1;
        } else {
          nsel = topk;
          uint64_t keys[J];
          const float* rrow = slot + (wave * 16 + qq) * NCP;
#pragma unroll
          for (int j = 0; j < J; ++j) {
            const int64_t c = lane + 64 * j;
            keys[j] = c < nc ? full_key(order_key(rrow[c]), c) : 0ull;
          }
          const uint64_t thr = wave_kth_u64<J>(keys, topk, lane, sbuf[wave]);
          emit_ascending<J>(keys, thr, lane, sidx[wave]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int32_t cs = (lane < nsel) ? sidx[wave][lane] : -1;
        if (lane < topk) orow[lane] = cs;
        // each head's retrieval score on the selected chunks (lane = slot)
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const int h = g * G + hh;
          float v = kNegInf;
          if (cs >= 0) {
            const T* qrow = qh + (((int64_t)b * Hq + h) * T_ + i) * D;
            const T* krow = ksum + (((int64_t)b * Hq + h) * NCs + cs) * D;
            const float acc = dot_row<T, D>(qrow, krow);
            v = fmaf(acc, a.scale, a.bsum[((int64_t)b * Hq + h) * NCs + cs]);
          }
          if (lane < topk) a.ssel[(((int64_t)b * Hq + h) * T_ + i) * topk + lane] = v;
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
    __syncthreads();
  }
}

template <typename T, int D, int G>
hipError_t launch_rank(const SelArgs& a, int J, hipStream_t st) {
  dim3 grid((unsigned)a.n_slots), block(256);
  switch (J) {
    case 1: hipLaunchKernelGGL((rank_select_kernel<T, D, G, 1>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((rank_select_kernel<T, D, G, 4>), grid, block, 0, st, a); break;
    case 16: hipLaunchKernelGGL((rank_select_kernel<T, D, G, 16>), grid, block, 0, st, a); break;
    case 32: hipLaunchKernelGGL((rank_select_kernel<T, D, G, 32>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((rank_select_kernel<T, D, G, 64>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_select_t(const SelArgs& a, int J, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  if (G > 1) {
    dim3 grid((unsigned)((a.T + 63) / 64), (unsigned)a.Hq, (unsigned)a.B);
    hipLaunchKernelGGL((score_lse_kernel<T, D>), grid, dim3(256), 0, st,
                       static_cast<const T*>(a.qh), static_cast<const T*>(a.ksum), a.bsum, a.L,
                       a.Hq, a.T, a.NCs, a.S, a.W, a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  switch (G) {
    case 1: return launch_rank<T, D, 1>(a, J, st);
    case 2: return launch_rank<T, D, 2>(a, J, st);
    case 4: return launch_rank<T, D, 4>(a, J, st);
    default: return launch_rank<T, D, 8>(a, J, st);
  }
}

int pick_J(int64_t NCs) {
  const int64_t need = (NCs + 63) / 64;
  if (need <= 1) return 1;
  if (need <= 4) return 4;
  if (need <= 16) return 16;
  if (need <= 32) return 32;
  return 64;
}

}  // namespace

size_t select_workspace(int B, int Hq, int Hkv, int64_t T, int S, int* n_slots,
                        int64_t* slot_stride) {
  const int64_t NCs = T / S;
  const int J = pick_J(NCs);
  const int64_t nqt = (T + 63) / 64;
  const int64_t ntiles = (int64_t)B * Hkv * nqt;
  const int slots = (int)(ntiles < 2048 ? ntiles : 2048);
  const int64_t stride = 64 * 64 * (int64_t)J;
  if (n_slots) *n_slots = slots;
  if (slot_stride) *slot_stride = stride;
  size_t bytes = (size_t)slots * stride * sizeof(float);
  if (Hq / Hkv > 1) bytes += (size_t)B * Hq * T * sizeof(float);
  return bytes + 256;
}

hipError_t launch_select(const SelArgs& a, hipStream_t st) {
  const int J = pick_J(a.NCs);
  if (a.bf16) return a.D == 128 ? launch_select_t<bf16_t, 128>(a, J, st) : launch_select_t<bf16_t, 64>(a, J, st);
  return a.D == 128 ? launch_select_t<float, 128>(a, J, st) : launch_select_t<float, 64>(a, J, st);
}

}  // namespace hils
