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
//   score_lse   (G > 1 only) L_{h,i} = LSE_{c in C_i} s_hat_{h,i,c}: MFMA score
//               tiles with an online log-sum-exp epilogue; one workgroup = one
//               head x 256 queries, k' tiles staged once in LDS.
//   rank_select persistent workgroups, each owning a scratch slot of rank keys.
//               For 64 queries x one group it recomputes every head's score
//               tiles, forms the rank key per (query, chunk), selects the top-k of
//               each query (below) and computes each head's s_hat on the choice.
//
// Wave-level top-k of n <= 64*J rank keys held J per lane (candidate c = lane +
// 64*j; keys are order-preserving unsigned images of the fp32 rank key):
//   1. theta = the k-th largest of the 64 per-lane maxima: a lower bound of the
//      k-th largest key (the top-k lane maxima are k distinct candidates);
//   2. if at most 64 candidates reach theta, they are compacted one per lane and
//      bitonic-sorted across the wave, giving the k-th largest key K exactly;
//      otherwise K is found by bisection on the key bits;
//   3. every key above K is chosen, plus the lowest-index keys equal to K up to k,
//      and the ids are written in ascending order with ballot prefix scans.
#include "hils_internal.h"
#include "topk.h"

namespace hils {

namespace {

template <typename T> struct KPad;
template <> struct KPad<bf16_t> { static constexpr int P = 8; };
template <> struct KPad<float> { static constexpr int P = 4; };

// A tile of k' (16 chunks of NH heads, padded LDS rows) and b', fetched into
// registers by all 256 threads and committed to LDS later, so that the next
// tile's loads overlap the current tile's MFMAs.
template <typename T, int D, int NH>
struct KTile {
  static constexpr int EPV = 16 / sizeof(T);
  static constexpr int PPR = D / EPV;                 // 16-byte pieces per row
  static constexpr int KP = D + KPad<T>::P;           // padded row (elements)
  static constexpr int NPIECE = NH * 16 * PPR;
  static constexpr int NPT = (NPIECE + 255) / 256;    // pieces per thread
  uint4 reg[NPT];
  float breg;
  __device__ void fetch(const T* kg, const float* bg, int64_t NCs, int c0, int cl_last) {
#pragma unroll
    for (int t = 0; t < NPT; ++t) {
      const int p = t * 256 + threadIdx.x;
      if (p < NPIECE) {
        const int hh = p / (16 * PPR), rem = p % (16 * PPR), row = rem / PPR, pc = rem % PPR;
        const int cl = min(c0 + row, cl_last);
        reg[t] = *reinterpret_cast<const uint4*>(kg + ((int64_t)hh * NCs + cl) * D + pc * EPV);
      }
    }
    if (threadIdx.x < NH * 16) {
      const int hh = threadIdx.x / 16, row = threadIdx.x % 16;
      breg = bg[(int64_t)hh * NCs + min(c0 + row, cl_last)];
    }
  }
  __device__ void commit(T* kt, float* bt) const {
#pragma unroll
    for (int t = 0; t < NPT; ++t) {
      const int p = t * 256 + threadIdx.x;
      if (p < NPIECE) {
        const int hh = p / (16 * PPR), rem = p % (16 * PPR), row = rem / PPR, pc = rem % PPR;
        *reinterpret_cast<uint4*>(kt + (hh * 16 + row) * KP + pc * EPV) = reg[t];
      }
    }
    if (threadIdx.x < NH * 16) bt[threadIdx.x] = breg;
  }
};

// L_{h,i} = LSE_{c in C_i} s_hat_{h,i,c}.  Workgroup = one head x 256 queries; a
// wave owns 64 queries (four 16-row MFMA tiles, A fragments in registers) and
// every 16-chunk k' tile is staged once in LDS for the four waves.
template <typename T, int D>
__global__ __launch_bounds__(256) void score_lse_kernel(const T* __restrict__ qh,
                                                        const T* __restrict__ ksum,
                                                        const float* __restrict__ bsum,
                                                        float* __restrict__ Lout, int Hq,
                                                        int64_t T_, int64_t NCs, int S, int W,
                                                        float scale) {
  constexpr int KS = D / 32;
  using Tile = KTile<T, D, 1>;
  __shared__ __align__(16) T kt[16 * Tile::KP];
  __shared__ float bt[16];
  const int h = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r16 = lane % 16, grp = lane / 16;
  const int64_t qb = (int64_t)blockIdx.x * 256;
  const int64_t q0 = qb + wave * 64;
  const bool live = q0 < T_;

  Frag<T> a[4][KS];
  int ncq[4][4];
  float m[4][4], s[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int64_t qa = min(q0 + 16 * rt + r16, T_ - 1);
    const T* qrow = qh + (((int64_t)b * Hq + h) * T_ + qa) * D + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) load_frag(a[rt][ks], qrow + 32 * ks);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t qi = q0 + 16 * rt + 4 * grp + i;
      ncq[rt][i] = qi < T_ ? (int)num_candidates(qi, S, W) : 0;
      m[rt][i] = kNegInf;
      s[rt][i] = 0.f;
    }
  }
  const int nc_block = (int)num_candidates(min(qb + 255, T_ - 1), S, W);
  const int ncmin = live ? (int)num_candidates(q0, S, W) : 0;
  const int ncmax = live ? (int)num_candidates(min(q0 + 63, T_ - 1), S, W) : 0;
  const float sl2 = scale * kLog2e;
  const T* kg = ksum + ((int64_t)b * Hq + h) * NCs * D;
  const float* bg = bsum + ((int64_t)b * Hq + h) * NCs;
  const int cl_last = nc_block > 0 ? nc_block - 1 : 0;
  Tile tile;
  if (nc_block > 0) tile.fetch(kg, bg, NCs, 0, cl_last);
  for (int c0 = 0; c0 < nc_block; c0 += 16) {
    __syncthreads();
    tile.commit(kt, bt);
    __syncthreads();
    if (c0 + 16 < nc_block) tile.fetch(kg, bg, NCs, c0 + 16, cl_last);  // in flight meanwhile
    if (c0 >= ncmax) continue;
    Frag<T> bf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) load_frag(bf[ks], kt + r16 * Tile::KP + 8 * grp + 32 * ks);
    const float b2 = bt[r16] * kLog2e;
    const int c = c0 + r16;
    const bool full = c0 + 16 <= ncmin;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) mma(acc, a[rt][ks], bf[ks]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (full || c < ncq[rt][i]) {
          // the running reference m moves only when a score exceeds it by 16
          const float x = fmaf(acc[i], sl2, b2);
          if (x > m[rt][i] + 16.f) {
            s[rt][i] *= hw_exp2(m[rt][i] - x);
            m[rt][i] = x;
          }
          s[rt][i] += hw_exp2(x - m[rt][i]);
        }
      }
    }
  }
  if (!live) return;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mm = m[rt][i], ss = s[rt][i];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float mo = __shfl_xor(mm, o, kWave);
        const float so = __shfl_xor(ss, o, kWave);
        const float mn = fmaxf(mm, mo);
        if (mn != kNegInf)
          ss = (mm == kNegInf ? 0.f : ss * hw_exp2(mm - mn)) + (mo == kNegInf ? 0.f : so * hw_exp2(mo - mn));
        mm = mn;
      }
      const int64_t qi = q0 + 16 * rt + 4 * grp + i;
      if (r16 == 0 && qi < T_)
        Lout[((int64_t)b * Hq + h) * T_ + qi] = ncq[rt][i] > 0 ? (mm + log2f(ss)) * kLn2 : kNegInf;
    }
  }
}

// Rank keys, top-k and each head's s_hat on the selection, for one (b, group,
// 64-query tile) per workgroup iteration (persistent workgroups, each owning a
// scratch slot of rank keys).  Wave w handles heads w and w + 4 of the group:
//   phase 1: per 16-chunk tile (k' of all G heads staged in LDS), each head's
//            x = s_hat - L_h for the 64 queries goes to LDS, and the rank key
//            r = max over heads (r = s_hat for one head) to the scratch slot;
//   phase 2: each wave selects the top-k of 16 queries; then each head's wave
//            computes its s_hat on every chosen chunk of the 64 queries.
// Two waves per SIMD fit without spilling unless the candidate keys are wide.
template <typename T, int D, int J>
constexpr int rank_waves() { return (J <= 16 || (J == 32 && (sizeof(T) == 2 || D == 64))) ? 2 : 1; }

template <typename T, int D, int G, int J>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(rank_waves<T, D, J>(), 2)))
void rank_select_kernel(SelArgs a) {
  constexpr int KS = D / 32;
  constexpr int NCP = 64 * J;
  constexpr int HW = (G + 3) / 4;        // heads per wave
  using Tile = KTile<T, D, G>;
  __shared__ __align__(16) T kt[G * 16 * Tile::KP];
  __shared__ float bt[G * 16];
  __shared__ float xs[G][64][17];       // x = s_hat - L per head, 64 queries x 16 chunks
  __shared__ uint32_t sbuf[4][64];
  __shared__ int32_t sidx[64 * 64];      // 64 queries x up to 64 chosen ids
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r16 = lane % 16, grp = lane / 16;
  const T* qh = static_cast<const T*>(a.qh);
  const T* ksum = static_cast<const T*>(a.ksum);
  const int64_t T_ = a.T, NCs = a.NCs;
  const int Hq = a.Hq, Hkv = a.Hkv, S = a.S, W = a.W, topk = a.topk;
  const int64_t nqt = (T_ + 63) / 64;
  const int64_t ntiles = (int64_t)a.B * Hkv * nqt;
  float* slot = a.scratch + (int64_t)blockIdx.x * a.slot_stride;  // [64][NCP]

  for (int64_t tile_id = blockIdx.x; tile_id < ntiles; tile_id += gridDim.x) {
    const int64_t qt = tile_id % nqt;
    const int g = (int)((tile_id / nqt) % Hkv);
    const int b = (int)(tile_id / (nqt * Hkv));
    const int64_t qb = qt * 64;
    const T* kg = ksum + ((int64_t)b * Hq + g * G) * NCs * D;   // head g*G, chunk 0
    const float* bg = a.bsum + ((int64_t)b * Hq + g * G) * NCs;

    // this wave's heads: q_hat of the 64 queries (A operand) and L per row.  The
    // fragments are loaded again for phase 2b so they are not live across the top-k.
    Frag<T> af[HW][4][KS];
    float Lr[HW][4][4];
    auto load_a = [&](int u) {
      const int h = g * G + wave + 4 * u;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int64_t qa = min(qb + 16 * rt + r16, T_ - 1);
        const T* qrow = qh + (((int64_t)b * Hq + h) * T_ + qa) * D + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) load_frag(af[u][rt][ks], qrow + 32 * ks);
      }
    };
#pragma unroll
    for (int u = 0; u < HW; ++u) {
      const int hh = wave + 4 * u;
      if (hh < G) {
        const int h = g * G + hh;
        load_a(u);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t qi = qb + 16 * rt + 4 * grp + i;
            Lr[u][rt][i] = (G > 1 && qi < T_) ? a.L[((int64_t)b * Hq + h) * T_ + qi] : 0.f;
          }
        }
      }
    }

    // ---------- phase 1
    const int nc_block = (int)num_candidates(min(qb + 63, T_ - 1), S, W);
    const int cl_last = nc_block > 0 ? nc_block - 1 : 0;
    Tile tile;
    if (nc_block > 0) tile.fetch(kg, bg, NCs, 0, cl_last);
    for (int c0 = 0; c0 < nc_block; c0 += 16) {
      __syncthreads();
      tile.commit(kt, bt);
      __syncthreads();
      if (c0 + 16 < nc_block) tile.fetch(kg, bg, NCs, c0 + 16, cl_last);
#pragma unroll
      for (int u = 0; u < HW; ++u) {
        const int hh = wave + 4 * u;
        if (hh < G) {
          Frag<T> bf[KS];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            load_frag(bf[ks], kt + (hh * 16 + r16) * Tile::KP + 8 * grp + 32 * ks);
          const float bv = bt[hh * 16 + r16];
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) mma(acc, af[u][rt][ks], bf[ks]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              xs[hh][16 * rt + 4 * grp + i][r16] = fmaf(acc[i], a.scale, bv) - Lr[u][rt][i];
          }
        }
      }
      __syncthreads();
      // wave w: rows 16w..16w+15 of the rank keys for this tile
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * wave + 4 * grp + i;
        float r = xs[0][row][r16];
#pragma unroll
        for (int hh = 1; hh < G; ++hh) r = fmaxf(r, xs[hh][row][r16]);
        slot[row * NCP + c0 + r16] = r;
      }
    }
    __threadfence_block();
    __syncthreads();

    // ---------- phase 2a: top-k of the wave's 16 queries (rows 16w..16w+15)
    for (int qq = 0; qq < 16; ++qq) {
      const int row = 16 * wave + qq;
      const int64_t i = qb + row;
      int32_t* sel = sidx + row * 64;
      const int nc = i < T_ ? (int)num_candidates(i, S, W) : 0;
      if (nc <= topk) {
        if (lane < topk) sel[lane] = lane < nc ? lane : -1;
      } else {
        uint32_t keys[J];
        const float* rrow = slot + row * NCP;
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const int c = lane + 64 * j;
          keys[j] = c < nc ? order_key(rrow[c]) : 0u;
        }
        wave_topk_u32<J>(keys, topk, lane, sbuf[wave], sel);
      }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * topk; e += 256) {
      const int row = e / topk, t = e % topk;
      const int64_t i = qb + row;
      if (i < T_) a.idx[(((int64_t)b * Hkv + g) * T_ + i) * topk + t] = sidx[row * 64 + t];
    }
    // ---------- phase 2b: each head's s_hat on the selection.  Column tiles of 16
    // chosen slots (slot s belongs to query s / topk) against the 16-query row
    // tile(s) that own them; only the entry in the slot's own row is kept.
#pragma unroll
    for (int u = 0; u < HW; ++u) {
      const int hh = wave + 4 * u;
      if (hh >= G) continue;
      const int h = g * G + hh;
      load_a(u);
      const int nslots = 64 * topk;
      for (int t0 = 0; t0 < nslots; t0 += 16) {
        const int sl = t0 + r16;
        const int sq = sl / topk, st = sl % topk;         // this lane's column: query, slot
        const int32_t cs = sl < nslots ? sidx[sq * 64 + st] : -1;
        Frag<T> bf[KS];
        float bv = 0.f;
        if (cs >= 0) {  // pad slots read nothing: there may be no summaries at all
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            load_frag(bf[ks], kg + ((int64_t)hh * NCs + cs) * D + 8 * grp + 32 * ks);
          bv = bg[(int64_t)hh * NCs + cs];
        } else {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) zero_frag(bf[ks]);
        }
        const int rt_lo = (t0 / topk) / 16, rt_hi = (min(t0 + 15, nslots - 1) / topk) / 16;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          if (rt < rt_lo || rt > rt_hi) continue;   // uniform across the wave
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) mma(acc, af[u][rt][ks], bf[ks]);
          const int ii = sq - 16 * rt - 4 * grp;
          if (sl < nslots && ii >= 0 && ii < 4 && qb + sq < T_) {
            const float v = ii == 0 ? acc[0] : ii == 1 ? acc[1] : ii == 2 ? acc[2] : acc[3];
            a.ssel[(((int64_t)b * Hq + h) * T_ + qb + sq) * topk + st] =
                cs >= 0 ? fmaf(v, a.scale, bv) : kNegInf;
          }
        }
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
    dim3 grid((unsigned)((a.T + 255) / 256), (unsigned)a.Hq, (unsigned)a.B);
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
