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
// 64*j; keys are order-preserving unsigned images of the fp32 rank key): a
// lower bound theta from the 64 lane maxima, the exact k-th key by bitwise
// bisection with ballot counts over the few keys that reach theta, then the
// chosen ids in ascending order with ballot prefix counts (ties at the k-th key
// to the lowest ids).
#include "hils_internal.h"
#include "topk.h"

namespace hils {

namespace {

template <typename T> struct KPad;
template <> struct KPad<bf16_t> { static constexpr int P = 8; };
template <> struct KPad<float> { static constexpr int P = 4; };

// A tile of k' (16 chunks of NH heads, padded LDS rows) and b' is fetched into
// registers by all 256 threads and committed to LDS one iteration later, so the
// next tile's loads overlap the current tile's MFMAs.
template <typename T, int D, int NH>
struct KTile {
  static constexpr int EPV = 16 / sizeof(T);
  static constexpr int PPR = D / EPV;                 // 16-byte pieces per row
  static constexpr int KP = D + KPad<T>::P;           // padded row (elements)
  static constexpr int NPIECE = NH * 16 * PPR;
  static constexpr int NPT = (NPIECE + 255) / 256;    // pieces per thread
};

// The prefetched pieces live in one vector value (not an array), so that they
// stay in registers whatever the unrolling order.
template <int N> using u32v = uint32_t __attribute__((ext_vector_type(N)));

template <typename T, int D, int NH, int NPT = KTile<T, D, NH>::NPT>
__device__ __forceinline__ void tile_fetch(u32v<4 * NPT>& reg, float& breg, const T* kg,
                                           const float* bg, int64_t NCs, int c0, int cl_last) {
  using K = KTile<T, D, NH>;
#pragma unroll
  for (int t = 0; t < NPT; ++t) {
    const int p = t * 256 + threadIdx.x;
    if (K::NPIECE % 256 == 0 || p < K::NPIECE) {
      const int hh = p / (16 * K::PPR), rem = p % (16 * K::PPR), row = rem / K::PPR, pc = rem % K::PPR;
      const int cl = min(c0 + row, cl_last);
      const uint4 v = *reinterpret_cast<const uint4*>(kg + ((int64_t)hh * NCs + cl) * D + pc * K::EPV);
      reg[4 * t] = v.x; reg[4 * t + 1] = v.y; reg[4 * t + 2] = v.z; reg[4 * t + 3] = v.w;
    }
  }
  if (threadIdx.x < NH * 16) {
    const int hh = threadIdx.x / 16, row = threadIdx.x % 16;
    breg = bg[(int64_t)hh * NCs + min(c0 + row, cl_last)];
  }
}

template <typename T, int D, int NH, int NPT = KTile<T, D, NH>::NPT>
__device__ __forceinline__ void tile_commit(const u32v<4 * NPT>& reg, float breg, T* kt, float* bt) {
  using K = KTile<T, D, NH>;
#pragma unroll
  for (int t = 0; t < NPT; ++t) {
    const int p = t * 256 + threadIdx.x;
    if (K::NPIECE % 256 == 0 || p < K::NPIECE) {
      const int hh = p / (16 * K::PPR), rem = p % (16 * K::PPR), row = rem / K::PPR, pc = rem % K::PPR;
      *reinterpret_cast<uint4*>(kt + (hh * 16 + row) * K::KP + pc * K::EPV) =
          make_uint4(reg[4 * t], reg[4 * t + 1], reg[4 * t + 2], reg[4 * t + 3]);
    }
  }
  if (threadIdx.x < NH * 16) bt[threadIdx.x] = breg;
}

// Running log-sum-exp reference: finite, so that masked (-inf) scores add zero
// without inf - inf; any real score exceeds it by far more than the 16 slack.
constexpr float kRefInit = -1e30f;

// L_{h,i} = LSE_{c in C_i} s_hat_{h,i,c}.  Workgroup = one head x 256 queries; a
// wave owns 64 queries and every 16-chunk k' tile is staged once in LDS for the
// four waves.  Score tiles are transposed (rows = chunks, columns = queries), so
// each lane holds four chunks of one query and keeps one running (m, s) per
// 16-query tile.
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
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r16 = lane % 16, grp = lane / 16;
  const int64_t qb = (int64_t)blockIdx.x * 256;
  const int64_t q0 = qb + wave * 64;
  const bool live = q0 < T_;

  Frag<T> qf[4][KS];   // column r16 of query tile rt
  int ncq[4];
  float m[4], s[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int64_t qi = q0 + 16 * rt + r16;
    const T* qrow = qh + (((int64_t)b * Hq + h) * T_ + min(qi, T_ - 1)) * D + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) load_frag(qf[rt][ks], qrow + 32 * ks);
    ncq[rt] = qi < T_ ? (int)num_candidates(qi, S, W) : 0;
    m[rt] = kRefInit;
    s[rt] = 0.f;
  }
  const int nc_block = (int)num_candidates(min(qb + 255, T_ - 1), S, W);
  const int ncmin = live ? (int)num_candidates(q0, S, W) : 0;
  const int ncmax = live ? (int)num_candidates(min(q0 + 63, T_ - 1), S, W) : 0;
  const float sl2 = scale * kLog2e;
  const T* kg = ksum + ((int64_t)b * Hq + h) * NCs * D;
  const float* bg = bsum + ((int64_t)b * Hq + h) * NCs;
  const int cl_last = nc_block > 0 ? nc_block - 1 : 0;
  u32v<4 * Tile::NPT> kreg;
  float breg = 0.f;
  if (nc_block > 0) tile_fetch<T, D, 1>(kreg, breg, kg, bg, NCs, 0, cl_last);
  for (int c0 = 0; c0 < nc_block; c0 += 16) {
    __syncthreads();
    tile_commit<T, D, 1>(kreg, breg, kt, bt);
    __syncthreads();
    if (c0 + 16 < nc_block) tile_fetch<T, D, 1>(kreg, breg, kg, bg, NCs, c0 + 16, cl_last);
    if (c0 >= ncmax) continue;
    Frag<T> kf[KS];   // row r16 = chunk c0 + r16
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) load_frag(kf[ks], kt + r16 * Tile::KP + 8 * grp + 32 * ks);
    float b2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) b2[i] = bt[4 * grp + i] * kLog2e;
    f32x4_t acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) mma(acc[rt], kf[ks], qf[rt][ks]);
    }
    const bool full = c0 + 16 <= ncmin;   // every query of the wave sees all 16 chunks
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = fmaf(acc[rt][i], sl2, b2[i]);
        if (!full && c0 + 4 * grp + i >= ncq[rt]) x[i] = kNegInf;
      }
      const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      if (mx > m[rt] + 16.f) {   // the reference moves only when a score passes it by 16
        s[rt] *= hw_exp2(m[rt] - mx);
        m[rt] = mx;
      }
      s[rt] += (hw_exp2(x[0] - m[rt]) + hw_exp2(x[1] - m[rt])) +
               (hw_exp2(x[2] - m[rt]) + hw_exp2(x[3] - m[rt]));
    }
  }
  if (!live) return;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    float mm = m[rt], ss = s[rt];
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
      const float mo = __shfl_xor(mm, o, kWave);
      const float so = __shfl_xor(ss, o, kWave);
      const float mn = fmaxf(mm, mo);
      ss = ss * hw_exp2(mm - mn) + so * hw_exp2(mo - mn);
      mm = mn;
    }
    const int64_t qi = q0 + 16 * rt + r16;
    if (grp == 0 && qi < T_)
      Lout[((int64_t)b * Hq + h) * T_ + qi] = ncq[rt] > 0 ? (mm + log2f(ss)) * kLn2 : kNegInf;
  }
}

// Two waves per SIMD fit without spilling unless the candidate keys are wide.
template <typename T, int D, int J>
constexpr int rank_waves() { return (J <= 16 || (J == 32 && (sizeof(T) == 2 || D == 64))) ? 2 : 1; }

// Rank keys, top-k and each head's s_hat on the selection, for one (b, group,
// 64-query tile) per workgroup iteration (persistent workgroups, each owning a
// scratch slot of rank keys).  Wave w handles heads w and w + 4 of the group:
//   phase 1: per 16-chunk tile (k' of all G heads staged in LDS), each head's
//            x = s_hat - L_h for the 64 queries goes to LDS (transposed score
//            tiles: a lane holds four chunks of one query), and the rank key
//            r = max over heads (r = s_hat for one head) to the scratch slot;
//   phase 2: each wave selects the top-k of 16 queries; then each head's wave
//            computes its s_hat on every chosen chunk of the 64 queries.
template <typename T, int D, int G, int J>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(rank_waves<T, D, J>(), 2)))
void rank_select_kernel(SelArgs a) {
  constexpr int KS = D / 32;
  constexpr int NCP = 64 * J;
  constexpr int HW = (G + 3) / 4;        // heads per wave
  constexpr int XP = 20;                 // padded LDS row of 16 chunk values
  using Tile = KTile<T, D, G>;
  __shared__ __align__(16) T kt[G * 16 * Tile::KP];
  __shared__ float bt[G * 16];
  __shared__ __align__(16) float xs[G][64][XP];   // x = s_hat - L per head, 64 queries x 16 chunks
  __shared__ uint32_t sbuf[4][64];
  __shared__ int32_t sidx[64 * 64];      // 64 queries x up to 64 chosen ids
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r16 = lane % 16, grp = lane / 16;
  const T* qh = static_cast<const T*>(a.qh);
  const T* ksum = static_cast<const T*>(a.ksum);
  const int64_t T_ = a.T, NCs = a.NCs;
  const int Hq = a.Hq, Hkv = a.Hkv, S = a.S, W = a.W, topk = a.topk;
  const int64_t nqt = (T_ + 63) / 64;
  const int64_t ntiles = (int64_t)a.B * Hkv * nqt;
  // rank keys as order-preserving unsigned images of the fp32 values, [64][NCP]
  uint32_t* slot = reinterpret_cast<uint32_t*>(a.scratch) + (int64_t)blockIdx.x * a.slot_stride;

  for (int64_t tile_id = blockIdx.x; tile_id < ntiles; tile_id += gridDim.x) {
    const int64_t qt = tile_id % nqt;
    const int g = (int)((tile_id / nqt) % Hkv);
    const int b = (int)(tile_id / (nqt * Hkv));
    const int64_t qb = qt * 64;
    const T* kg = ksum + ((int64_t)b * Hq + g * G) * NCs * D;   // head g*G, chunk 0
    const float* bg = a.bsum + ((int64_t)b * Hq + g * G) * NCs;

    // this wave's heads: q_hat of the 64 queries (fragment r16 of tile rt = query
    // 16 rt + r16) and L of those queries.  The fragments are loaded again for
    // phase 2b so they are not live across the top-k.
    Frag<T> qf[HW][4][KS];
    float Lq[HW][4];
    auto load_q = [&](int u) {
      const int h = g * G + wave + 4 * u;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int64_t qa = min(qb + 16 * rt + r16, T_ - 1);
        const T* qrow = qh + (((int64_t)b * Hq + h) * T_ + qa) * D + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) load_frag(qf[u][rt][ks], qrow + 32 * ks);
      }
    };
#pragma unroll
    for (int u = 0; u < HW; ++u) {
      const int hh = wave + 4 * u;
      if (hh < G) {
        const int h = g * G + hh;
        load_q(u);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const int64_t qi = qb + 16 * rt + r16;
          Lq[u][rt] = (G > 1 && qi < T_) ? a.L[((int64_t)b * Hq + h) * T_ + qi] : 0.f;
        }
      }
    }

    // ---------- phase 1
    const int nc_block = (int)num_candidates(min(qb + 63, T_ - 1), S, W);
    const int cl_last = nc_block > 0 ? nc_block - 1 : 0;
    u32v<4 * Tile::NPT> kreg;
    float breg = 0.f;
    if (nc_block > 0) tile_fetch<T, D, G>(kreg, breg, kg, bg, NCs, 0, cl_last);
    for (int c0 = 0; c0 < nc_block; c0 += 16) {
      __syncthreads();
      tile_commit<T, D, G>(kreg, breg, kt, bt);
      __syncthreads();
      if (c0 + 16 < nc_block) tile_fetch<T, D, G>(kreg, breg, kg, bg, NCs, c0 + 16, cl_last);
#pragma unroll
      for (int u = 0; u < HW; ++u) {
        const int hh = wave + 4 * u;
        if (hh < G) {
          Frag<T> kf[KS];   // row r16 = chunk c0 + r16
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            load_frag(kf[ks], kt + (hh * 16 + r16) * Tile::KP + 8 * grp + 32 * ks);
          const float4 bk = *reinterpret_cast<const float4*>(bt + hh * 16 + 4 * grp);
          f32x4_t acc[4];
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) mma(acc[rt], kf[ks], qf[u][rt][ks]);
          }
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            float4 x;
            x.x = fmaf(acc[rt][0], a.scale, bk.x) - Lq[u][rt];
            x.y = fmaf(acc[rt][1], a.scale, bk.y) - Lq[u][rt];
            x.z = fmaf(acc[rt][2], a.scale, bk.z) - Lq[u][rt];
            x.w = fmaf(acc[rt][3], a.scale, bk.w) - Lq[u][rt];
            *reinterpret_cast<float4*>(&xs[hh][16 * rt + r16][4 * grp]) = x;
          }
        }
      }
      __syncthreads();
      // wave w: queries 16w + r16, chunks c0 + 4 grp .. + 3
      {
        const int row = 16 * wave + r16;
        float4 r = *reinterpret_cast<const float4*>(&xs[0][row][4 * grp]);
#pragma unroll
        for (int hh = 1; hh < G; ++hh) {
          const float4 y = *reinterpret_cast<const float4*>(&xs[hh][row][4 * grp]);
          r.x = fmaxf(r.x, y.x); r.y = fmaxf(r.y, y.y); r.z = fmaxf(r.z, y.z); r.w = fmaxf(r.w, y.w);
        }
        *reinterpret_cast<uint4*>(slot + row * NCP + c0 + 4 * grp) =
            make_uint4(order_key(r.x), order_key(r.y), order_key(r.z), order_key(r.w));
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
        const uint32_t* rrow = slot + row * NCP;
        const int jn = (nc + 63) / 64;
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const int c = lane + 64 * j;
          keys[j] = (j < jn && c < nc) ? rrow[c] : 0u;
        }
        wave_topk_u32<J>(keys, jn, topk, lane, sbuf[wave], sel);
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
      load_q(u);
      const int nslots = 64 * topk;
      const T* kh = kg + (int64_t)hh * NCs * D;
      const float* bh = bg + (int64_t)hh * NCs;
      // P column tiles are gathered together, so P gathers are in flight at once
      constexpr int P = sizeof(T) == 2 ? 4 : (D == 64 ? 2 : 1);
      for (int t00 = 0; t00 < nslots; t00 += 16 * P) {
        Frag<T> bf[P][KS];
        float bv[P];
        int32_t cs[P];
#pragma unroll
        for (int pp = 0; pp < P; ++pp) {
          const int sl = t00 + 16 * pp + r16;
          cs[pp] = sl < nslots ? sidx[(sl / topk) * 64 + sl % topk] : -1;
          if (cs[pp] >= 0) {  // pad slots read nothing: there may be no summaries at all
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
              load_frag(bf[pp][ks], kh + (int64_t)cs[pp] * D + 8 * grp + 32 * ks);
            bv[pp] = bh[cs[pp]];
          } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) zero_frag(bf[pp][ks]);
            bv[pp] = 0.f;
          }
        }
#pragma unroll
        for (int pp = 0; pp < P; ++pp) {
          const int t0 = t00 + 16 * pp;
          if (t0 >= nslots) break;   // uniform
          const int sl = t0 + r16;
          const int sq = sl / topk, st = sl % topk;       // this lane's column: query, slot
          const int rt_lo = (t0 / topk) / 16, rt_hi = (min(t0 + 15, nslots - 1) / topk) / 16;
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            if (rt < rt_lo || rt > rt_hi) continue;   // uniform across the wave
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) mma(acc, qf[u][rt][ks], bf[pp][ks]);
            const int ii = sq - 16 * rt - 4 * grp;
            if (sl < nslots && ii >= 0 && ii < 4 && qb + sq < T_) {
              const float v = ii == 0 ? acc[0] : ii == 1 ? acc[1] : ii == 2 ? acc[2] : acc[3];
              a.ssel[(((int64_t)b * Hq + h) * T_ + qb + sq) * topk + st] =
                  cs[pp] >= 0 ? fmaf(v, a.scale, bv[pp]) : kNegInf;
            }
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
  KTimer tm(K_RANK_SELECT, st);
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
    KTimer tm(K_SCORE_LSE, st);
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
