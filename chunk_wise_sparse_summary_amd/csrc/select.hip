// select.hip -- retrieval scores and GQA-aware top-k chunk selection (prefill).
//
// Paper-body page, RQ1: a query's score for a chunk is the linear (Eq. 7)
// estimate of its log-mass from the chunk's summary, computed for every complete
// chunk before the k highest are chosen; this is the one part of the method
// whose cost grows with T^2.  Summary page, Eq. 10: s_hat = q_hat . k' /
// sqrt(d) + b'.
// Paper-body page, GQA-aware chunk selection: per-head normalised chunk weights,
// max over the heads of a group, top-k per group.  The normalised weight is
// exp(s_hat - LSE_{C_i} s_hat), so ranking by max_h (s_hat_h - L_h) is ranking by
// the max weight; for a group of one head the rank key is s_hat itself.  Ties
// go to the lower chunk index.
//
// Kernels (per (b, group) after the first):
//   score_lse   (G > 1 only) L_{h,i} = LSE_{c in C_i} s_hat_{h,i,c}: MFMA score
//               tiles with an online log-sum-exp epilogue; one workgroup = one
//               head x 256 queries, k' tiles staged once in LDS.
//   rank_keys   rank key per (query, candidate) into a scratch row per query;
//   topk_scores one wave per query: its top-k (below), then each head's s_hat
//               on the chosen chunks from the chosen k' rows.
//
// Wave-level top-k of n <= 64*J rank keys held J per lane (candidate c = lane +
// 64*j; keys are order-preserving unsigned images of the fp32 rank key): a
// lower bound theta from the 64 lane maxima, the exact k-th key by bitwise
// bisection with ballot counts over the few keys that reach theta, then the
// chosen ids in ascending order with ballot prefix counts (ties at the k-th key
// to the lowest ids).
#include "attend_tiles.h"   // score_tile (naive BSA), load4_add, store4
#include "hils_internal.h"
#include "qcal_tile.h"
#include "topk.h"

namespace hils {

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <typename T> struct KPad;
template <> struct KPad<bf16_t> { static constexpr int P = 8; };
template <> struct KPad<float> { static constexpr int P = 4; };

// A tile of k' (16 chunks of NH heads, padded LDS rows) and b' is fetched into
// registers by all 256 threads and committed to LDS one iteration later, so the
// next tile's loads overlap the current tile's MFMAs.
template <typename T, int D, int NH, int NT = 256>
struct KTile {
  static constexpr int EPV = 16 / sizeof(T);
  static constexpr int PPR = D / EPV;                 // 16-byte pieces per row
  static constexpr int KP = D + KPad<T>::P;           // padded row (elements)
  static constexpr int NPIECE = NH * 16 * PPR;
  static constexpr int NPT = (NPIECE + NT - 1) / NT;  // pieces per thread (NT threads)
};

// The prefetched pieces live in one vector value (not an array), so that they
// stay in registers whatever the unrolling order.
template <int N> using u32v = uint32_t __attribute__((ext_vector_type(N)));

template <typename T, int D, int NH, int NT = 256, int NPT = KTile<T, D, NH, NT>::NPT>
__device__ __forceinline__ void tile_fetch(u32v<4 * NPT>& reg, float& breg, const T* kg,
                                           const float* bg, int64_t NCs, int c0, int cl_last) {
  using K = KTile<T, D, NH, NT>;
#pragma unroll
  for (int t = 0; t < NPT; ++t) {
    const int p = t * NT + threadIdx.x;
    if (K::NPIECE % NT == 0 || p < K::NPIECE) {
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

template <typename T, int D, int NH, int NT = 256, int NPT = KTile<T, D, NH, NT>::NPT>
__device__ __forceinline__ void tile_commit(const u32v<4 * NPT>& reg, float breg, T* kt, float* bt) {
  using K = KTile<T, D, NH, NT>;
#pragma unroll
  for (int t = 0; t < NPT; ++t) {
    const int p = t * NT + threadIdx.x;
    if (K::NPIECE % NT == 0 || p < K::NPIECE) {
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
// With R > 0 the low-rank query calibration is fused in (paper-body page,
// implementation: Q-Cal): each wave forms its queries' q_hat = q + W_up[h] z
// (z = W_down h from zdown_kernel) with the arithmetic of the Q-Cal kernel
// (qcal_tile.h), stores it for the later passes and reads its score operands
// back from the stored (rounded) rows.  Lout = null (a group of one head needs
// no LSE) stops after that.
template <typename T, int D, int R = 0>
__global__ __launch_bounds__(256) void score_lse_kernel(const T* __restrict__ qh,
                                                        const T* __restrict__ ksum,
                                                        const float* __restrict__ bsum,
                                                        float* __restrict__ Lout, int Hq,
                                                        int64_t T_, int64_t NCs, int S, int W,
                                                        float scale, QcFuse qc) {
  constexpr int KS = D / 32;
  using Tile = KTile<T, D, 1>;
  __shared__ __align__(16) T kt[16 * Tile::KP];
  __shared__ float bt[16];
  const int h = blockIdx.x, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r16 = lane % 16, grp = lane / 16;
  // the query tiles with the most candidates first, so the last wave of blocks is short
  const int64_t qb = (int64_t)(gridDim.y - 1 - blockIdx.y) * 256;
  const int64_t q0 = qb + wave * 64;
  const bool live = q0 < T_;

  Frag<T> qf[4][KS];   // column r16 of query tile rt
  int ncq[4];
  float m[4], s[4];
  if constexpr (R > 0) {
    constexpr int RG = R / 4;
    const T* qtok = static_cast<const T*>(qc.q);
    T* qout = static_cast<T*>(qc.qh);
    float zr[4][RG];   // z of this lane's token (an MFMA column) in each query tile
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const float* zp = qc.z + ((int64_t)b * T_ + min(q0 + 16 * rt + r16, T_ - 1)) * R + RG * grp;
#pragma unroll
      for (int e = 0; e < RG; e += 4) {
        const float4 v = *reinterpret_cast<const float4*>(zp + e);
        zr[rt][e] = v.x; zr[rt][e + 1] = v.y; zr[rt][e + 2] = v.z; zr[rt][e + 3] = v.w;
      }
    }
    // one W_up piece per 16 elements serves the four tiles: four independent chains
#pragma unroll 1
    for (int md = 0; md < D / 16; ++md) {
      float wa[RG];
      qcal_wup_piece<T, D, R>(static_cast<const T*>(qc.wu), h, 16 * md + r16, grp, wa);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const f32x4_t acc = qcal_chain<R>(wa, zr[rt]);   // elements 16 md + 4 grp + i
        const int64_t qi = q0 + 16 * rt + r16;
        const int64_t o = (((int64_t)b * Hq + h) * T_ + min(qi, T_ - 1)) * D + 16 * md + 4 * grp;
        f32x4_t val = f32x4_t{0.f, 0.f, 0.f, 0.f};
        load4_add<T>(val, qtok + o);
        val += acc;
        if (qi < T_) store4<T>(qout + o, val, 1.f);
      }
    }
    // the wave reads back the rows it has just stored (other lanes' stores):
    // workgroup-scope release and acquire make them visible
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int64_t qi = q0 + 16 * rt + r16;
      // a column past T reads a row it did not store; its scores are never kept
      const T* qrow = qout + (((int64_t)b * Hq + h) * T_ + min(qi, T_ - 1)) * D + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) load_frag(qf[rt][ks], qrow + 32 * ks);
      ncq[rt] = qi < T_ ? (int)num_candidates(qi, S, W) : 0;
      m[rt] = kRefInit;
      s[rt] = 0.f;
    }
    if (Lout == nullptr) return;   // uniform over the workgroup
  } else {
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
    float x[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[rt][i] = fmaf(acc[rt][i], sl2, b2[i]);
    if (c0 + 16 > ncmin) {   // some query of the wave does not see all 16 chunks
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (c0 + 4 * grp + i >= ncq[rt]) x[rt][i] = kNegInf;
    }
    // The reference moves only when a score passes it by 16, which after the
    // first tiles is rare: the check is one wave vote, the rescale a branch.
    float mx[4];
    bool move = false;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      mx[rt] = fmaxf(fmaxf(x[rt][0], x[rt][1]), fmaxf(x[rt][2], x[rt][3]));
      move |= mx[rt] > m[rt] + 16.f;
    }
    if (__any(move)) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        if (mx[rt] > m[rt] + 16.f) {
          s[rt] *= hw_exp2(m[rt] - mx[rt]);
          m[rt] = mx[rt];
        }
      }
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
      s[rt] += (hw_exp2(x[rt][0] - m[rt]) + hw_exp2(x[rt][1] - m[rt])) +
               (hw_exp2(x[rt][2] - m[rt]) + hw_exp2(x[rt][3] - m[rt]));
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

// Workgroup of the rank pass: 4 waves, each with two 16-query tiles, so every
// k' fragment read from LDS feeds two MFMAs (with one tile per wave the LDS
// reads of the fragments bounded the kernel).
// (two tiles when their q fragments fit half the registers: bf16 and G d <= 512)
constexpr int kRankWaves = 4;
template <typename T, int D, int G> constexpr int rank_tq() { return sizeof(T) == 2 && G * D <= 512 ? 2 : 1; }
template <typename T, int D, int G> constexpr int rank_q() { return kRankWaves * 16 * rank_tq<T, D, G>(); }

// The prefill selection runs as two kernels over every (b, group) of a pass
// (the grids' second dimension), each group's rank keys in its own [T][64 J]
// scratch:
//   rank_keys  per 64- or 128-query tile and 16-chunk k' tile (k' of all G heads
//              staged once in LDS): wave w owns one or two 16-query MFMA column
//              tiles and every head of the group, so the rank
//              key r = max over heads of s_hat - L_h (r = s_hat for one head)
//              forms in registers (transposed score tiles: a lane holds four
//              chunks of one query) and goes straight to the scratch.
//   topk_scores one wave per query: the exact top-k of its rank keys (below)
//              and each head's s_hat on the chosen chunks.
template <typename T, int D, int G, int RQ_ = rank_q<T, D, G>()>
struct RankTiles {
  static constexpr int KS = D / 32;
  static constexpr int RQ = RQ_, NT = kRankWaves * kWave;
  using Tile = KTile<T, D, G, NT>;
};

template <typename T, int D, int G, int NCP>
__global__ __launch_bounds__(kRankWaves * kWave) void rank_keys_kernel(SelArgs a, int bg0,
                                                                       uint32_t* __restrict__ keys) {
  // (b, group) bg0 + blockIdx.y of this launch's groups, each with its own keys
  const int b = (bg0 + (int)blockIdx.y) / a.Hkv, g = (bg0 + (int)blockIdx.y) % a.Hkv;
  keys += (int64_t)blockIdx.y * a.group_words;
  using R = RankTiles<T, D, G>;
  constexpr int KS = R::KS, RQ = R::RQ, NT = R::NT;
  using Tile = typename R::Tile;
  constexpr int NW = kRankWaves, TQ = rank_tq<T, D, G>();
  constexpr int KSP = 64 + 4;        // padded staging row (words)
  __shared__ __align__(16) T kt[G * 16 * Tile::KP];
  __shared__ float bt[G * 16];
  // each wave's rank keys of 64 candidates x 16 TQ queries, written back to HBM as
  // row-contiguous 256-byte runs (one lane per query row and 16-byte piece, as
  // the score tiles leave them, costs a cache line per lane)
  __shared__ __align__(16) uint32_t kst[NW][16 * TQ * KSP];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r16 = lane % 16, grp = lane / 16;
  const T* qh = static_cast<const T*>(a.qh);
  const int64_t T_ = a.T, NCs = a.NCs;
  const int Hq = a.Hq;
  const int64_t qb = (int64_t)(gridDim.x - 1 - blockIdx.x) * RQ;   // longest rows first
  const int64_t qw0 = qb + 16 * TQ * wave;   // the wave's first query
  const T* kg = static_cast<const T*>(a.ksum) + ((int64_t)b * Hq + g * G) * NCs * D;
  const float* bg = a.bsum + ((int64_t)b * Hq + g * G) * NCs;
  Frag<T> qf[TQ][G][KS];   // column r16 of tile t: query qw0 + 16 t + r16
  float Lq[TQ][G];
#pragma unroll
  for (int t = 0; t < TQ; ++t) {
    const int64_t qi = qw0 + 16 * t + r16;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const int h = g * G + hh;
      const T* qrow = qh + (((int64_t)b * Hq + h) * T_ + min(qi, T_ - 1)) * D + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) load_frag(qf[t][hh][ks], qrow + 32 * ks);
      Lq[t][hh] = (G > 1 && qi < T_) ? a.L[((int64_t)b * Hq + h) * T_ + qi] : 0.f;
    }
  }
  const int nc_block = (int)num_candidates(min(qb + RQ - 1, T_ - 1), a.S, a.W);
  const int nc_wave = (int)num_candidates(min(qw0 + 16 * TQ - 1, T_ - 1), a.S, a.W);
  const int cl_last = nc_block > 0 ? nc_block - 1 : 0;
  u32v<4 * Tile::NPT> kreg;
  float breg = 0.f;
  if (nc_block > 0) tile_fetch<T, D, G, NT>(kreg, breg, kg, bg, NCs, 0, cl_last);
  for (int c0 = 0; c0 < nc_block; c0 += 16) {
    __syncthreads();
    tile_commit<T, D, G, NT>(kreg, breg, kt, bt);
    __syncthreads();
    if (c0 + 16 < nc_block) tile_fetch<T, D, G, NT>(kreg, breg, kg, bg, NCs, c0 + 16, cl_last);
    if (c0 >= nc_wave) continue;   // no query of this wave has these candidates
    float r[TQ][4];
#pragma unroll
    for (int t = 0; t < TQ; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) r[t][i] = kNegInf;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      Frag<T> kf[KS];   // row r16 = chunk c0 + r16
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        load_frag(kf[ks], kt + (hh * 16 + r16) * Tile::KP + 8 * grp + 32 * ks);
      const float4 bk = *reinterpret_cast<const float4*>(bt + hh * 16 + 4 * grp);
#pragma unroll
      for (int t = 0; t < TQ; ++t) {
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) mma(acc, kf[ks], qf[t][hh][ks]);
        r[t][0] = fmaxf(r[t][0], fmaf(acc[0], a.scale, bk.x) - Lq[t][hh]);
        r[t][1] = fmaxf(r[t][1], fmaf(acc[1], a.scale, bk.y) - Lq[t][hh]);
        r[t][2] = fmaxf(r[t][2], fmaf(acc[2], a.scale, bk.z) - Lq[t][hh]);
        r[t][3] = fmaxf(r[t][3], fmaf(acc[3], a.scale, bk.w) - Lq[t][hh]);
      }
    }
    uint32_t* kw = kst[wave];
#pragma unroll
    for (int t = 0; t < TQ; ++t)
      *reinterpret_cast<uint4*>(kw + (16 * t + r16) * KSP + c0 % 64 + 4 * grp) =
          make_uint4(order_key(r[t][0]), order_key(r[t][1]), order_key(r[t][2]), order_key(r[t][3]));
    if (c0 % 64 == 48 || c0 + 16 >= nc_wave) {   // a run of 64 candidates, or the wave's last
      wave_lds_sync();
      const int64_t off = qw0 * NCP + (c0 - c0 % 64) + 4 * (lane % 16);
      const int qr = lane / 16;
#pragma unroll
      for (int j = 0; j < 4 * TQ; ++j) {
        const int qq = 4 * j + qr;
        if (qw0 + qq < T_)
          __builtin_nontemporal_store(*reinterpret_cast<const u32v<4>*>(kw + qq * KSP + 4 * (lane % 16)),
                                      reinterpret_cast<u32v<4>*>(keys + off + (int64_t)qq * NCP));
      }
      wave_lds_sync();
    }
  }
}

// One reduce-scatter step over lane mask M on the first N entries of v: lanes
// with bit M set keep the upper half and send the lower, the others the
// reverse; each kept entry gains the partner's copy.  Steps run for masks M,
// M/2, ..., 1, so the kept entry's index is the lane's low bits.
template <int M, int N, int CAP>
__device__ __forceinline__ void rs_rows(float (&v)[CAP], int lane) {
  const bool up = (lane & M) != 0;
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    const float send = up ? v[k] : v[k + N / 2];
    const float keep = up ? v[k + N / 2] : v[k];
    v[k] = keep + xor_lane<M>(send);
  }
  if constexpr (M > 1) rs_rows<M / 2, N / 2, CAP>(v, lane);
}

// One wave per query of one (b, group): the exact top-k of its rank keys, then
// each head's s_hat on the chosen chunks.  The chosen (slot, head) rows of k'
// (the group's k' is a few MB, resident in L2) are read 64 at a time with
// whole-wave contiguous loads, PPR lanes per row; each lane takes the packed
// dot products (fp32 accumulation) of its 16-byte pieces with the matching
// piece of its row's q_hat, and a reduce-scatter over the PPR lanes of a row
// group leaves one row's s_hat per lane.
// The kernel waits on its loads (the rank-key row, then the chosen k' rows) and
// issues many vector instructions per query, so it keeps six waves per SIMD:
// at most 80 VGPRs for bf16 up to 2048 candidates (eight waves at 64 VGPRs
// measured 2% slower).
template <typename T, int D, int G, int J>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(J <= 32 && sizeof(T) == 2 ? 6 : 1)))
void topk_scores_kernel(SelArgs a, int bg0, const uint32_t* __restrict__ keys) {
  const int b = (bg0 + (int)blockIdx.y) / a.Hkv, g = (bg0 + (int)blockIdx.y) % a.Hkv;
  keys += (int64_t)blockIdx.y * a.group_words;
  constexpr int EPP = 16 / (int)sizeof(T);   // elements per 16-byte piece
  constexpr int PPR = D / EPP;               // pieces per row
  constexpr int RPI = kWave / PPR;           // rows per load instruction
  constexpr int NQ = G > RPI ? G / RPI : 1;  // q_hat pieces per lane
  __shared__ uint32_t sbuf[4][64];
  __shared__ int32_t sel[4][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int64_t i = (int64_t)(gridDim.x - 1 - blockIdx.x) * 4 + wave;   // longest rows first
  if (i >= a.T) return;
  const int topk = a.topk;
  const int nc = (int)num_candidates(i, a.S, a.W);
  const int64_t T_ = a.T, NCs = a.NCs;
  const int Hq = a.Hq;
  const int p = lane % PPR, grp = lane / PPR;
  // q_hat pieces: row r = slot*G + head has head r % G = (grp + RPI t) % G
  uint32_t qp[NQ][4];
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    const int hh = (grp + RPI * u) % G;
    const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.qh) +
                                                   (((int64_t)b * Hq + g * G + hh) * T_ + i) * D + p * EPP);
    qp[u][0] = q.x; qp[u][1] = q.y; qp[u][2] = q.z; qp[u][3] = q.w;
  }
  int nsel;
  if (nc <= topk) {
    if (lane < topk) sel[wave][lane] = lane < nc ? lane : -1;
    nsel = nc;
  } else if constexpr (J <= 64) {
    const uint32_t* rrow = keys + i * (64 * J);
    const int jn = (nc + 63) / 64;
    uint32_t kv[J];
#pragma unroll
    // the row holds 64 J keys: the loads need no guard, only their values do
    // (masked once every load is out)
    for (int j = 0; j < J; ++j) kv[j] = j < jn ? __builtin_nontemporal_load(rrow + lane + 64 * j) : 0u;
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (lane + 64 * j >= nc) kv[j] = 0u;
    wave_topk_u32<J>(kv, jn, topk, lane, sbuf[wave], sel[wave]);
    nsel = topk;
  } else {
    // more keys than a lane holds: the top-k of each half (64 J/2 candidates),
    // then the top-k of the two lists, kept in candidate order (so equal keys
    // still go to the lower chunk)
    constexpr int JH = J / 2;
    __shared__ uint32_t hkey[4][64], mkey[4][128];
    __shared__ int32_t hpos[4][64], mid[4][128];
    const uint32_t* rrow = keys + i * (64 * J);
    int n2 = 0;
    auto half = [&](const int base) {   // candidates [base, base + 64 JH)
      const int nch = min(nc - base, 64 * JH);
      const int jn = (nch + 63) / 64;
      uint32_t kv[JH];
#pragma unroll
      for (int j = 0; j < JH; ++j) {
        const int c = lane + 64 * j;
        kv[j] = (j < jn && c < nch) ? __builtin_nontemporal_load(rrow + base + c) : 0u;
      }
      int n = nch;
      if (nch > topk) {
        wave_topk_u32<JH>(kv, jn, topk, lane, sbuf[wave], hpos[wave], hkey[wave]);
        n = topk;
      } else if (lane < nch) {   // a short half: every candidate (one per lane)
        hpos[wave][lane] = lane;
        hkey[wave][lane] = kv[0];
      }
      wave_lds_sync();
      if (lane < n) {
        mkey[wave][n2 + lane] = hkey[wave][lane];
        mid[wave][n2 + lane] = base + hpos[wave][lane];
      }
      n2 += n;
      wave_lds_sync();
    };
    half(0);
    if (nc > 64 * JH) half(64 * JH);
    uint32_t k2[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) k2[j] = lane + 64 * j < n2 ? mkey[wave][lane + 64 * j] : 0u;
    const int n = list_topk<2>(k2, (n2 + 63) / 64, n2, topk, lane, sbuf[wave], hpos[wave], hkey[wave]);
    wave_lds_sync();
    if (lane < topk) sel[wave][lane] = lane < n ? mid[wave][hpos[wave][lane]] : -1;
    nsel = topk;
  }
  wave_lds_sync();
  if (lane < topk) a.idx[(((int64_t)b * a.Hkv + g) * T_ + i) * topk + lane] = sel[wave][lane];
  if (a.ssel == nullptr) return;   // selection only (naive BSA)
  // 64 rows per batch: lane (grp, p) loads piece p of rows r0 + grp + RPI t.
  // Every row's chunk id first; then the row loads go out NB at a time with no
  // condition (a padding row reads row 0 of its head and is dropped by a
  // select), so they are in flight together rather than one after another.
  constexpr int NB = 4;
  const T* kbase = static_cast<const T*>(a.ksum) + ((int64_t)b * Hq + g * G) * NCs * D + p * EPP;
  for (int r0 = 0; r0 < topk * G; r0 += kWave) {
    int cs[PPR];
#pragma unroll
    for (int t = 0; t < PPR; ++t) {
      const int slot = (r0 + grp + RPI * t) / G;
      cs[t] = slot < nsel ? sel[wave][min(slot, kWave - 1)] : -1;
    }
    float part[PPR];
#pragma unroll
    for (int t = 0; t < PPR; ++t) part[t] = 0.f;
    if (nsel > 0) {   // uniform: with no chunk k' may be empty
#pragma unroll
      for (int t0 = 0; t0 < PPR; t0 += NB) {
        uint4 ku[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int hh = (r0 + grp + RPI * (t0 + u)) % G;
          ku[u] = *reinterpret_cast<const uint4*>(kbase + ((int64_t)hh * NCs + max(cs[t0 + u], 0)) * D);
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const uint32_t kw[4] = {ku[u].x, ku[u].y, ku[u].z, ku[u].w};
          const int q = NQ > 1 ? (t0 + u) % NQ : 0;
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (sizeof(T) == 2)
              acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qp[q][e]),
                                                    __builtin_bit_cast(bf16x2_t, kw[e]), acc, false);
            else
              acc = fmaf(__uint_as_float(qp[q][e]), __uint_as_float(kw[e]), acc);
          }
          part[t0 + u] = cs[t0 + u] >= 0 ? acc : 0.f;
        }
      }
    }
    rs_rows<PPR / 2, PPR, PPR>(part, lane);
    const int r = r0 + grp + RPI * p, slot = r / G, hh = r % G;   // the row this lane now holds
    if (slot < topk) {
      const int h = g * G + hh;
      float sh = kNegInf;
      if (slot < nsel) sh = fmaf(part[0], a.scale, a.bsum[((int64_t)b * Hq + h) * NCs + sel[wave][slot]]);
      a.ssel[(((int64_t)b * Hq + h) * T_ + i) * topk + slot] = sh;
    }
  }
}

template <typename T, int D, int G, int J>
hipError_t launch_rank_j(const SelArgs& a, hipStream_t st) {
  constexpr int RQ = rank_q<T, D, G>();
  const dim3 tiles((unsigned)((a.T + RQ - 1) / RQ)), rows((unsigned)((a.T + 3) / 4));
  uint32_t* keys = reinterpret_cast<uint32_t*>(a.scratch);
  // as many (b, group) pairs per launch as the workspace holds rank keys for
  const int nbg = a.B * a.Hkv;
  for (int bg0 = 0; bg0 < nbg; bg0 += a.gpass) {
    const int n = min(a.gpass, nbg - bg0);
    {
      KTimer tm(K_RANK_KEYS, st);
      hipLaunchKernelGGL((rank_keys_kernel<T, D, G, 64 * J>), dim3(tiles.x, (unsigned)n), dim3(kRankWaves * kWave), 0, st,
                         a, bg0, keys);
    }
    KTimer tm(K_TOPK_SCORES, st);
    hipLaunchKernelGGL((topk_scores_kernel<T, D, G, J>), dim3(rows.x, (unsigned)n), dim3(256), 0, st, a, bg0, keys);
  }
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t launch_rank(const SelArgs& a, int J, hipStream_t st) {
  switch (J) {
    case 1: return launch_rank_j<T, D, G, 1>(a, st);
    case 4: return launch_rank_j<T, D, G, 4>(a, st);
    case 16: return launch_rank_j<T, D, G, 16>(a, st);
    case 32: return launch_rank_j<T, D, G, 32>(a, st);
    case 64: return launch_rank_j<T, D, G, 64>(a, st);
    default: return launch_rank_j<T, D, G, 128>(a, st);
  }
}

template <typename T, int D, int R>
void launch_score_lse_r(const SelArgs& a, float* L, hipStream_t st) {
  const dim3 grid((unsigned)a.Hq, (unsigned)((a.T + 255) / 256), (unsigned)a.B);
  hipLaunchKernelGGL((score_lse_kernel<T, D, R>), grid, dim3(256), 0, st, static_cast<const T*>(a.qh),
                     static_cast<const T*>(a.ksum), a.bsum, L, a.Hq, a.T, a.NCs, a.S, a.W, a.scale, a.qc);
}

template <typename T, int D>
hipError_t launch_select_t(const SelArgs& a, int J, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  if (G > 1 || a.qc_r > 0) {   // with Q-Cal fused, the first pass also forms q_hat
    float* L = G > 1 ? a.L : nullptr;
    KTimer tm(K_SCORE_LSE, st);
    switch (a.qc_r) {
      case 0: launch_score_lse_r<T, D, 0>(a, L, st); break;
      case 16: launch_score_lse_r<T, D, 16>(a, L, st); break;
      case 32: launch_score_lse_r<T, D, 32>(a, L, st); break;
      case 64: launch_score_lse_r<T, D, 64>(a, L, st); break;
      default: launch_score_lse_r<T, D, 128>(a, L, st); break;
    }
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

// ---------------------------------------------------------------- naive BSA
// Exact chunk masses (paper-body page, Block Sparse Attention preliminaries):
// log Z_{h,i,c} = LSE over the chunk's 64 tokens of scale q_{h,i} . k_j, for
// every candidate c of every query, from MFMA score tiles of the chunk's keys
// (staged once per workgroup in LDS) against 16-row query tiles (16/G queries x
// G heads, TPW tiles per wave).  For G > 1 a first sweep over the chunks forms
// each head's L_{h,i} = LSE_c log Z_{h,i,c}, the second the rank keys
// max_h (log Z - L); a group of one head ranks by log Z.  Keys go to the same
// per-query rows as the retrieval rank keys (16-chunk runs staged in LDS), and
// the same wave top-k picks the selection.  Cost: every token logit left of the
// window, twice for G > 1; a diagnostic, not part of the path.
template <typename T> constexpr int bsa_tpw() { return sizeof(T) == 2 ? 4 : 2; }

template <typename T, int D, int G, int NCP>
__global__ __launch_bounds__(256) void bsa_keys_kernel(SelArgs a, int bg0, uint32_t* __restrict__ keys) {
  const int b = (bg0 + (int)blockIdx.y) / a.Hkv, g = (bg0 + (int)blockIdx.y) % a.Hkv;
  keys += (int64_t)blockIdx.y * a.group_words;
  constexpr int TPW = bsa_tpw<T>();
  constexpr int KS = D / 32, EPV = 16 / (int)sizeof(T), PK = D / EPV;
  constexpr int NE = 16 / G;        // queries per 16-row tile
  constexpr int QW = TPW * NE;      // queries per wave
  constexpr int QB = 4 * QW;        // queries per workgroup
  constexpr int RUN = 16;           // chunks per flush of the staged keys
  constexpr int KSP = RUN + 4;      // padded words per query
  __shared__ __align__(16) T ks[64 * D];
  __shared__ __align__(16) uint32_t kst[4][QW * KSP];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r16 = lane % 16, grp = lane / 16;
  const int64_t T_ = a.T;
  const int64_t qb = (int64_t)(gridDim.x - 1 - blockIdx.x) * QB;   // longest rows first
  const int64_t qw0 = qb + (int64_t)wave * QW;
  const T* qg = static_cast<const T*>(a.qh);
  const T* kg = static_cast<const T*>(a.ksum) + ((int64_t)b * a.Hkv + g) * T_ * D;
  Frag<T> bq[TPW][KS];
  int nct[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int64_t qi = qw0 + t * NE + r16 / G;
    const int h = g * G + r16 % G;
    const T* qrow = qg + (((int64_t)b * a.Hq + h) * T_ + min(qi, T_ - 1)) * D + 8 * grp;
#pragma unroll
    for (int kq = 0; kq < KS; ++kq) load_frag(bq[t][kq], qrow + 32 * kq);
    nct[t] = qi < T_ ? (int)num_candidates(qi, a.S, a.W) : 0;
  }
  const int nc_block = (int)num_candidates(min(qb + QB - 1, T_ - 1), a.S, a.W);
  const int nc_wave = (int)num_candidates(min(qw0 + QW - 1, T_ - 1), a.S, a.W);
  const float sl2 = a.scale * kLog2e;
  constexpr float kLn2 = 0.6931471805599453f;
  float L2[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) L2[t] = 0.f;
  for (int sweep = G > 1 ? 0 : 1; sweep < 2; ++sweep) {
    float M[TPW], Z[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      M[t] = -1e30f;
      Z[t] = 0.f;
    }
    for (int c = 0; c < nc_block; ++c) {
      __syncthreads();
      for (int e = threadIdx.x; e < 64 * PK; e += 256) {
        const int row = e / PK, p = e % PK;
        *reinterpret_cast<uint4*>(ks + swz<PK>(row, p) * EPV) =
            *reinterpret_cast<const uint4*>(kg + ((int64_t)c * 64 + row) * D + p * EPV);
      }
      __syncthreads();
      if (c >= nc_wave) continue;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        f32x4_t acc[4];
        score_tile<T, D>(ks, bq[t], acc, r16, grp);
        float mx = kNegInf;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) mx = fmaxf(mx, acc[mt][q4]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        mx *= sl2;
        float z = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) z += hw_exp2(fmaf(acc[mt][q4], sl2, -mx));
        z += __shfl_xor(z, 16, kWave);
        z += __shfl_xor(z, 32, kWave);
        const float lz2 = mx + __log2f(z);   // log2 of the chunk mass
        const bool valid = c < nct[t];
        if (sweep == 0) {
          if (valid) {
            const float m2 = fmaxf(M[t], lz2);
            Z[t] = Z[t] * hw_exp2(M[t] - m2) + hw_exp2(lz2 - m2);
            M[t] = m2;
          }
        } else {
          float r = valid ? (G > 1 ? lz2 - L2[t] : lz2) : kNegInf;
#pragma unroll
          for (int o = 1; o < G; o <<= 1) r = fmaxf(r, __shfl_xor(r, o, kWave));
          if (grp == 0 && r16 % G == 0) kst[wave][(t * NE + r16 / G) * KSP + c % RUN] = order_key(r * kLn2);
        }
      }
      if (sweep == 1 && (c % RUN == RUN - 1 || c == nc_wave - 1)) {
        wave_lds_sync();
#pragma unroll
        for (int qq0 = 0; qq0 < QW; qq0 += 16) {
          const int qq = qq0 + lane / 4, p = lane % 4;
          const int64_t qi = qw0 + qq;
          if (qq < QW && qi < T_)
            *reinterpret_cast<uint4*>(keys + qi * NCP + (c - c % RUN) + 4 * p) =
                *reinterpret_cast<const uint4*>(&kst[wave][qq * KSP + 4 * p]);
        }
        wave_lds_sync();
      }
    }
    if (sweep == 0) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) L2[t] = nct[t] > 0 ? M[t] + __log2f(Z[t]) : 0.f;
    }
  }
}

// |A n B| per row of two selections (ascending ids, -1 pads at the end).
__global__ __launch_bounds__(256) void overlap_kernel(const int32_t* __restrict__ ia,
                                                      const int32_t* __restrict__ ib,
                                                      int32_t* __restrict__ cnt, int64_t nrows, int topk) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= nrows) return;
  const int32_t* x = ia + r * topk;
  const int32_t* y = ib + r * topk;
  int u = 0, v = 0, n = 0;
  while (u < topk && v < topk && x[u] >= 0 && y[v] >= 0) {
    if (x[u] == y[v]) {
      ++n;
      ++u;
      ++v;
    } else if (x[u] < y[v]) {
      ++u;
    } else {
      ++v;
    }
  }
  cnt[r] = n;
}

template <typename T, int D, int G, int J>
hipError_t launch_bsa_j(const SelArgs& a, hipStream_t st) {
  constexpr int QB = 4 * bsa_tpw<T>() * (16 / G);
  const dim3 tiles((unsigned)((a.T + QB - 1) / QB)), rows((unsigned)((a.T + 3) / 4));
  uint32_t* keys = reinterpret_cast<uint32_t*>(a.scratch);
  const int nbg = a.B * a.Hkv;
  for (int bg0 = 0; bg0 < nbg; bg0 += a.gpass) {
    const int n = min(a.gpass, nbg - bg0);
    {
      KTimer tm(K_BSA_KEYS, st);
      hipLaunchKernelGGL((bsa_keys_kernel<T, D, G, 64 * J>), dim3(tiles.x, (unsigned)n), dim3(256), 0, st, a,
                         bg0, keys);
    }
    KTimer tm(K_BSA_TOPK, st);
    hipLaunchKernelGGL((topk_scores_kernel<T, D, G, J>), dim3(rows.x, (unsigned)n), dim3(256), 0, st, a, bg0, keys);
  }
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t launch_bsa_g(const SelArgs& a, int J, hipStream_t st) {
  switch (J) {
    case 1: return launch_bsa_j<T, D, G, 1>(a, st);
    case 4: return launch_bsa_j<T, D, G, 4>(a, st);
    case 16: return launch_bsa_j<T, D, G, 16>(a, st);
    case 32: return launch_bsa_j<T, D, G, 32>(a, st);
    case 64: return launch_bsa_j<T, D, G, 64>(a, st);
    default: return launch_bsa_j<T, D, G, 128>(a, st);
  }
}

template <typename T, int D>
hipError_t launch_bsa_t(const SelArgs& a, int J, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_bsa_g<T, D, 1>(a, J, st);
    case 2: return launch_bsa_g<T, D, 2>(a, J, st);
    case 4: return launch_bsa_g<T, D, 4>(a, J, st);
    default: return launch_bsa_g<T, D, 8>(a, J, st);
  }
}

int pick_J(int64_t NCs) {
  const int64_t need = (NCs + 63) / 64;
  if (need <= 1) return 1;
  if (need <= 4) return 4;
  if (need <= 16) return 16;
  if (need <= 32) return 32;
  if (need <= 64) return 64;
  return 128;   // up to 8192 candidates: 128 keys per lane
}

}  // namespace

size_t select_workspace(int B, int Hq, int Hkv, int64_t T, int S, bool bf16, int* n_slots,
                        int64_t* slot_stride, size_t* fixed, size_t* per_group) {
  (void)bf16;
  const int64_t NCs = T / S;
  const int J = pick_J(NCs);
  const int64_t stride = 64 * (int64_t)J;   // rank keys of one query
  if (n_slots) *n_slots = (int)T;            // rows of one (b, group)
  if (slot_stride) *slot_stride = stride;
  // the per-head LSE, then the rank keys of every (b, group) (fewer make passes)
  const size_t f = ((Hq / Hkv > 1 ? (size_t)B * Hq * T * sizeof(float) : 0) + 255) / 256 * 256 + 256;
  const size_t pg = ((size_t)T * stride * sizeof(uint32_t) + 255) / 256 * 256;
  if (fixed) *fixed = f;
  if (per_group) *per_group = pg;
  return f + (size_t)B * Hkv * pg;
}

hipError_t launch_select(const SelArgs& a, hipStream_t st) {
  const int J = pick_J(a.NCs);
  if (a.bf16) return a.D == 128 ? launch_select_t<bf16_t, 128>(a, J, st) : launch_select_t<bf16_t, 64>(a, J, st);
  return a.D == 128 ? launch_select_t<float, 128>(a, J, st) : launch_select_t<float, 64>(a, J, st);
}

hipError_t launch_bsa_select(const SelArgs& a, hipStream_t st) {
  const int J = pick_J(a.NCs);
  if (a.bf16) return a.D == 128 ? launch_bsa_t<bf16_t, 128>(a, J, st) : launch_bsa_t<bf16_t, 64>(a, J, st);
  return a.D == 128 ? launch_bsa_t<float, 128>(a, J, st) : launch_bsa_t<float, 64>(a, J, st);
}

hipError_t launch_overlap(const int32_t* ia, const int32_t* ib, int32_t* cnt, int64_t nrows, int topk,
                          hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  hipLaunchKernelGGL(overlap_kernel, dim3((unsigned)((nrows + 255) / 256)), dim3(256), 0, st, ia, ib, cnt,
                     nrows, topk);
  return hipGetLastError();
}

}  // namespace hils
