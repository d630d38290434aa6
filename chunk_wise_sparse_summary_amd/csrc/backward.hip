// backward.hip -- gradients of the prefill attention and fusion, and of the
// landmark summaries (paper-body page, RQ2: the loss reaches the retrieval
// scores, hence the summaries and the calibrated query, through the fused
// weights; summary page, Methodology 1, Eq. 8 carries it on to the landmark
// queries and the keys).  The selection is held fixed (it is piecewise constant
// in the inputs).  Gradients are fp32.
//
// For a row (b, h, i) with upstream gradients g = dout, gl = dlse and the
// forward's out, lse = L:
//   w_c = exp(s_hat_c - L) for a selected chunk, D = g . out,
//   chunk token j:  alpha = w_c p_cj, ds = alpha (g . v_j - D_c), D_c = sum_j p_cj g . v_j
//   window token j: alpha = exp(s_ij - L), ds = alpha (g . v_j - D + gl)
//   dv_j += alpha g,  dk_j += scale ds q_i,  dq_i += scale ds k_j
//   d s_hat_c = w_c (D_c - D + gl): dq_hat += scale d s_hat k'_c, dk'_c += scale d s_hat q_hat,
//   db'_c += d s_hat.
// Kernels:
//   bwd_rowstat  D per row.
//   bwd_kv       key-major, one workgroup per (b, group, chunk): every row that
//                attends the chunk (the window's queries and the entries that
//                selected it) in 16-row MFMA tiles fetched one tile ahead; the
//                four waves split d for the dK / dV accumulators (kept in
//                registers for the whole chunk, so each key row is written once,
//                deterministically).  For selected rows it also writes d s_hat
//                and the row's dq part from this chunk (scale ds K, in the I/O
//                dtype), and it accumulates the chunk's dk', db'.
//   bwd_dq       query-major: the window's part of dq plus the selected parts.
//   bwd_qhat     dq_hat per row.
//   sum_bwd      Eq. 8 backward per (b, group, chunk): dq' and dk += ... .
#include "attend_tiles.h"
#include <type_traits>

#include "hils_internal.h"
#include "topk.h"   // wave_lds_sync

namespace hils {

namespace {

constexpr int kS = 64;
constexpr int kBT = 256;   // threads of the tile kernels (4 waves)

struct BwdKArgs {
  BwdArgs a;
  EntryLists el;
  float* Drow;    // [B, Hq, T]
  float* dshat;   // [B, Hq, T, topk]
  void* dqp;      // [ng, B, T, topk, G, D] io dtype: the selected chunks' dq parts of groups g0 ..
  int g0;         // first KV head of this pass
};

// 16x16x16 products (contraction over the 16 rows of a tile): A lane l holds row
// l%16 and contraction elements 4(l/16) .. +3; B lane l holds column l%16 and the
// same elements.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
template <typename T> struct R4;
template <> struct R4<bf16_t> { s16x4_t v; };
template <> struct R4<float> { float v[4]; };

__device__ __forceinline__ void mma16(f32x4_t& c, const R4<bf16_t>& a, const R4<bf16_t>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4_t& c, const R4<float>& a, const R4<float>& b) {
#pragma unroll
  for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], c, 0, 0, 0);
}
__device__ __forceinline__ void set4(R4<bf16_t>& r, const bf16_t* x) {
  r.v = s16x4_t{(short)x[0], (short)x[1], (short)x[2], (short)x[3]};
}
__device__ __forceinline__ void set4(R4<float>& r, const float* x) {
#pragma unroll
  for (int e = 0; e < 4; ++e) r.v[e] = x[e];
}
// Four consecutive elements (8 bytes for bf16, 16 for fp32) of LDS.
__device__ __forceinline__ void load4(R4<bf16_t>& r, const bf16_t* p) {
  r.v = __builtin_bit_cast(s16x4_t, *reinterpret_cast<const uint2*>(p));
}
__device__ __forceinline__ void load4(R4<float>& r, const float* p) {
  const float4 x = *reinterpret_cast<const float4*>(p);
  r.v[0] = x.x; r.v[1] = x.y; r.v[2] = x.z; r.v[3] = x.w;
}

// Position of token `tok` in a V^T-ordered row (the inverse of vt_token).
__device__ __forceinline__ int vt_pos(int tok) {
  const int k2 = tok >> 5, h = (tok >> 4) & 1, grp = (tok >> 2) & 3, i = tok & 3;
  return 32 * k2 + 8 * grp + 4 * h + i;
}

// The chunk's K and V rows (zero past the sequence) into swizzled [token][d]
// tiles, and K^T into a swizzled [d][token] tile with its tokens in natural
// order (VT = false) or in V^T order (VT = true).
template <typename T, int D, bool VT>
__device__ __forceinline__ void stage_kv(const T* kc, const T* vc, T* ks, T* vs, T* kt, int nvalid) {
  constexpr int EPV = 16 / (int)sizeof(T), PK = D / EPV, PV = kS / EPV;
  for (int e = threadIdx.x; e < kS * PK; e += kBT) {
    const int row = e / PK, p = e % PK;
    uint4 uk = make_uint4(0u, 0u, 0u, 0u), uv = make_uint4(0u, 0u, 0u, 0u);
    if (row < nvalid) {
      uk = *reinterpret_cast<const uint4*>(kc + (int64_t)row * D + p * EPV);
      uv = *reinterpret_cast<const uint4*>(vc + (int64_t)row * D + p * EPV);
    }
    *reinterpret_cast<uint4*>(ks + swz<PK>(row, p) * EPV) = uk;
    *reinterpret_cast<uint4*>(vs + swz<PK>(row, p) * EPV) = uv;
    const T* x = reinterpret_cast<const T*>(&uk);
    const int col = VT ? vt_pos(row) : row;
#pragma unroll
    for (int t = 0; t < EPV; ++t) {
      const int d = p * EPV + t;
      kt[swz<PV>(d, col / EPV) * EPV + col % EPV] = x[t];
    }
  }
}

// ---------------------------------------------------------------- row statistics
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_rowstat_kernel(BwdKArgs k) {
  const BwdArgs& a = k.a;
  constexpr int DPL = D / kWave;
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t nrows = (int64_t)a.B * a.Hq * a.T;
  if (row >= nrows) return;
  const T* g = static_cast<const T*>(a.dout) + row * D + lane * DPL;
  const T* o = static_cast<const T*>(a.out) + row * D + lane * DPL;
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc = fmaf(to_f<T>(g[e]), to_f<T>(o[e]), acc);
  acc = wave_sum(acc);
  if (lane == 0) k.Drow[row] = acc;
}

// ---------------------------------------------------------------- key-major pass
template <typename T, int D>
struct KvSmem {
  static constexpr int EPV = 16 / (int)sizeof(T);
  static constexpr int OP = D + EPV;    // padded row of the q / dout / q_hat tiles
  static constexpr int DRP = kS + EPV;  // padded row of ds as [row][token]
  T ks[kS * D];
  T vs[kS * D];
  T kt[D * kS];
  T qt[16 * OP];
  T gt[16 * OP];
  T ht[16 * OP];    // q_hat rows (selected tiles)
  T at[kS * 16];    // alpha as [token][row]
  T dt[kS * 16];    // ds as [token][row]
  T dr[16 * DRP];   // ds as [row][token]
  float rp[4][3][16];   // each wave's row max, sum and sum of p (g . v) over its tokens
  float rl[16], rd[16], rg[16], rw[16], rds[16];
  int64_t ri[16];
  int rs[16];
};

// The rows of one 16-row tile, fetched into registers one tile ahead: this
// thread's 16-byte pieces of the q, dout (and, for selected tiles, q_hat) rows,
// and for threads < 16 the row's statistics.
template <typename T, int D>
struct TileRegs {
  static constexpr int EPV = 16 / (int)sizeof(T), PK = D / EPV;
  static constexpr int NP = (16 * PK + kBT - 1) / kBT;   // pieces per thread
  uint4 q[NP], g[NP], h[NP];
  float L, Dr, gl, w;
  int64_t i;
  int slot;
};

// One workgroup per (b, KV head, 64-token chunk).  Wave w scores the chunk's
// tokens 16w .. 16w+15 against each 16-row tile (S = K Q^T and U = V G^T, G the
// rows' dout), forms alpha and ds, and shares them through LDS; then each wave
// accumulates dV^T += G^T alpha^T and dK^T += Q^T ds^T for its quarter of d.
// Tiles: the queries whose window holds the chunk (16/G queries x G heads), then
// the entries that selected it; each tile's rows are fetched one tile ahead.
// For a selected row it also writes the row's dq part from this chunk
// (scale K^T ds^T) and accumulates the chunk's dk' = scale sum d s_hat q_hat and
// db' = sum d s_hat (every entry of the chunk passes through this workgroup).
template <typename T, int D, int G>
__global__ __launch_bounds__(kBT) void bwd_kv_kernel(BwdKArgs k) {
  const BwdArgs& a = k.a;
  using SM = KvSmem<T, D>;
  using TR = TileRegs<T, D>;
  constexpr int KS = D / 32, MDW = D / 64;   // d tiles of 16 per wave
  constexpr int EPV = SM::EPV, PK = D / EPV, PV = kS / EPV, OP = SM::OP, DRP = SM::DRP;
  constexpr int NE = 16 / G;                 // queries / entries per tile
  constexpr int DPW = D / 4;                 // dims of dk' per wave
  constexpr int LPH = kWave / G;             // lanes per head for dk'
  constexpr int DPLH = DPW > LPH ? DPW / LPH : 1;
  __shared__ __align__(16) SM sm;
  // the group index fastest: every group's early chunks (the longest entry
  // lists) are dispatched first, so none of them starts late and sets the tail
  const int64_t c = blockIdx.y;
  const int g = k.g0 + blockIdx.x, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r16 = lane % 16, grp = lane / 16;
  const int64_t T_ = a.T;
  const int64_t j0 = c * kS;
  const int nvalid = (int)min<int64_t>(kS, T_ - j0);
  const int64_t bgo = (int64_t)b * a.Hkv + g;
  const float sl2 = a.scale * kLog2e;
  const bool has_sum = c < k.el.NCs;        // a complete chunk: it has k', b'
  stage_kv<T, D, false>(static_cast<const T*>(a.k) + (bgo * T_ + j0) * D,
                        static_cast<const T*>(a.v) + (bgo * T_ + j0) * D, sm.ks, sm.vs, sm.kt, nvalid);
  // rows that attend this chunk: the window's queries [j0, iw1], then the entries
  // that selected it (complete chunks only)
  const int64_t iw1 = min<int64_t>(T_ - 1, j0 + a.W + kS - 2);
  const int nwt = (int)((iw1 - j0 + 1 + NE - 1) / NE);
  int nsel = 0;
  int64_t ebase = 0;
  if (a.topk > 0 && has_sum) {
    const int64_t bucket = bgo * k.el.NCs + c;
    nsel = k.el.bcount[bucket];
    ebase = k.el.bbase[bucket];
  }
  const int nst = (nsel + NE - 1) / NE;
  const int ntile = nwt + nst;
  // The entry word (query << 6 | slot) of row rho of a selected tile, or none.
  // Words are loaded a tile before the rows they name, so a tile's row loads
  // never wait on its entry loads.
  auto word_of = [&](int tile, int rho) -> uint32_t {
    if (tile < nwt || tile >= ntile) return 0xffffffffu;
    const int en = (tile - nwt) * NE + rho / G;
    return en < nsel ? k.el.entries[ebase + en] : 0xffffffffu;
  };
  // row rho of tile `tile`: (query or entry, head)
  auto row_of = [&](int tile, int rho, uint32_t word, int64_t& i, int& slot) -> bool {
    slot = 0;
    if (tile < nwt) {
      i = j0 + (int64_t)tile * NE + rho / G;
      return i <= iw1;
    }
    if (word == 0xffffffffu) {
      i = 0;
      return false;
    }
    i = word >> 6;
    slot = (int)(word & 63u);
    return true;
  };
  // the rows this thread fetches: its pieces' rows, and for threads < 16 row threadIdx.x
  uint32_t wp[TR::NP], wst;
  auto load_words = [&](int tile) {
#pragma unroll
    for (int t = 0; t < TR::NP; ++t) wp[t] = word_of(tile, (int)((threadIdx.x + t * kBT) / PK));
    wst = threadIdx.x < 16 ? word_of(tile, (int)threadIdx.x) : 0xffffffffu;
  };
  auto fetch = [&](int tile, TR& r) {
    const bool selt = tile >= nwt;
#pragma unroll
    for (int t = 0; t < TR::NP; ++t) {
      const int e = threadIdx.x + t * kBT;
      r.q[t] = r.g[t] = r.h[t] = make_uint4(0u, 0u, 0u, 0u);
      if (TR::NP * kBT == 16 * PK || e < 16 * PK) {
        const int rho = e / PK, p = e % PK;
        int64_t i;
        int slot;
        if (row_of(tile, rho, wp[t], i, slot)) {
          const int64_t ro = (((int64_t)b * a.Hq + g * G + rho % G) * T_ + i) * D + p * EPV;
          r.q[t] = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.q) + ro);
          r.g[t] = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.dout) + ro);
          if (selt) r.h[t] = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.qh) + ro);
        }
      }
    }
    if (threadIdx.x < 16) {
      const int rho = threadIdx.x;
      int64_t i;
      int slot;
      const bool valid = row_of(tile, rho, wst, i, slot);
      const int64_t rq = ((int64_t)b * a.Hq + g * G + rho % G) * T_ + (valid ? i : 0);
      r.L = valid ? a.lse[rq] : 0.f;
      r.Dr = valid ? k.Drow[rq] : 0.f;
      r.gl = (valid && a.dlse) ? a.dlse[rq] : 0.f;
      r.w = (valid && selt) ? a.ssel[rq * a.topk + slot] : 0.f;
      r.i = valid ? i : -1;
      r.slot = slot;
    }
  };
  f32x4_t dka[MDW][4], dva[MDW][4];
#pragma unroll
  for (int t = 0; t < MDW; ++t)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      dka[t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      dva[t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  float dks_acc[DPLH];
#pragma unroll
  for (int j = 0; j < DPLH; ++j) dks_acc[j] = 0.f;
  float dbs_acc = 0.f;
  const int hk = lane / LPH, lk = lane % LPH;   // this lane's dk' head and its dims
  TR nxt;
  if (ntile > 0) {
    load_words(0);
    fetch(0, nxt);
    load_words(1);
  }
  // this wave's 16 key and value rows are the A operands of every tile's S and
  // U: held in registers for the whole chunk instead of re-read from LDS per tile
  __syncthreads();   // the staged chunk
  Frag<T> akf[KS], avf[KS];
#pragma unroll
  for (int kq = 0; kq < KS; ++kq) {
    load_frag_swz<PK>(akf[kq], sm.ks, 16 * wave + r16, 8 * grp + 32 * kq);
    load_frag_swz<PK>(avf[kq], sm.vs, 16 * wave + r16, 8 * grp + 32 * kq);
  }
  for (int tile = 0; tile < ntile; ++tile) {
    const bool selt = tile >= nwt;
    __syncthreads();   // the previous tile is done with the shared tiles
#pragma unroll
    for (int t = 0; t < TR::NP; ++t) {
      const int e = threadIdx.x + t * kBT;
      if (TR::NP * kBT == 16 * PK || e < 16 * PK) {
        const int rho = e / PK, p = e % PK;
        *reinterpret_cast<uint4*>(sm.qt + rho * OP + p * EPV) = nxt.q[t];
        *reinterpret_cast<uint4*>(sm.gt + rho * OP + p * EPV) = nxt.g[t];
        if (selt) *reinterpret_cast<uint4*>(sm.ht + rho * OP + p * EPV) = nxt.h[t];
      }
    }
    if (threadIdx.x < 16) {
      const int rho = threadIdx.x;
      sm.rl[rho] = nxt.L * kLog2e;
      sm.rd[rho] = nxt.Dr;
      sm.rg[rho] = nxt.gl;
      sm.rw[rho] = selt && nxt.i >= 0 ? __expf(nxt.w - nxt.L) : 0.f;
      sm.ri[rho] = nxt.i;
      sm.rs[rho] = nxt.slot;
    }
    if (tile + 1 < ntile) {   // in flight during this tile: the next tile's rows, the words after
      fetch(tile + 1, nxt);
      load_words(tile + 2);
    }
    __syncthreads();
    // this wave's 16 tokens: S^T and U^T (token 16 wave + 4 grp + q4, row r16)
    f32x4_t sa = f32x4_t{0.f, 0.f, 0.f, 0.f}, ua = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kq = 0; kq < KS; ++kq) {
      Frag<T> bq, bg;
      load_frag(bq, sm.qt + r16 * OP + 8 * grp + 32 * kq);
      load_frag(bg, sm.gt + r16 * OP + 8 * grp + 32 * kq);
      mma(sa, akf[kq], bq);
      mma(ua, avf[kq], bg);
    }
    const int64_t i = sm.ri[r16];
    const bool valid = i >= 0;
    const float L2 = sm.rl[r16], Dr = sm.rd[r16], gl = sm.rg[r16];
    float al[4], ds[4];
    if (selt) {
      // the chunk's softmax per row: partial max / sum / sum p (g . v) per wave,
      // combined through LDS
      float mx = fmaxf(fmaxf(sa[0], sa[1]), fmaxf(sa[2], sa[3])) * sl2;
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      float e[4], z = 0.f, t = 0.f;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        e[q4] = hw_exp2(fmaf(sa[q4], sl2, -mx));
        z += e[q4];
        t = fmaf(e[q4], ua[q4], t);
      }
      z += __shfl_xor(z, 16, kWave);
      z += __shfl_xor(z, 32, kWave);
      t += __shfl_xor(t, 16, kWave);
      t += __shfl_xor(t, 32, kWave);
      if (grp == 0) {
        sm.rp[wave][0][r16] = mx;
        sm.rp[wave][1][r16] = z;
        sm.rp[wave][2][r16] = t;
      }
      __syncthreads();
      float m = sm.rp[0][0][r16];
#pragma unroll
      for (int w = 1; w < 4; ++w) m = fmaxf(m, sm.rp[w][0][r16]);
      float Z = 0.f, U = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = hw_exp2(sm.rp[w][0][r16] - m);
        Z = fmaf(sm.rp[w][1][r16], f, Z);
        U = fmaf(sm.rp[w][2][r16], f, U);
      }
      const float inv = 1.f / Z;
      const float dc = U * inv;
      const float wr = valid ? sm.rw[r16] : 0.f;
      const float sc = wr * inv * hw_exp2(mx - m);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        al[q4] = sc * e[q4];
        ds[q4] = al[q4] * (ua[q4] - dc);
      }
      const float dsh = valid ? wr * (dc - Dr + gl) : 0.f;
      if (wave == 0 && grp == 0) {
        sm.rds[r16] = dsh;
        if (valid) {
          const int64_t rq = ((int64_t)b * a.Hq + g * G + r16 % G) * T_ + i;
          k.dshat[rq * a.topk + sm.rs[r16]] = dsh;
        }
      }
    } else {
      const int64_t lw = valid ? window_left(i, a.S, a.W) : 0;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int64_t j = j0 + 16 * wave + 4 * grp + q4;
        const bool ok = valid && j >= lw && j <= i;
        al[q4] = ok ? hw_exp2(fmaf(sa[q4], sl2, -L2)) : 0.f;
        ds[q4] = al[q4] * (ua[q4] - Dr + gl);
      }
    }
    {
      const int tok0 = 16 * wave + 4 * grp;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        sm.at[(tok0 + q4) * 16 + r16] = from_f<T>(al[q4]);
        sm.dt[(tok0 + q4) * 16 + r16] = from_f<T>(ds[q4]);
      }
      if (selt) {
        T x[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) x[q4] = from_f<T>(ds[q4]);
        if constexpr (sizeof(T) == 2)
          *reinterpret_cast<uint2*>(sm.dr + r16 * DRP + tok0) = *reinterpret_cast<const uint2*>(x);
        else
          *reinterpret_cast<float4*>(sm.dr + r16 * DRP + tok0) = *reinterpret_cast<const float4*>(x);
      }
    }
    __syncthreads();
    // dV^T += G^T alpha^T, dK^T += Q^T ds^T over the tile's 16 rows, d slice of this wave
#pragma unroll
    for (int t = 0; t < MDW; ++t) {
      const int d = (wave * MDW + t) * 16 + r16;
      T xg[4], xq[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xg[e] = sm.gt[(4 * grp + e) * OP + d];
        xq[e] = sm.qt[(4 * grp + e) * OP + d];
      }
      R4<T> ag, aq;
      set4(ag, xg);
      set4(aq, xq);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        R4<T> ba, bd;
        load4(ba, sm.at + (16 * mt + r16) * 16 + 4 * grp);
        load4(bd, sm.dt + (16 * mt + r16) * 16 + 4 * grp);
        mma16(dva[t][mt], ag, ba);
        mma16(dka[t][mt], aq, bd);
      }
    }
    if (selt) {
      // dq part^T (d slice, 16 rows) = scale K^T ds^T over the chunk
      const bool vrow = sm.ri[r16] >= 0;
      const int slot = sm.rs[r16];
      const int64_t ir = sm.ri[r16];
#pragma unroll
      for (int t = 0; t < MDW; ++t) {
        const int md = wave * MDW + t;
        f32x4_t o = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          Frag<T> af, bf;
          load_frag_swz<PV>(af, sm.kt, 16 * md + r16, 32 * k2 + 8 * grp);
          load_frag(bf, sm.dr + r16 * DRP + 32 * k2 + 8 * grp);
          mma(o, af, bf);
        }
        if (vrow)
          store4<T>(static_cast<T*>(k.dqp) +
                        (((((int64_t)(g - k.g0) * a.B + b) * T_ + ir) * a.topk + slot) * G + r16 % G) * D +
                        16 * md + 4 * grp,
                    o, a.scale);
      }
      // dk' (this wave's dims, lane's head) and db' over the tile's rows of that head
      if (lk * DPLH < DPW) {
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const int rho = e * G + hk;
          const float w = sm.rds[rho];
#pragma unroll
          for (int j = 0; j < DPLH; ++j)
            dks_acc[j] = fmaf(w, to_f<T>(sm.ht[rho * OP + wave * DPW + lk * DPLH + j]), dks_acc[j]);
          if (wave == 0 && lk == 0) dbs_acc += w;
        }
      }
    }
  }
  // the chunk's key rows: lane holds token 16 mt + r16 and dims 16 dt + 4 grp + q4
#pragma unroll
  for (int t = 0; t < MDW; ++t)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int tok = 16 * mt + r16;
      if (tok < nvalid) {
        const int64_t o = (bgo * T_ + j0 + tok) * D + (wave * MDW + t) * 16 + 4 * grp;
        *reinterpret_cast<float4*>(a.dk + o) = make_float4(dka[t][mt][0] * a.scale, dka[t][mt][1] * a.scale,
                                                           dka[t][mt][2] * a.scale, dka[t][mt][3] * a.scale);
        *reinterpret_cast<float4*>(a.dv + o) =
            make_float4(dva[t][mt][0], dva[t][mt][1], dva[t][mt][2], dva[t][mt][3]);
      }
    }
  // the chunk's summary gradients (zero when nothing selected it)
  if (has_sum && lk * DPLH < DPW) {
    const int64_t bhc = ((int64_t)b * a.Hq + g * G + hk) * k.el.NCs + c;
#pragma unroll
    for (int j = 0; j < DPLH; ++j) a.dks[bhc * D + wave * DPW + lk * DPLH + j] = dks_acc[j] * a.scale;
    if (wave == 0 && lk == 0) a.dbs[bhc] = dbs_acc;
  }
}

// ---------------------------------------------------------------- query-major dq
// Four waves of 16 rows (16/G queries x G heads each); the window's chunks are
// staged once per workgroup.  dq = scale K^T ds^T over the window, plus the
// selected chunks' parts written by bwd_kv.
template <typename T, int D, int G>
__global__ __launch_bounds__(kBT) void bwd_dq_kernel(BwdKArgs k) {
  const BwdArgs& a = k.a;
  constexpr int KS = D / 32, MD = D / 16;
  constexpr int NE = 16 / G;
  constexpr int QB = 4 * NE;   // queries per workgroup
  __shared__ __align__(16) T kvs[2 * kS * D];   // K then V tiles; the window part of dq at the end
  __shared__ __align__(16) T kt[D * kS];
  T* ks = kvs;
  T* vs = kvs + kS * D;
  const int g = k.g0 + blockIdx.y, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r16 = lane % 16, grp = lane / 16;
  const int64_t T_ = a.T;
  const int64_t qb0 = (int64_t)blockIdx.x * QB;
  const int64_t qlast = min<int64_t>(qb0 + QB - 1, T_ - 1);
  const int64_t i = qb0 + wave * NE + r16 / G;
  const int hh = r16 % G;
  const bool valid = i < T_;
  const int64_t ic = valid ? i : T_ - 1;
  const int64_t rq = ((int64_t)b * a.Hq + g * G + hh) * T_ + ic;
  const float sl2 = a.scale * kLog2e;
  Frag<T> bq[KS], bg[KS];
#pragma unroll
  for (int kq = 0; kq < KS; ++kq) {
    load_frag(bq[kq], static_cast<const T*>(a.q) + rq * D + 8 * grp + 32 * kq);
    load_frag(bg[kq], static_cast<const T*>(a.dout) + rq * D + 8 * grp + 32 * kq);
  }
  const float L2 = a.lse[rq] * kLog2e, Dr = k.Drow[rq], gl = a.dlse ? a.dlse[rq] : 0.f;
  const int64_t lw = window_left(ic, a.S, a.W);
  f32x4_t acc[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) acc[md] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int64_t bgo = (int64_t)b * a.Hkv + g;
  const int64_t c_lo = window_left(qb0, a.S, a.W) / kS, c_hi = qlast / kS;
  for (int64_t c = c_lo; c <= c_hi; ++c) {
    const int64_t j0 = c * kS;
    __syncthreads();
    stage_kv<T, D, true>(static_cast<const T*>(a.k) + (bgo * T_ + j0) * D,
                         static_cast<const T*>(a.v) + (bgo * T_ + j0) * D, ks, vs, kt,
                         (int)min<int64_t>(kS, T_ - j0));
    __syncthreads();
    f32x4_t sa[4], ua[4];
    score_tile<T, D>(ks, bq, sa, r16, grp);
    score_tile<T, D>(vs, bg, ua, r16, grp);
    float ds[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int64_t j = j0 + 16 * mt + 4 * grp + q4;
        const bool ok = valid && j >= lw && j <= i;
        const float al = ok ? hw_exp2(fmaf(sa[mt][q4], sl2, -L2)) : 0.f;
        ds[mt][q4] = al * (ua[mt][q4] - Dr + gl);
      }
    pv_tile<T, D>(kt, ds, acc, r16, grp);
  }
  // The window part goes through LDS (the K/V tiles are free now), so that the
  // selected chunks' dq parts are read as whole 16-byte row pieces, RPI rows
  // per load instruction, and summed slot by slot (the same order for every
  // element).  A padding slot's piece is read from slot 0's row (inside the
  // buffer) and dropped by a select.
  __syncthreads();   // every wave is done with the staged chunk
  float* accl = reinterpret_cast<float*>(kvs) + wave * 16 * D;   // [16 rows][D]
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int e = 0; e < 4; ++e) accl[r16 * D + 16 * md + 4 * grp + e] = acc[md][e] * a.scale;
  wave_lds_sync();
  constexpr int EPV = 16 / (int)sizeof(T), PPR = D / EPV, RPI = kWave / PPR, NR = 16 / RPI;
  using Raw = typename std::conditional<sizeof(T) == 2, uint4, float4>::type;   // EPV elements
  const int pr = lane % PPR, rr0 = lane / PPR;   // this lane's piece and first row
  const int64_t NCs = T_ / a.S;
  float sum[NR][EPV];
  const int32_t* irr[NR];
  const T* pbr[NR];
  bool vr[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int r = rr0 + RPI * j;   // row r of the wave: query r / G, head r % G
    const int64_t qj = qb0 + wave * NE + r / G;
    vr[j] = qj < T_;
    const int64_t qc = vr[j] ? qj : T_ - 1;
    irr[j] = a.idx + (bgo * T_ + qc) * a.topk;
    pbr[j] = static_cast<const T*>(k.dqp) +
             ((((int64_t)blockIdx.y * a.B + b) * T_ + qc) * a.topk * G + r % G) * D + pr * EPV;
#pragma unroll
    for (int e = 0; e < EPV; ++e) sum[j][e] = accl[r * D + pr * EPV + e];
  }
  constexpr int US = 2;
  for (int s0 = 0; s0 < a.topk; s0 += US) {
    Raw v[US][NR];
    bool ok[US][NR];
#pragma unroll
    for (int u = 0; u < US; ++u)
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const int s = s0 + u;
        const int32_t cs = s < a.topk ? irr[j][s] : -1;
        ok[u][j] = cs >= 0 && cs < NCs;
        v[u][j] = *reinterpret_cast<const Raw*>(pbr[j] + (int64_t)(ok[u][j] ? s : 0) * G * D);
      }
#pragma unroll
    for (int u = 0; u < US; ++u)
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const T* x = reinterpret_cast<const T*>(&v[u][j]);
#pragma unroll
        for (int e = 0; e < EPV; ++e) sum[j][e] += ok[u][j] ? to_f<T>(x[e]) : 0.f;
      }
  }
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    if (!vr[j]) continue;
    const int r = rr0 + RPI * j;
    const int64_t qj = qb0 + wave * NE + r / G;
    float* dst = a.dq + (((int64_t)b * a.Hq + g * G + r % G) * T_ + qj) * D + pr * EPV;
#pragma unroll
    for (int e = 0; e < EPV; e += 4)
      *reinterpret_cast<float4*>(dst + e) = make_float4(sum[j][e], sum[j][e + 1], sum[j][e + 2], sum[j][e + 3]);
  }
}

// ---------------------------------------------------------------- dq_hat
// dq_hat_i = scale sum_slots d s_hat k'_c: one wave per row.  Lanes take 16-byte
// pieces of the k' rows, so one load instruction covers SG slots' rows at once;
// the SG slot groups' sums are added across lanes at the end.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void bwd_qhat_kernel(BwdKArgs k) {
  const BwdArgs& a = k.a;
  constexpr int EPV = 16 / (int)sizeof(T);   // elements per 16-byte piece
  constexpr int PPR = D / EPV;               // pieces per row
  constexpr int SG = kWave / PPR;            // slot groups
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;   // (b, h, i)
  const int lane = threadIdx.x % kWave;
  const int sg = lane / PPR, pc = lane % PPR;
  const int64_t nrows = (int64_t)a.B * a.Hq * a.T;
  if (row >= nrows) return;
  const int64_t i = row % a.T;
  const int h = (int)((row / a.T) % a.Hq);
  const int b = (int)(row / (a.T * a.Hq));
  const int g = h / G;
  const int64_t NCs = a.T / a.S;
  float acc[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc[e] = 0.f;
  const int32_t* ir = a.idx + (((int64_t)b * a.Hkv + g) * a.T + i) * a.topk;
  const T* kb = static_cast<const T*>(a.ksum) + ((int64_t)b * a.Hq + h) * NCs * D + pc * EPV;
  // US slot steps per batch, their loads issued before any is used; a padding
  // slot reads chunk 0's row and adds nothing
  constexpr int US = 4;
  if (NCs > 0)
    for (int s0 = 0; s0 < a.topk; s0 += US * SG) {
      float dsh[US];
      uint4 kv[US];
#pragma unroll
      for (int u = 0; u < US; ++u) {
        const int s = s0 + u * SG + sg;
        const int32_t c = s < a.topk ? ir[s] : -1;
        const bool ok = c >= 0 && c < NCs;
        dsh[u] = ok ? k.dshat[row * a.topk + s] : 0.f;
        kv[u] = *reinterpret_cast<const uint4*>(kb + (int64_t)(ok ? c : 0) * D);
      }
#pragma unroll
      for (int u = 0; u < US; ++u) {
        const T* x = reinterpret_cast<const T*>(&kv[u]);
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[e] = fmaf(dsh[u], to_f<T>(x[e]), acc[e]);
      }
    }
#pragma unroll
  for (int e = 0; e < EPV; ++e)
#pragma unroll
    for (int o = PPR; o < kWave; o <<= 1) acc[e] += __shfl_xor(acc[e], o, kWave);
  if (sg == 0) {
    float* dst = a.dqh + row * D + pc * EPV;
#pragma unroll
    for (int e = 0; e < EPV; e += 4)
      *reinterpret_cast<float4*>(dst + e) =
          make_float4(acc[e] * a.scale, acc[e + 1] * a.scale, acc[e + 2] * a.scale, acc[e + 3] * a.scale);
  }
}

// ---------------------------------------------------------------- summaries
// Eq. 8 backward for one (b, group, chunk), a wave: lane j = token j for the
// chunk's softmax of each head, then lanes over d for dq' and dk.
//   e_j = dk' . k_j - db' s_j,  ds_j = p_j (e_j - sum_l p_l e_l)
//   dq' = scale sum_j ds_j k_j,  dk_j += sum_h (p_hj dk'_h + scale ds_hj q'_h)
template <typename T, int D, int G>
__global__ __launch_bounds__(64) void sum_bwd_kernel(SumBwdArgs a) {
  constexpr int DPL = D / kWave;
  __shared__ float pl[G][kS], dl[G][kS];
  const int64_t c = a.c0 + blockIdx.x;
  const int g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const T* kc = static_cast<const T*>(a.k) + (((int64_t)b * a.Hkv + g) * a.kT + c * kS) * D;
  const float sl2 = a.scale * kLog2e;
  for (int hh = 0; hh < G; ++hh) {
    const int64_t bhc = ((int64_t)b * a.Hq + g * G + hh) * a.NCs + c;
    const T* qr = static_cast<const T*>(a.ql) + bhc * D;
    const float* dkr = a.dks + bhc * D;
    float s = 0.f, e = 0.f;
    for (int d = 0; d < D; ++d) {
      const float kv = to_f<T>(kc[(int64_t)lane * D + d]);
      s = fmaf(to_f<T>(qr[d]), kv, s);
      e = fmaf(dkr[d], kv, e);
    }
    const float s2 = s * sl2;
    const float m = wave_max(s2);
    const float z = wave_sum(hw_exp2(s2 - m));
    const float p = hw_exp2(s2 - m) / z;
    e -= a.dbs[bhc] * s * a.scale;
    const float pe = wave_sum(p * e);
    pl[hh][lane] = p;
    dl[hh][lane] = p * (e - pe);
  }
  wave_lds_sync();
  for (int hh = 0; hh < G; ++hh) {
    const int64_t bhc = ((int64_t)b * a.Hq + g * G + hh) * a.NCs + c;
    float acc[DPL];
#pragma unroll
    for (int t = 0; t < DPL; ++t) acc[t] = 0.f;
    for (int j = 0; j < kS; ++j) {
      const float w = dl[hh][j];
#pragma unroll
      for (int t = 0; t < DPL; ++t) acc[t] = fmaf(w, to_f<T>(kc[(int64_t)j * D + lane * DPL + t]), acc[t]);
    }
#pragma unroll
    for (int t = 0; t < DPL; ++t) a.dql[bhc * D + lane * DPL + t] = acc[t] * a.scale;
  }
  float* dkc = a.dk + (((int64_t)b * a.Hkv + g) * a.kT + c * kS) * D;
  for (int j = 0; j < kS; ++j) {
#pragma unroll
    for (int t = 0; t < DPL; ++t) {
      const int d = lane * DPL + t;
      float add = 0.f;
      for (int hh = 0; hh < G; ++hh) {
        const int64_t bhc = ((int64_t)b * a.Hq + g * G + hh) * a.NCs + c;
        add = fmaf(pl[hh][j], a.dks[bhc * D + d], add);
        add = fmaf(dl[hh][j] * a.scale, to_f<T>(static_cast<const T*>(a.ql)[bhc * D + d]), add);
      }
      dkc[(int64_t)j * D + d] += add;
    }
  }
}

// ---------------------------------------------------------------- host side
size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

template <typename T, int D, int G>
hipError_t launch_bwd_tg(BwdKArgs k, int gpp, hipStream_t st) {
  const BwdArgs& a = k.a;
  const int64_t nrows = (int64_t)a.B * a.Hq * a.T;
  {
    KTimer tm(K_BWD_ROWSTAT, st);
    hipLaunchKernelGGL((bwd_rowstat_kernel<T, D>), dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, st, k);
  }
  const int64_t NCf = (a.T + kS - 1) / kS;
  constexpr int QB = 4 * (16 / G);
  for (int g0 = 0; g0 < a.Hkv; g0 += gpp) {
    k.g0 = g0;
    const int ng = min(gpp, a.Hkv - g0);
    {
      KTimer tm(K_BWD_KV, st);
      hipLaunchKernelGGL((bwd_kv_kernel<T, D, G>), dim3((unsigned)ng, (unsigned)NCf, a.B), dim3(kBT), 0, st, k);
    }
    {
      KTimer tm(K_BWD_DQ, st);
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, G>), dim3((unsigned)((a.T + QB - 1) / QB), ng, a.B), dim3(kBT),
                         0, st, k);
    }
  }
  {
    KTimer tm(K_BWD_QHAT, st);
    hipLaunchKernelGGL((bwd_qhat_kernel<T, D, G>), dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, st, k);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_t(const BwdKArgs& k, int gpp, hipStream_t st) {
  switch (k.a.Hq / k.a.Hkv) {
    case 1: return launch_bwd_tg<T, D, 1>(k, gpp, st);
    case 2: return launch_bwd_tg<T, D, 2>(k, gpp, st);
    case 4: return launch_bwd_tg<T, D, 4>(k, gpp, st);
    default: return launch_bwd_tg<T, D, 8>(k, gpp, st);
  }
}

template <typename T, int D>
hipError_t launch_sum_bwd_t(const SumBwdArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.n_chunks, a.Hkv, a.B);
  KTimer tm(K_SUM_BWD, st);
  switch (a.Hq / a.Hkv) {
    case 1: hipLaunchKernelGGL((sum_bwd_kernel<T, D, 1>), grid, dim3(64), 0, st, a); break;
    case 2: hipLaunchKernelGGL((sum_bwd_kernel<T, D, 2>), grid, dim3(64), 0, st, a); break;
    case 4: hipLaunchKernelGGL((sum_bwd_kernel<T, D, 4>), grid, dim3(64), 0, st, a); break;
    default: hipLaunchKernelGGL((sum_bwd_kernel<T, D, 8>), grid, dim3(64), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

void attend_backward_workspace(int B, int Hq, int Hkv, int64_t T, int S, int D, int topk, bool bf16,
                               size_t* fixed, size_t* per_group) {
  const int kk = topk > 0 ? topk : 1;
  const int G = Hq / Hkv;
  *fixed = entry_lists_bytes(B, Hkv, T, S, topk) + al256((size_t)B * Hq * T * 4) +
           al256((size_t)B * Hq * T * kk * 4) + 256;
  *per_group = topk > 0 ? al256((size_t)B * T * kk * G * D * (bf16 ? 2 : 4)) : 0;
}

hipError_t launch_attend_backward(const BwdArgs& a, hipStream_t st) {
  size_t fixed, per;
  attend_backward_workspace(a.B, a.Hq, a.Hkv, a.T, a.S, a.D, a.topk, a.bf16, &fixed, &per);
  BwdKArgs k{};
  k.a = a;
  char* w = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(a.ws) + 255) & ~(uintptr_t)255);
  hipError_t e = launch_entry_lists(a.idx, a.B, a.Hq, a.Hkv, a.T, a.S, a.topk, w, &k.el, st);
  if (e != hipSuccess) return e;
  w += entry_lists_bytes(a.B, a.Hkv, a.T, a.S, a.topk);
  const int kk = a.topk > 0 ? a.topk : 1;
  k.Drow = reinterpret_cast<float*>(w);
  w += al256((size_t)a.B * a.Hq * a.T * 4);
  k.dshat = reinterpret_cast<float*>(w);
  w += al256((size_t)a.B * a.Hq * a.T * kk * 4);
  k.dqp = w;
  // KV heads whose dq parts fit at once (the host checked room for one)
  int gpp = per > 0 ? (int)((a.ws_bytes - fixed) / per) : a.Hkv;
  if (gpp > a.Hkv) gpp = a.Hkv;
  if (gpp < 1) gpp = 1;
  if (a.bf16) return a.D == 128 ? launch_bwd_t<bf16_t, 128>(k, gpp, st) : launch_bwd_t<bf16_t, 64>(k, gpp, st);
  return a.D == 128 ? launch_bwd_t<float, 128>(k, gpp, st) : launch_bwd_t<float, 64>(k, gpp, st);
}

hipError_t launch_summarize_backward(const SumBwdArgs& a, hipStream_t st) {
  if (a.n_chunks <= 0) return hipSuccess;
  if (a.bf16) return a.D == 128 ? launch_sum_bwd_t<bf16_t, 128>(a, st) : launch_sum_bwd_t<bf16_t, 64>(a, st);
  return a.D == 128 ? launch_sum_bwd_t<float, 128>(a, st) : launch_sum_bwd_t<float, 64>(a, st);
}

}  // namespace hils
