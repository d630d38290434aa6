// decode.hip -- one HiLS decode step per sequence (query at position pos[b]).
//
// The step is the prefill row i = pos[b] of the same definitions (summary page,
// Summary and Methodology; paper-body page, RQ1 and GQA-aware selection).  One
// query has little work per byte, so every kernel here streams memory:
//   dec_score   two roles in one launch.  Scoring blocks stream every
//               candidate's k' once (whole-wave contiguous loads, a butterfly
//               reduction) and write s_hat, a (max, sum exp) partial of the
//               head's LSE, the slice's top-k of s_hat and its four largest
//               keys.  Window blocks (after them in the grid) attend the query
//               to each chunk of its window, which needs no selection; the one
//               holding the new token appends its key/value row to the caches.
//   dec_headsel one wave per (b, head, share of slices): the share's top-k of
//               s_hat from its slice lists, pruned by its slices' largest keys;
//               the first share also forms L_h.
//   dec_attend  one workgroup per (b, group, selected slot): every workgroup of
//               a group forms the group's selection from the heads' share lists
//               (for several heads: the top-k by rank key
//               r = max_h (s_hat_h - L_h) over the union of the heads'
//               choices), then attends the chunk of its slot.
//   dec_fuse    one workgroup per (b, head): the exp(log-weight) average of the
//               items' outputs and L = LSE(s_hat over Sel + {log Z_win}).
//   summarize   (list mode) chunks completed by this step's token.
//
// Why the union holds the selection: r_c is attained at some head h*; if c were
// not in h*'s top-k by s_hat (equal s_hat: lower chunk first), k chunks would
// precede it there, and each has r >= s_hat_{h*} - L_{h*} >= r_c, so c would
// not be chosen either.  Only an exact fp32 tie of two rank keys whose s_hat
// differ (a rounding tie, far below any decided gap) can make the choice differ
// from ranking every candidate.  A slice's top-k likewise holds every candidate
// of the slice that is in the head's top-k.
//
// Stages hand over through kernel boundaries: a device-wide fence per block (a
// last-block ticket) costs an L2 write-back on a multi-XCD part.
#include "hils_internal.h"
#include "topk.h"

namespace hils {

namespace {

constexpr int kS = 64;
constexpr int kThreads = 256;

struct DecPos {
  int64_t p[64];
};

struct DecWs {
  float* shat;        // [B, Hq, NCcap] every candidate's s_hat
  float2* lpart;      // [B, Hq, nslice] (max, sum) in log2 units
  uint32_t* lkey;     // [B, Hq, nslice, kk] each slice's top-k keys of s_hat (0: none)
  int32_t* lid;       // [B, Hq, nslice, kk] their chunk ids (ascending within a slice)
  uint32_t* lk4;      // [B, Hq, nslice, 4] the four largest keys of each slice (0: none)
  uint32_t* hkey;     // [B, Hq, kMaxShares, kk] each share's top-k keys of s_hat (0: none)
  int32_t* hid;       // [B, Hq, kMaxShares, kk] their chunk ids
  float* Lh;          // [B, Hq] each head's LSE over the candidates
  float* apart;       // [B, Hkv, nitems, G, D + 2]: items [0, kk) selected, [kk, kk + nwin) window
  // several queries per sequence (rows b*M + m of the arrays above):
  float* mpart;       // [Breal, Hkv, M, nitems_mq, G, D + 2]: each row's selected slots [0, kk), then window chunks
  int32_t* selw;      // [B, Hkv, kk] each row's selection (ascending, -1 pads)
  int nslice, sj, kk, nwin, nitems, mj, nwin_mq, nitems_mq;
  int direct;         // the group selection ranks the slice lists itself (no dec_headsel)
};

struct DecKArgs {
  DecPos pos;
  const void* q;
  const void* qh;
  const void* k_new;
  const void* v_new;
  void* kc;
  void* vc;
  const void* ksum;
  const float* bsum;
  void* out;
  float* lse;
  int32_t* idx_out;
  DecWs w;
  int B, Hq, Hkv, S, W, topk;
  int64_t Lcap, NCcap;
  float scale;
  int M;                // queries per sequence: rows b*M + m of q, q_hat, out, lse, pos
  int32_t* idx_user;    // several queries: the caller's selection output (or null)
};

__device__ __forceinline__ void lse_merge(float& M, float& Z, float mo, float so) {
  const float mn = fmaxf(M, mo);
  if (mn != kNegInf)
    Z = (M == kNegInf ? 0.f : Z * hw_exp2(M - mn)) + (mo == kNegInf ? 0.f : so * hw_exp2(mo - mn));
  M = mn;
}

// One butterfly step per mask M = PPR/2 .. 1 over N values: lanes with bit M set
// keep the upper half (and send the lower), the others the lower half.
template <int M, int N>
__device__ __forceinline__ void butterfly(float (&v)[N], int lane) {
  if constexpr (M >= 1) {
    const bool up = (lane & M) != 0;
#pragma unroll
    for (int k = 0; k < N / 2; ++k) {
      const float send = up ? v[k] : v[k + N / 2];
      const float keep = up ? v[k + N / 2] : v[k];
      v[k] = keep + xor_lane<M>(send);
    }
    if constexpr (M > 1) {
      float w[N / 2];
#pragma unroll
      for (int k = 0; k < N / 2; ++k) w[k] = v[k];
      butterfly<M / 2, N / 2>(w, lane);
      v[0] = w[0];
    }
  }
}

// ---------------------------------------------------------------- item attention
// One work item = one chunk c of (b, group g): the G heads of the group are the 16
// columns of MFMA tiles (zero-padded).  Wave w takes the logits of tokens 16w ..
// 16w + 15 (S^T = K Q^T, its K fragments loaded straight from HBM), the softmax
// statistics of each head meet in LDS, V goes transposed into LDS, and
// O^T = V^T P^T gives wave w the output dims 16(w + 4t) ...  The item's partial
// is its log-weight (s_hat for a selected chunk, the token-level log-mass for a
// window chunk) and its normalised output.  A window chunk masks tokens outside
// [l_i, i]; in the chunk holding i, row i is taken from k_new / v_new (and
// written to the caches here), and rows past i are read as zero.
template <typename T, int D>
struct ItemSmem {
  T vt[D * kS];       // V^T rows, swizzled
  T pt[16 * kS];      // P^T as [head][token]
  float red[2][4][16];
};

template <typename T, int D, int G>
__device__ __forceinline__ void attend_item(const DecKArgs& a, ItemSmem<T, D>& sm, int b, int g,
                                            int slot, int64_t c, bool is_win, const float* lnw) {
  constexpr int EPV = 16 / sizeof(T);
  constexpr int KS = D / 32, MD = D / 16;
  constexpr int PK = D / EPV, PV = kS / EPV;         // 16-byte pieces per K / V^T row
  constexpr int VPW = PK / 4;                        // V pieces per lane (wave w: pieces w*VPW ..)
  constexpr int MDW = MD / 4;                        // output dim tiles per wave
  static_assert(G <= 16 && PK % 4 == 0 && MD % 4 == 0, "tiling");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r16 = lane % 16, grp = lane / 16;
  const int64_t i = a.pos.p[b];
  const int64_t lw = window_left(i, a.S, a.W);
  const int64_t bg = (int64_t)b * a.Hkv + g;
  const float sl2 = a.scale * kLog2e;
  const bool hcol = r16 < G;                 // this lane's column is a real head
  const int h = g * G + (hcol ? r16 : 0);
  const T* kc = static_cast<const T*>(a.kc) + (bg * a.Lcap + c * kS) * D;
  const T* vc = static_cast<const T*>(a.vc) + (bg * a.Lcap + c * kS) * D;
  const T* kn = static_cast<const T*>(a.k_new) + bg * D;
  const T* vn = static_cast<const T*>(a.v_new) + bg * D;
  const int64_t j0 = c * kS;
  const bool last = is_win && c == i / kS;   // the chunk holding the new row
  const int tn = (int)(i - j0);              // its position in that chunk

  // every load up front: K fragments (row = token 16 wave + r16), V pieces
  // (token = lane), Q^T fragments (column r16 = head)
  Frag<T> kf[KS], bq[KS];
  {
    const int t = 16 * wave + r16;
    const T* kr = (last && t == tn) ? kn : kc + (int64_t)t * D;
#pragma unroll
    for (int kq = 0; kq < KS; ++kq) {
      if (!last || t <= tn) load_frag(kf[kq], kr + 8 * grp + 32 * kq);
      else zero_frag(kf[kq]);
    }
  }
  uint4 vr[VPW];
  {
    const T* vrow = (last && lane == tn) ? vn : vc + (int64_t)lane * D;
#pragma unroll
    for (int t = 0; t < VPW; ++t)
      vr[t] = (!last || lane <= tn) ? *reinterpret_cast<const uint4*>(vrow + (wave * VPW + t) * EPV)
                                    : make_uint4(0u, 0u, 0u, 0u);
  }
  {
    const T* qrow = static_cast<const T*>(a.q) + ((int64_t)b * a.Hq + h) * D + 8 * grp;
#pragma unroll
    for (int kq = 0; kq < KS; ++kq) {
      if (hcol) load_frag(bq[kq], qrow + 32 * kq);
      else zero_frag(bq[kq]);
    }
  }
  if (last && threadIdx.x < PK) {   // append this step's key/value row
    const int64_t row = (bg * a.Lcap + i) * D + threadIdx.x * EPV;
    *reinterpret_cast<uint4*>(static_cast<T*>(a.kc) + row) =
        *reinterpret_cast<const uint4*>(kn + threadIdx.x * EPV);
    *reinterpret_cast<uint4*>(static_cast<T*>(a.vc) + row) =
        *reinterpret_cast<const uint4*>(vn + threadIdx.x * EPV);
  }
  const float lnw_sel = (!is_win && hcol) ? lnw[r16] : 0.f;

  // S^T tile of tokens 16 wave + (4 grp + q4), column r16
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kq = 0; kq < KS; ++kq) mma(acc, kf[kq], bq[kq]);
  float x[4], mx = kNegInf;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int64_t j = j0 + 16 * wave + 4 * grp + q4;
    const bool ok = !is_win || (j >= lw && j <= i);
    x[q4] = ok ? acc[q4] * sl2 : kNegInf;
    mx = fmaxf(mx, x[q4]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
  mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
  if (grp == 0) sm.red[0][wave][r16] = mx;
  // V transposed into LDS: row d, token = lane
#pragma unroll
  for (int t = 0; t < VPW; ++t) {
    const T* xv = reinterpret_cast<const T*>(&vr[t]);
    const int d0 = (wave * VPW + t) * EPV;
#pragma unroll
    for (int e = 0; e < EPV; ++e) sm.vt[swz<PV>(d0 + e, lane / EPV) * EPV + lane % EPV] = xv[e];
  }
  __syncthreads();
  const float m = fmaxf(fmaxf(sm.red[0][0][r16], sm.red[0][1][r16]), fmaxf(sm.red[0][2][r16], sm.red[0][3][r16]));
  float p[4], ps = 0.f;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    p[q4] = hw_exp2(x[q4] - m);   // every item has an unmasked token for every head
    ps += p[q4];
  }
  ps += __shfl_xor(ps, 16, kWave);
  ps += __shfl_xor(ps, 32, kWave);
  if (grp == 0) sm.red[1][wave][r16] = ps;
  {
    T* prow = sm.pt + r16 * kS + 16 * wave + 4 * grp;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) prow[q4] = from_f<T>(p[q4]);
  }
  __syncthreads();
  const float l = (sm.red[1][0][r16] + sm.red[1][1][r16]) + (sm.red[1][2][r16] + sm.red[1][3][r16]);

  // O^T tiles: dims 16 md + 4 grp + q4, column r16
  f32x4_t o[MDW];
#pragma unroll
  for (int t = 0; t < MDW; ++t) {
    const int md = wave + 4 * t;
    o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k2 = 0; k2 < kS / 32; ++k2) {
      Frag<T> af, pf;
      load_frag_swz<PV>(af, sm.vt, 16 * md + r16, 8 * grp + 32 * k2);
      load_frag(pf, sm.pt + r16 * kS + 8 * grp + 32 * k2);
      mma(o[t], af, pf);
    }
  }
  // partial: log-weight (natural log) and the normalised output
  if (hcol) {
    float* ap = a.w.apart + ((bg * a.w.nitems + slot) * G + r16) * (D + 2);
    const float inv = 1.f / l;
#pragma unroll
    for (int t = 0; t < MDW; ++t)
      *reinterpret_cast<float4*>(ap + 16 * (wave + 4 * t) + 4 * grp) =
          make_float4(o[t][0] * inv, o[t][1] * inv, o[t][2] * inv, o[t][3] * inv);
    if (wave == 0 && grp == 0) ap[D] = is_win ? (m + hw_log2(l)) * kLn2 : lnw_sel;
  }
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o, kWave));
  return x;
}

// The k-th largest of the keys held J per lane (0 when fewer than k are nonzero),
// bit by bit from the top with ballot counts.
template <int J>
__device__ __forceinline__ uint32_t wave_kth_u32(const uint32_t (&keys)[J], int jn, int k) {
  uint32_t t = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = t | (1u << bit);
    int n = 0;
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (j < jn) n += __popcll(__ballot(keys[j] >= c));
    if (n >= k) t = c;
  }
  return t;
}

// ---------------------------------------------------------------- scoring
struct ListSmem {
  float red[4][2];
  uint32_t wkey[4][64];   // each wave's top-k keys, ascending chunk order
  int32_t wpos[4][64];
  uint32_t sbuf[4][64];
  int nw[4];
  int32_t msel[64];
};

// The slice's outputs for one query row (bh = its (row, head) index): the head's
// LSE partial over the slice, the slice's top-k of s_hat (keys and chunk ids,
// ascending chunk order) and its four largest keys.  sv[j]: the wave's s_hat of
// candidate cw0 + 64 j + lane (-inf where absent).  AGAIN: another row follows
// in the same workgroup (a closing barrier frees the LDS lists).
template <int SJ, bool AGAIN = false>
__device__ __forceinline__ void slice_lists(const DecKArgs& a, ListSmem& sm, int64_t bh, int slice, int64_t c0,
                                            int64_t cw0, int64_t nc, const float (&sv)[SJ]) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int kk = a.w.kk;
  // the head's LSE partial of the slice (log2 units)
  float mw = kNegInf;
#pragma unroll
  for (int j = 0; j < SJ; ++j) mw = fmaxf(mw, sv[j] * kLog2e);
  mw = wave_max(mw);
  float zl = 0.f;
#pragma unroll
  for (int j = 0; j < SJ; ++j) zl += sv[j] == kNegInf ? 0.f : hw_exp2(sv[j] * kLog2e - mw);
  const float zw = wave_sum(zl);
  // this wave's top-k of s_hat (ties: lower chunk), ascending chunk order
  const int nvw = (int)max<int64_t>(0, min<int64_t>(nc - cw0, 64 * SJ));
  uint32_t keys[SJ];
#pragma unroll
  for (int j = 0; j < SJ; ++j) keys[j] = sv[j] == kNegInf ? 0u : order_key(sv[j]);
  const int nl = list_topk<SJ>(keys, (nvw + 63) / 64, nvw, kk, lane, sm.sbuf[wave], sm.wpos[wave],
                               sm.wkey[wave]);
  if (lane == 0) {
    sm.red[wave][0] = mw;
    sm.red[wave][1] = zw;
    sm.nw[wave] = nl;
  }
  __syncthreads();
  if (wave == 0) {
  if (lane == 0) {
    float M = kNegInf, Z = 0.f;
    for (int w = 0; w < 4; ++w) lse_merge(M, Z, sm.red[w][0], sm.red[w][1]);
    a.w.lpart[bh * a.w.nslice + slice] = make_float2(M, Z);
  }
  // merge the four wave lists: entry e of wave w's list sits at position
  // 64 jj + lane with w = LPJ jj + lane / TP, e = lane % TP (ascending chunk order)
  const int TP = kk <= 16 ? 16 : (kk <= 32 ? 32 : 64);
  const int LPJ = kWave / TP;
  const int ml = lane / TP, me = lane % TP;
  uint32_t mk[4];
  int tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) tot += sm.nw[w];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int w = LPJ * jj + ml;
    mk[jj] = (w < 4 && me < sm.nw[w]) ? sm.wkey[w][me] : 0u;
  }
  const int jn = (4 + LPJ - 1) / LPJ;
  int32_t* mpos = sm.msel;
  uint32_t* mkey = sm.sbuf[1];   // wave 1's buffer is free once the lists are merged
  const int n = list_topk<4>(mk, jn, tot, kk, lane, sm.sbuf[0], mpos, mkey);
  wave_lds_sync();
  if (lane < kk) {
    uint32_t key = 0u;
    int32_t id = -1;
    if (lane < n) {
      const int ps = mpos[lane];
      const int w = LPJ * (ps / 64) + (ps % 64) / TP, e = (ps % 64) % TP;
      key = mkey[lane];
      id = (int32_t)(c0 + (int64_t)w * 64 * SJ + sm.wpos[w][e]);
    }
    const int64_t o = (bh * a.w.nslice + slice) * kk + lane;
    a.w.lkey[o] = key;
    a.w.lid[o] = id;
  }
  // the slice's four largest keys: the selection prunes the lists with them
  uint32_t x = lane < n ? mkey[lane] : 0u;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t m = wave_max_u32(x);
    if (lane == 0) a.w.lk4[(bh * a.w.nslice + slice) * 4 + r] = m;
    const uint64_t at = __ballot(x == m && m != 0u);
    if (at && lane == __ffsll((long long)at) - 1) x = 0u;
  }
  }
  if constexpr (AGAIN) __syncthreads();   // the LDS lists are used again by the next row
}

// A slice of 256*SJ candidates of one (b, head): wave w streams candidates
// [c0 + 64 SJ w, + 64 SJ) in SJ blocks of 64.  PPR lanes cover one k' row with
// 16-byte pieces, so one load instruction reads RPI consecutive rows; each lane
// multiplies its piece by the matching piece of q_hat and a butterfly over the
// PPR lanes of a row leaves one row's dot product per lane, which a permute moves
// to lane order (lane l: candidate l of the block).
template <typename T, int D, int SJ>
__device__ __forceinline__ void score_slice(const DecKArgs& a, ListSmem& sm, int sblk) {
  constexpr int EPV = 16 / sizeof(T);
  constexpr int PPR = D / EPV;        // lanes per k' row
  constexpr int RPI = kWave / PPR;    // rows per load instruction
  constexpr int NI = PPR;             // load instructions per 64 rows
  const int slice = sblk % a.w.nslice;
  const int h = (sblk / a.w.nslice) % a.Hq;
  const int b = sblk / (a.w.nslice * a.Hq);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int64_t i = a.pos.p[b];
  const int64_t nc = num_candidates(i, a.S, a.W);
  const int64_t c0 = (int64_t)slice * (kThreads * SJ);
  if (c0 >= nc) return;                                 // the selection reads slices < nc only
  const int64_t bh = (int64_t)b * a.Hq + h;
  const int kk = a.w.kk;
  const int pc = lane % PPR, rg = lane / PPR;
  float qv[EPV];
  {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.qh) + bh * D + pc * EPV);
    const T* t = reinterpret_cast<const T*>(&u);
#pragma unroll
    for (int e = 0; e < EPV; ++e) qv[e] = to_f<T>(t[e]);
  }
  const int64_t cw0 = c0 + (int64_t)wave * 64 * SJ;     // this wave's first candidate
  const T* kb = static_cast<const T*>(a.ksum) + (bh * a.NCcap + cw0) * D + pc * EPV;
  const int src = (lane % RPI) * PPR + lane / RPI;      // lane holding row `lane`'s dot product
  // Loads go out in batches of NB, two batches ahead of the arithmetic, so every
  // wave keeps a steady number of loads in flight across its SJ blocks.
  constexpr int NB = NI >= 8 ? NI / 2 : NI;             // loads per batch
  constexpr int NBS = NI / NB;                          // batches per block of 64 rows
  constexpr int NBAT = NBS * SJ;
  auto issue = [&](int q, uint4 (&u)[NB]) {
    const int j = q / NBS, t0 = (q % NBS) * NB;
    const int64_t cb = cw0 + 64 * j;
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const int row = RPI * (t0 + t) + rg;
      u[t] = cb + row < nc ? *reinterpret_cast<const uint4*>(kb + (int64_t)(64 * j + row) * D)
                           : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  float bv[SJ];
#pragma unroll
  for (int j = 0; j < SJ; ++j) {
    const int64_t c = cw0 + 64 * j + lane;
    bv[j] = c < nc ? a.bsum[bh * a.NCcap + c] : 0.f;
  }
  uint4 buf[2][NB];
  issue(0, buf[0]);
  if (NBAT > 1) issue(1, buf[1]);
  float sv[SJ];
  float v[NI];
#pragma unroll
  for (int q = 0; q < NBAT; ++q) {
    const int t0 = (q % NBS) * NB;
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const T* x = reinterpret_cast<const T*>(&buf[q % 2][t]);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc = fmaf(qv[e], to_f<T>(x[e]), acc);
      v[t0 + t] = acc;
    }
    if (q + 2 < NBAT) issue(q + 2, buf[q % 2]);
    // keep the loads where they are: hoisting every block's loads to the top
    // would hold all of them in registers at once
    __builtin_amdgcn_sched_barrier(0);
    if (q % NBS == NBS - 1) {   // a block of 64 rows is complete
      const int j = q / NBS;
      float w[NI];
#pragma unroll
      for (int t = 0; t < NI; ++t) w[t] = v[t];
      butterfly<PPR / 2, NI>(w, lane);
      const float dot = __shfl(w[0], src, kWave);
      const int64_t c = cw0 + 64 * j + lane;
      const bool ok = c < nc;
      const float sc = fmaf(dot, a.scale, bv[j]);
      if (ok) a.w.shat[bh * a.NCcap + c] = sc;
      sv[j] = ok ? sc : kNegInf;
    }
  }
  slice_lists<SJ>(a, sm, bh, slice, c0, cw0, nc, sv);
}

template <typename T, int D>
union ScoreSmem {
  ItemSmem<T, D> it;
  ListSmem l;
};

template <typename T, int D, int G, int SJ>
__global__ __launch_bounds__(kThreads) void dec_score_kernel(DecKArgs a) {
  __shared__ __align__(16) ScoreSmem<T, D> sm;
  // scoring blocks first: the window blocks fill the tail of the k' stream
  const int nsb = a.B * a.Hq * a.w.nslice;
  if ((int)blockIdx.x >= nsb) {   // a window item: chunk lw/S + w of (b, g)
    const int x = (int)blockIdx.x - nsb;
    const int w = x % a.w.nwin;
    const int g = (x / a.w.nwin) % a.Hkv;
    const int b = x / (a.w.nwin * a.Hkv);
    const int64_t i = a.pos.p[b];
    const int64_t lw = window_left(i, a.S, a.W);
    if (w > (int)(i / kS - lw / kS)) return;
    attend_item<T, D, G>(a, sm.it, b, g, a.w.kk + w, lw / kS + w, true, nullptr);
    return;
  }
  score_slice<T, D, SJ>(a, sm.l, (int)blockIdx.x);
}

// ---------------------------------------------------------------- selection
// Two stages, spread over many workgroups (one compute unit per (b, group)
// would run thousands of ballot steps while the rest of the chip idles):
//  dec_headsel  one wave per (b, head, share of kSPS slices): the share's top-k
//               of s_hat from its slices' lists (entry e of slice s at position
//               s*kk + e: ascending chunk order).  The share's k-th largest key is
//               at least theta, the k-th largest of its slices' four largest keys
//               (at least k entries reach theta), so entries below theta cannot
//               be chosen: when few reach it, the exact top-k runs on those
//               survivors (compacted in position order), otherwise on every
//               entry.  The first share's wave also forms L_h from the slice
//               partials.
//  dec_attend   each workgroup of a (b, group) forms the group's selection in
//               its prologue, the same in every workgroup: each head's top-k
//               from its share lists; for one head that is the selection,
//               otherwise the union of the heads' choices is marked in an LDS
//               bitmap over the candidates, listed in ascending chunk order with
//               a block prefix count, each member's rank key
//               r = max_h (s_hat_h - L_h) is formed from every head's s_hat, and
//               wave 0 takes the top-k of the union by r.  The workgroup then
//               attends the chunk of its slot.
constexpr int kSPS = 32;          // slices per share
constexpr int kMaxShares = 8;     // shares per head (<= kSPS * kMaxShares slices)
constexpr int kDirectJ = 16;      // list entries per lane when the group selection ranks
                                  // a head's slice lists itself (<= 1024 entries)
constexpr int kMaxUnion = 8 * 64;

// Entries present in slices [s0, s1) of a head: min(kk, candidates) each.
__device__ __forceinline__ int slice_entries(int64_t nc, int slen, int kk, int s0, int s1) {
  int n = 0;
  for (int s = s0; s < s1; ++s) n += (int)min<int64_t>(kk, min<int64_t>(slen, nc - (int64_t)s * slen));
  return n;
}

struct HeadSelSmem {
  uint32_t sbuf[64];
  uint32_t pkey[128];
  int32_t ppos[128];
  int32_t opos[64];
  uint32_t okey[64];
};

// The natural-log LSE of the lanes' (max, sum) partials in log2 units.
__device__ __forceinline__ float wave_lse(float M, float Z) {
  const float Mw = wave_max(M);
  const float Zw = wave_sum(M == kNegInf ? 0.f : Z * hw_exp2(M - Mw));
  return (Mw + hw_log2(Zw)) * kLn2;
}

// Head bh's LSE over its candidates, from the slice partials (one wave).
__device__ __forceinline__ float head_lse(const DecKArgs& a, int64_t bh, int ns, int lane) {
  const float2* lp = a.w.lpart + bh * a.w.nslice;
  float M = kNegInf, Z = 0.f;
  for (int s = lane; s < ns; s += kWave) lse_merge(M, Z, lp[s].x, lp[s].y);
  return wave_lse(M, Z);
}

// One wave: the top-k of s_hat of head bh over the lists of slices [s0, s1)
// (entry e of slice s at position (s - s0) kk + e: ascending chunk order).  The
// share's k-th largest key is at least theta, the k-th largest of its slices'
// four largest keys (at least k entries reach theta), so entries below theta
// cannot be chosen: when few reach it, the exact top-k runs on those survivors
// (compacted in position order), otherwise on every entry.  Leaves the chosen
// entries' positions in sm.opos and keys in sm.okey (ascending chunk order) and
// returns their number; with IDS, their chunk ids go to oid as well (the ids are
// loaded with the keys and picked by lane permutes, saving a dependent gather).
// MJ >= entries / 64.
template <int MJ, bool IDS = false>
__device__ __forceinline__ int share_topk(const DecKArgs& a, HeadSelSmem& sm, int64_t bh, int s0, int s1,
                                          int64_t nc, int lane, int32_t* oid = nullptr) {
  const int topk = a.topk, kk = a.w.kk;
  const int slen = kThreads * a.w.sj;
  const int64_t lbase = (bh * a.w.nslice + s0) * kk;
  const int nent = (s1 - s0) * kk;
  const int jn = (nent + 63) / 64;
  uint32_t keys[MJ];
  int32_t ids[IDS ? MJ : 1];
#pragma unroll
  for (int j = 0; j < MJ; ++j) {
    const int p = lane + 64 * j;
    const bool in = j < jn && p < nent;
    keys[j] = in ? a.w.lkey[lbase + p] : 0u;
    if constexpr (IDS) ids[j] = in ? a.w.lid[lbase + p] : -1;
  }
  uint32_t pool[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = lane + 64 * j;
    pool[j] = p < 4 * (s1 - s0) ? a.w.lk4[(bh * a.w.nslice + s0) * 4 + p] : 0u;
  }
  const int npw = slice_entries(nc, slen, kk, s0, s1);
  int nl = -1;
  if (npw > topk) {
    const uint32_t theta = wave_kth_u32<2>(pool, 2, topk);
    int nsv = 0;
#pragma unroll
    for (int j = 0; j < MJ; ++j)
      if (j < jn) nsv += __popcll(__ballot(theta != 0u && keys[j] >= theta));
    if (theta != 0u && nsv <= 128) {
      int base = 0;
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        if (j < jn) {
          const bool sv = keys[j] >= theta;
          const uint64_t msk = __ballot(sv);
          if (sv) {
            const int ps = base + lane_prefix(msk, lane);
            sm.pkey[ps] = keys[j];
            sm.ppos[ps] = lane + 64 * j;
          }
          base += __popcll(msk);
        }
      }
      wave_lds_sync();
      uint32_t k2[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) k2[j] = lane + 64 * j < nsv ? sm.pkey[lane + 64 * j] : 0u;
      nl = list_topk<2>(k2, nsv <= 64 ? 1 : 2, nsv, topk, lane, sm.sbuf, sm.opos, sm.okey);
      wave_lds_sync();
      if (lane < nl) sm.opos[lane] = sm.ppos[sm.opos[lane]];
    }
  }
  if (nl < 0) nl = list_topk<MJ>(keys, jn, npw, topk, lane, sm.sbuf, sm.opos, sm.okey);
  if constexpr (IDS) {
    wave_lds_sync();
    const int p = lane < nl ? sm.opos[lane] : 0;
    int32_t id = -1;
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
      if (j < jn) {
        const int32_t v = __shfl(ids[j], p % 64, kWave);
        if (p / 64 == j) id = v;
      }
    }
    if (lane < nl) oid[lane] = id;
  }
  return nl;
}

template <int MJ>
__global__ __launch_bounds__(64) void dec_headsel_kernel(DecKArgs a) {
  __shared__ HeadSelSmem sm;
  const int q = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int64_t i = a.pos.p[b];
  const int64_t nc = num_candidates(i, a.S, a.W);
  const int topk = a.topk, kk = a.w.kk;
  if (nc <= topk) return;                 // every candidate is chosen: nothing to rank
  const int slen = kThreads * a.w.sj;
  const int ns = (int)((nc + slen - 1) / slen);
  const int s0 = q * kSPS;
  if (s0 >= ns) return;
  const int s1 = min(ns, s0 + kSPS);
  const int64_t bh = (int64_t)b * a.Hq + h;
  if (q == 0) {   // the head's LSE from the slice partials
    const float L = head_lse(a, bh, ns, lane);
    if (lane == 0) a.w.Lh[bh] = L;
  }
  const int nl = share_topk<MJ>(a, sm, bh, s0, s1, nc, lane);
  wave_lds_sync();
  if (lane < kk) {
    const int64_t o = (bh * kMaxShares + q) * kk + lane;
    a.w.hkey[o] = lane < nl ? sm.okey[lane] : 0u;
    a.w.hid[o] = lane < nl ? a.w.lid[(bh * a.w.nslice + s0) * kk + sm.opos[lane]] : -1;
  }
}

struct GroupSelSmem {
  float L[8];
  uint32_t sbuf[4][64];
  int32_t hpos[4][64];
  uint32_t hkey[8][64];
  int32_t hid[8][64];
  int nh[8];
  int32_t ulist[kMaxUnion];
  uint32_t ukey[kMaxUnion];
  int32_t scan[4];
  int32_t osel[64];
  int32_t chosen[64];
  float lnw[8];
  HeadSelSmem hs[4];   // per wave, when the heads' lists are ranked here
};

// The group's selection (ascending chunk ids in sm.chosen[0..min(nc, k))) and, for
// slot `slot`, each head's s_hat in sm.lnw.  Every workgroup of (b, g) forms the
// same selection; the one of slot 0 writes it to idx_out.
template <int G>
__device__ void group_select(const DecKArgs& a, GroupSelSmem& sm, uint32_t* bitmap, int b, int g,
                             int slot) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int64_t i = a.pos.p[b];
  const int64_t nc = num_candidates(i, a.S, a.W);
  const int topk = a.topk, kk = a.w.kk;
  auto shat = [&](int hh, int64_t c) { return a.w.shat[((int64_t)b * a.Hq + g * G + hh) * a.NCcap + c]; };
  if (nc <= topk) {   // every candidate is chosen
    for (int t = threadIdx.x; t < topk; t += kThreads) sm.chosen[t] = t < nc ? t : -1;
  } else {
    const int slen = kThreads * a.w.sj;
    const int ns = (int)((nc + slen - 1) / slen);
    const int nsh = (ns + kSPS - 1) / kSPS;
    // each head's top-k: from its slices' lists directly when they form one
    // share (no head-selection kernel ran), else from its share lists (share q:
    // position q*kk + e)
    for (int hh = wave; hh < G; hh += kThreads / kWave) {
      const int64_t bh = (int64_t)b * a.Hq + g * G + hh;
      if (a.w.direct) {
        // the slice partials are loaded first, so their latency overlaps the ranking
        const float2 lp = lane < ns ? a.w.lpart[bh * a.w.nslice + lane] : make_float2(kNegInf, 0.f);
        const int n = share_topk<kDirectJ, true>(a, sm.hs[wave], bh, 0, ns, nc, lane, sm.hid[hh]);
        const float L = wave_lse(lp.x, lp.y);   // ns <= kSPS <= 64: one partial per lane
        if (lane == 0) {
          sm.nh[hh] = n;
          sm.L[hh] = L;
        }
        wave_lds_sync();
        continue;
      }
      const int64_t hb = bh * kMaxShares * kk;
      constexpr int JH = kMaxShares;   // kk <= 64 keys per share
      uint32_t keys[JH];
      int npres = 0;
#pragma unroll
      for (int j = 0; j < JH; ++j) {
        const int p = lane + 64 * j;
        keys[j] = p < nsh * kk ? a.w.hkey[hb + p] : 0u;
      }
      for (int q = 0; q < nsh; ++q)
        npres += min(kk, slice_entries(nc, slen, kk, q * kSPS, min(ns, (q + 1) * kSPS)));
      const int n = list_topk<JH>(keys, (nsh * kk + 63) / 64, npres, topk, lane, sm.sbuf[wave],
                                  sm.hpos[wave], sm.hkey[hh]);
      wave_lds_sync();
      if (lane < n) sm.hid[hh][lane] = a.w.hid[hb + sm.hpos[wave][lane]];
      if (lane == 0) {
        sm.nh[hh] = n;
        sm.L[hh] = a.w.Lh[bh];
      }
      wave_lds_sync();
    }
    __syncthreads();
    if constexpr (G == 1) {
      for (int t = threadIdx.x; t < topk; t += kThreads) sm.chosen[t] = sm.hid[0][t];   // nh = topk
    } else {
      // union of the heads' choices, in ascending chunk order
      const int nwords = (int)((nc + 31) / 32);
      for (int t = threadIdx.x; t < nwords; t += kThreads) bitmap[t] = 0u;
      __syncthreads();
      for (int t = threadIdx.x; t < G * 64; t += kThreads) {
        const int hh = t / 64, e = t % 64;
        if (e < sm.nh[hh]) {
          const int32_t c = sm.hid[hh][e];
          atomicOr(&bitmap[c >> 5], 1u << (c & 31));
        }
      }
      __syncthreads();
      const int wpt = (nwords + kThreads - 1) / kThreads;
      const int w0 = min(nwords, (int)threadIdx.x * wpt), w1 = min(w0 + wpt, nwords);
      int cnt = 0;
      for (int t = w0; t < w1; ++t) cnt += __popc(bitmap[t]);
      int incl = cnt;   // block prefix count: within the wave, then over the waves
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
      }
      if (lane == kWave - 1) sm.scan[wave] = incl;
      __syncthreads();
      int pos = incl - cnt, nu = 0;
#pragma unroll
      for (int w = 0; w < kThreads / kWave; ++w) {
        pos += w < wave ? sm.scan[w] : 0;
        nu += sm.scan[w];
      }
      for (int t = w0; t < w1; ++t) {
        uint32_t m = bitmap[t];
        while (m) {
          const int bit = __ffs(m) - 1;
          m &= m - 1u;
          sm.ulist[pos++] = t * 32 + bit;
        }
      }
      __syncthreads();   // nu >= topk: each head chose topk distinct chunks
      for (int u = threadIdx.x; u < nu; u += kThreads) {
        const int32_t c = sm.ulist[u];
        float r = kNegInf;
#pragma unroll
        for (int h2 = 0; h2 < G; ++h2) r = fmaxf(r, shat(h2, c) - sm.L[h2]);
        sm.ukey[u] = order_key(r);
      }
      __syncthreads();
      if (wave == 0) {
        constexpr int JU = kMaxUnion / 64;
        uint32_t uk[JU];
#pragma unroll
        for (int j = 0; j < JU; ++j) {
          const int u = lane + 64 * j;
          uk[j] = u < nu ? sm.ukey[u] : 0u;
        }
        const int n = list_topk<JU>(uk, (nu + 63) / 64, nu, topk, lane, sm.sbuf[0], sm.osel, sm.hkey[0]);
        wave_lds_sync();
        if (lane < topk) sm.chosen[lane] = lane < n ? sm.ulist[sm.osel[lane]] : -1;
      }
    }
  }
  __syncthreads();
  if (slot == 0 && a.idx_out) {
    const int64_t bg = (int64_t)b * a.Hkv + g;
    for (int t = threadIdx.x; t < topk; t += kThreads) a.idx_out[bg * topk + t] = sm.chosen[t];
  }
  const int32_t c = sm.chosen[slot];
  if ((int)threadIdx.x < G) sm.lnw[threadIdx.x] = c >= 0 ? shat((int)threadIdx.x, c) : 0.f;
  __syncthreads();
}

// ---------------------------------------------------------------- selected items
template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads) void dec_attend_kernel(DecKArgs a) {
  __shared__ __align__(16) ItemSmem<T, D> it;
  __shared__ GroupSelSmem sel;
  extern __shared__ uint32_t bitmap[];   // ceil(candidates / 32) words
  const int slot = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int64_t i = a.pos.p[b];
  const int64_t nc = num_candidates(i, a.S, a.W);
  if (slot >= (int)min<int64_t>(nc, a.topk)) {
    if (slot == 0 && a.idx_out)   // no candidate yet: the selection is all padding
      for (int t = threadIdx.x; t < a.topk; t += kThreads)
        a.idx_out[((int64_t)b * a.Hkv + g) * a.topk + t] = -1;
    return;
  }
  group_select<G>(a, sel, bitmap, b, g, slot);
  attend_item<T, D, G>(a, it, b, g, slot, sel.chosen[slot], false, sel.lnw);
}

// ---------------------------------------------------------------- fusion
// One workgroup of kFuseWaves waves per (b, query head): the output is the
// average of the items' normalised outputs weighted by exp(log-weight), and L
// the log of the total weight (the LSE over the selected chunks' s_hat and the
// window's log-mass).  The weights take one item per thread; wave w sums every
// kFuseWaves-th item and the waves' sums meet in LDS.
constexpr int kFuseWaves = 4;
static_assert(64 * kFuseWaves >= 256, "one thread per item (at most 256 items)");
template <typename T, int D, int G>
__global__ __launch_bounds__(64 * kFuseWaves) void dec_fuse_kernel(DecKArgs a) {
  constexpr int DPL = D / kWave;
  __shared__ float wts[256];
  __shared__ float red[kFuseWaves][D];
  __shared__ float mz[kFuseWaves][2];
  const int h = blockIdx.x, b = blockIdx.y;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int g = h / G, hl = h % G;
  const int64_t i = a.pos.p[b];
  const int64_t lw = window_left(i, a.S, a.W);
  const int nsel = (int)min<int64_t>(lw / kS, a.topk);
  const int nitems = nsel + (int)(i / kS - lw / kS + 1);   // <= 256 (checked on the host)
  const int64_t bg = (int64_t)b * a.Hkv + g;
  const float* ap = a.w.apart + (bg * a.w.nitems * G + hl) * (D + 2);
  const int kk = a.w.kk;
  auto slot_of = [&](int it) { return it < nsel ? it : kk + (it - nsel); };
  // item weights exp(lw_item - max): one item per thread, block max and sum
  const int it0 = threadIdx.x;
  const float lwi = it0 < nitems ? ap[(int64_t)slot_of(it0) * G * (D + 2) + D] : kNegInf;
  float mx = wave_max(lwi);
  if (lane == 0) mz[wave][0] = mx;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kFuseWaves; ++w) mx = fmaxf(mx, mz[w][0]);
  const float wi = it0 < nitems ? __expf(lwi - mx) : 0.f;
  wts[it0] = wi;
  const float zw = wave_sum(wi);
  if (lane == 0) mz[wave][1] = zw;
  __syncthreads();
  float z = 0.f;
#pragma unroll
  for (int w = 0; w < kFuseWaves; ++w) z += mz[w][1];
  // wave w sums items w, w + kFuseWaves, ..., eight loads in flight per lane
  float res[DPL];
#pragma unroll
  for (int t = 0; t < DPL; ++t) res[t] = 0.f;
  constexpr int U = 8;
  for (int itb = wave; itb < nitems; itb += U * kFuseWaves) {
    float x[U][DPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = itb + u * kFuseWaves;
      const float* pp = ap + (int64_t)slot_of(min(it, nitems - 1)) * G * (D + 2) + lane * DPL;
#pragma unroll
      for (int t = 0; t < DPL; ++t) x[u][t] = pp[t];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = itb + u * kFuseWaves;
      const float w = it < nitems ? wts[it] : 0.f;
#pragma unroll
      for (int t = 0; t < DPL; ++t) res[t] = fmaf(w, x[u][t], res[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < DPL; ++t) red[wave][lane * DPL + t] = res[t];
  __syncthreads();
  if (wave != 0) return;
  const float inv = 1.f / z;
  T* orow = static_cast<T*>(a.out) + ((int64_t)b * a.Hq + h) * D;
#pragma unroll
  for (int t = 0; t < DPL; ++t) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kFuseWaves; ++w) v += red[w][lane * DPL + t];
    orow[lane * DPL + t] = from_f<T>(v * inv);
  }
  if (a.lse && lane == 0) a.lse[(int64_t)b * a.Hq + h] = mx + __logf(z);
}


// ---------------------------------------------------------------- several queries
// M adjacent queries per sequence (speculative or multi-token decoding; the
// paper-body page's kernel design: adjacent queries attend the union of their
// selected chunks, which fills the matrix tiles with M x G rows and loads each
// chunk once for all of them).  Row v = b M + m is the prefill row
// i = pos[b] + m: the M new key/value rows go to the caches first, every query
// scores all its candidates (each k' row is read once for up to four queries of
// a sequence), selection runs per row as for one query, and the attention takes
// one workgroup per chunk of the union of the M selections of (b, group), the
// M G (query, head) pairs as the 16 columns of the tiles, each column masked to
// the chunks it selected (or, for window chunks, to its own window).

// The new rows into the caches (one workgroup per (row, KV head)).
template <typename T, int D>
__global__ __launch_bounds__(64) void dec_append_kernel(DecKArgs a) {
  constexpr int EPV = 16 / sizeof(T);
  const int g = blockIdx.x, v = blockIdx.y;
  const int br = v / a.M;
  const int64_t row = (((int64_t)br * a.Hkv + g) * a.Lcap + a.pos.p[v]) * D;
  const int64_t src = ((int64_t)v * a.Hkv + g) * D;
  for (int p = threadIdx.x; p < D / EPV; p += 64) {
    *reinterpret_cast<uint4*>(static_cast<T*>(a.kc) + row + p * EPV) =
        *reinterpret_cast<const uint4*>(static_cast<const T*>(a.k_new) + src + p * EPV);
    *reinterpret_cast<uint4*>(static_cast<T*>(a.vc) + row + p * EPV) =
        *reinterpret_cast<const uint4*>(static_cast<const T*>(a.v_new) + src + p * EPV);
  }
}

// One chunk c of (b, group g) for every (query, head) column col = m G + hh of
// the group's M G pairs: as attend_item, with the keys and values read from the
// caches (rows past the group's last position read as zero), and each column's
// tokens masked to its window (is_win) or to all of c when bit m of `member`
// is set (the chunk is then slot memslot[m] of row m's selection).  A window
// column with no token gets log-weight -inf and a zero output.
template <typename T, int D, int G>
__device__ __forceinline__ void attend_item_mq(const DecKArgs& a, ItemSmem<T, D>& sm, int br, int g, int win_slot,
                                               int64_t c, bool is_win, uint32_t member, const int* memslot) {
  constexpr int EPV = 16 / sizeof(T);
  constexpr int KS = D / 32, MD = D / 16;
  constexpr int PK = D / EPV, PV = kS / EPV;
  constexpr int VPW = PK / 4;
  constexpr int MDW = MD / 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r16 = lane % 16, grp = lane / 16;
  const int M = a.M;
  const bool hcol = r16 < M * G;
  const int m = hcol ? r16 / G : 0, hh = r16 % G;
  const int v = br * M + m;
  const int64_t i = a.pos.p[v];
  const int64_t lw = window_left(i, a.S, a.W);
  const int64_t ilast = a.pos.p[br * M + M - 1];   // the group's last written row
  const int64_t bg = (int64_t)br * a.Hkv + g;
  const float sl2 = a.scale * kLog2e;
  const T* kc = static_cast<const T*>(a.kc) + (bg * a.Lcap + c * kS) * D;
  const T* vc = static_cast<const T*>(a.vc) + (bg * a.Lcap + c * kS) * D;
  const int64_t j0 = c * kS;
  const bool colon = hcol && (is_win || ((member >> m) & 1u));
  Frag<T> kf[KS], bq[KS];
  {
    const int t = 16 * wave + r16;
    const bool ok = j0 + t <= ilast;
#pragma unroll
    for (int kq = 0; kq < KS; ++kq) {
      if (ok) load_frag(kf[kq], kc + (int64_t)t * D + 8 * grp + 32 * kq);
      else zero_frag(kf[kq]);
    }
  }
  uint4 vr[VPW];
  {
    const bool ok = j0 + lane <= ilast;
#pragma unroll
    for (int t = 0; t < VPW; ++t)
      vr[t] = ok ? *reinterpret_cast<const uint4*>(vc + (int64_t)lane * D + (wave * VPW + t) * EPV)
                 : make_uint4(0u, 0u, 0u, 0u);
  }
  {
    const T* qrow = static_cast<const T*>(a.q) + ((int64_t)v * a.Hq + g * G + hh) * D + 8 * grp;
#pragma unroll
    for (int kq = 0; kq < KS; ++kq) {
      if (colon) load_frag(bq[kq], qrow + 32 * kq);
      else zero_frag(bq[kq]);
    }
  }
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kq = 0; kq < KS; ++kq) mma(acc, kf[kq], bq[kq]);
  float x[4], mx = kNegInf;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int64_t j = j0 + 16 * wave + 4 * grp + q4;
    const bool ok = colon && (!is_win || (j >= lw && j <= i));
    x[q4] = ok ? acc[q4] * sl2 : kNegInf;
    mx = fmaxf(mx, x[q4]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
  mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
  if (grp == 0) sm.red[0][wave][r16] = mx;
#pragma unroll
  for (int t = 0; t < VPW; ++t) {
    const T* xv = reinterpret_cast<const T*>(&vr[t]);
    const int d0 = (wave * VPW + t) * EPV;
#pragma unroll
    for (int e = 0; e < EPV; ++e) sm.vt[swz<PV>(d0 + e, lane / EPV) * EPV + lane % EPV] = xv[e];
  }
  __syncthreads();
  const float mm = fmaxf(fmaxf(sm.red[0][0][r16], sm.red[0][1][r16]), fmaxf(sm.red[0][2][r16], sm.red[0][3][r16]));
  float p[4], ps = 0.f;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    p[q4] = x[q4] == kNegInf ? 0.f : hw_exp2(x[q4] - mm);
    ps += p[q4];
  }
  ps += __shfl_xor(ps, 16, kWave);
  ps += __shfl_xor(ps, 32, kWave);
  if (grp == 0) sm.red[1][wave][r16] = ps;
  {
    T* prow = sm.pt + r16 * kS + 16 * wave + 4 * grp;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) prow[q4] = from_f<T>(p[q4]);
  }
  __syncthreads();
  const float l = (sm.red[1][0][r16] + sm.red[1][1][r16]) + (sm.red[1][2][r16] + sm.red[1][3][r16]);
  f32x4_t o[MDW];
#pragma unroll
  for (int t = 0; t < MDW; ++t) {
    const int md = wave + 4 * t;
    o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k2 = 0; k2 < kS / 32; ++k2) {
      Frag<T> af, pf;
      load_frag_swz<PV>(af, sm.vt, 16 * md + r16, 8 * grp + 32 * k2);
      load_frag(pf, sm.pt + r16 * kS + 8 * grp + 32 * k2);
      mma(o[t], af, pf);
    }
  }
  if (colon) {
    // the column's own slot: its position in its row's selection, or window slot
    const int slot = is_win ? win_slot : memslot[m];
    float* ap = a.w.mpart + ((((int64_t)bg * M + m) * a.w.nitems_mq + slot) * G + hh) * (D + 2);
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int t = 0; t < MDW; ++t)
      *reinterpret_cast<float4*>(ap + 16 * (wave + 4 * t) + 4 * grp) =
          make_float4(o[t][0] * inv, o[t][1] * inv, o[t][2] * inv, o[t][3] * inv);
    if (wave == 0 && grp == 0) {
      float lw_ = kNegInf;
      if (l > 0.f)
        lw_ = is_win ? (mm + hw_log2(l)) * kLn2
                     : a.w.shat[((int64_t)v * a.Hq + g * G + hh) * a.NCcap + c];
      ap[D] = lw_;
    }
  }
  __syncthreads();   // the LDS tiles are free for the caller
}

// Scoring of up to four queries of one sequence per block: (b, query group mg,
// head, slice); each k' row piece is loaded once and dotted with every query.
// Window blocks follow: chunk lw(first query)/S + w of (b, group).
template <typename T, int D, int SJ>
union MScoreSmem {
  ItemSmem<T, D> it;
  struct {
    ListSmem l;
    float svs[4][kThreads * SJ];   // each query's s_hat of the slice
  } s;
};

template <typename T, int D, int G, int SJ>
__global__ __launch_bounds__(kThreads) void dec_mscore_kernel(DecKArgs a) {
  __shared__ __align__(16) MScoreSmem<T, D, SJ> sm;
  constexpr int MQ = 4;
  constexpr int EPV = 16 / sizeof(T);
  constexpr int PPR = D / EPV;
  constexpr int RPI = kWave / PPR;
  constexpr int NI = PPR;
  const int Br = a.B / a.M;
  const int nmg = (a.M + MQ - 1) / MQ;
  const int nsb = Br * nmg * a.Hq * a.w.nslice;
  if ((int)blockIdx.x >= nsb) {
    const int x = (int)blockIdx.x - nsb;
    const int w = x % a.w.nwin_mq;
    const int g = (x / a.w.nwin_mq) % a.Hkv;
    const int br = x / (a.w.nwin_mq * a.Hkv);
    const int64_t cfirst = window_left(a.pos.p[br * a.M], a.S, a.W) / kS;
    const int64_t clast = a.pos.p[br * a.M + a.M - 1] / kS;
    if (cfirst + w > clast) return;
    attend_item_mq<T, D, G>(a, sm.it, br, g, a.w.kk + w, cfirst + w, true, 0u, nullptr);
    return;
  }
  const int slice = (int)blockIdx.x % a.w.nslice;
  const int h = ((int)blockIdx.x / a.w.nslice) % a.Hq;
  const int mg = ((int)blockIdx.x / (a.w.nslice * a.Hq)) % nmg;
  const int br = (int)blockIdx.x / (a.w.nslice * a.Hq * nmg);
  const int m0 = mg * MQ;
  const int mn = min(MQ, a.M - m0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  int64_t ncm[MQ];
#pragma unroll
  for (int u = 0; u < MQ; ++u) ncm[u] = u < mn ? num_candidates(a.pos.p[br * a.M + m0 + u], a.S, a.W) : 0;
  const int64_t nc = ncm[mn - 1];   // the group's last query has the most candidates
  const int64_t c0 = (int64_t)slice * (kThreads * SJ);
  if (c0 >= nc) return;
  const int64_t bhr = (int64_t)br * a.Hq + h;   // k', b' of the real sequence
  const int pc = lane % PPR, rg = lane / PPR;
  float qv[MQ][EPV];
#pragma unroll
  for (int u = 0; u < MQ; ++u) {
    const int v = br * a.M + m0 + min(u, mn - 1);
    const uint4 q4 = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.qh) +
                                                    ((int64_t)v * a.Hq + h) * D + pc * EPV);
    const T* t = reinterpret_cast<const T*>(&q4);
#pragma unroll
    for (int e = 0; e < EPV; ++e) qv[u][e] = to_f<T>(t[e]);
  }
  const int64_t cw0 = c0 + (int64_t)wave * 64 * SJ;
  const T* kb = static_cast<const T*>(a.ksum) + (bhr * a.NCcap + cw0) * D + pc * EPV;
  const int src = (lane % RPI) * PPR + lane / RPI;
  float bv[SJ];
#pragma unroll
  for (int j = 0; j < SJ; ++j) {
    const int64_t c = cw0 + 64 * j + lane;
    bv[j] = c < nc ? a.bsum[bhr * a.NCcap + c] : 0.f;
  }
  // loads in batches of NB, two batches ahead of the arithmetic (as score_slice)
  constexpr int NB = NI >= 8 ? NI / 2 : NI;
  constexpr int NBS = NI / NB;
  constexpr int NBAT = NBS * SJ;
  auto issue = [&](int qb, uint4 (&u)[NB]) {
    const int j = qb / NBS, t0 = (qb % NBS) * NB;
    const int64_t cb = cw0 + 64 * j;
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const int row = RPI * (t0 + t) + rg;
      u[t] = cb + row < nc ? *reinterpret_cast<const uint4*>(kb + (int64_t)(64 * j + row) * D)
                           : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  uint4 buf[2][NB];
  issue(0, buf[0]);
  if (NBAT > 1) issue(1, buf[1]);
  float sv[MQ][SJ];
  float vacc[MQ][NI];
#pragma unroll
  for (int qb = 0; qb < NBAT; ++qb) {
    const int t0 = (qb % NBS) * NB;
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const T* xk = reinterpret_cast<const T*>(&buf[qb % 2][t]);
      float kx[EPV];
#pragma unroll
      for (int e = 0; e < EPV; ++e) kx[e] = to_f<T>(xk[e]);
#pragma unroll
      for (int u = 0; u < MQ; ++u) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc = fmaf(qv[u][e], kx[e], acc);
        vacc[u][t0 + t] = acc;
      }
    }
    if (qb + 2 < NBAT) issue(qb + 2, buf[qb % 2]);
    __builtin_amdgcn_sched_barrier(0);
    if (qb % NBS == NBS - 1) {   // a block of 64 rows is complete
      const int j = qb / NBS;
      const int64_t c = cw0 + 64 * j + lane;
#pragma unroll
      for (int u = 0; u < MQ; ++u) {
        float w[NI];
#pragma unroll
        for (int t = 0; t < NI; ++t) w[t] = vacc[u][t];
        butterfly<PPR / 2, NI>(w, lane);
        const float dot = __shfl(w[0], src, kWave);
        const bool ok = u < mn && c < ncm[u];
        const float sc = fmaf(dot, a.scale, bv[j]);
        if (ok) a.w.shat[((int64_t)(br * a.M + m0 + u) * a.Hq + h) * a.NCcap + c] = sc;
        sv[u][j] = ok ? sc : kNegInf;
      }
    }
  }
  // each query's slice outputs from one wave: wave u takes query u's s_hat of the
  // whole slice (through LDS) and forms its LSE partial, its top-k list
  // (ascending chunk order, ties to the lower chunk) and its four largest keys
#pragma unroll
  for (int u = 0; u < MQ; ++u)
#pragma unroll
    for (int j = 0; j < SJ; ++j) sm.s.svs[u][(int)(cw0 - c0) + 64 * j + lane] = sv[u][j];
  __syncthreads();
  const int u = wave;
  if (u >= mn || c0 >= ncm[u]) return;
  const int64_t bh = (int64_t)(br * a.M + m0 + u) * a.Hq + h;
  const int kk = a.w.kk;
  constexpr int JS = 4 * SJ;
  float x[JS];
#pragma unroll
  for (int jj = 0; jj < JS; ++jj) x[jj] = sm.s.svs[u][64 * jj + lane];
  float mw = kNegInf;
#pragma unroll
  for (int jj = 0; jj < JS; ++jj) mw = fmaxf(mw, x[jj] * kLog2e);
  mw = wave_max(mw);
  float zl = 0.f;
#pragma unroll
  for (int jj = 0; jj < JS; ++jj) zl += x[jj] == kNegInf ? 0.f : hw_exp2(x[jj] * kLog2e - mw);
  const float zw = wave_sum(zl);
  if (lane == 0) a.w.lpart[bh * a.w.nslice + slice] = make_float2(mw, zw);
  const int nv = (int)min<int64_t>(ncm[u] - c0, kThreads * SJ);
  uint32_t keys[JS];
#pragma unroll
  for (int jj = 0; jj < JS; ++jj) keys[jj] = x[jj] == kNegInf ? 0u : order_key(x[jj]);
  const int n = list_topk<JS>(keys, (nv + 63) / 64, nv, kk, lane, sm.s.l.sbuf[u], sm.s.l.wpos[u],
                              sm.s.l.wkey[u]);
  wave_lds_sync();
  if (lane < kk) {
    const int64_t o = (bh * a.w.nslice + slice) * kk + lane;
    a.w.lkey[o] = lane < n ? sm.s.l.wkey[u][lane] : 0u;
    a.w.lid[o] = lane < n ? (int32_t)(c0 + sm.s.l.wpos[u][lane]) : -1;
  }
  uint32_t y = lane < n ? sm.s.l.wkey[u][lane] : 0u;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t mk = wave_max_u32(y);
    if (lane == 0) a.w.lk4[(bh * a.w.nslice + slice) * 4 + r] = mk;
    const uint64_t at = __ballot(y == mk && mk != 0u);
    if (at && lane == __ffsll((long long)at) - 1) y = 0u;
  }
}

// Each row's group selection (one workgroup per (KV head, row)).
template <int G>
__global__ __launch_bounds__(kThreads) void dec_gsel_kernel(DecKArgs a) {
  __shared__ GroupSelSmem sel;
  extern __shared__ uint32_t bitmap[];
  const int g = blockIdx.x, v = blockIdx.y;
  DecKArgs k = a;
  k.idx_out = a.w.selw;   // slot 0 of group_select writes the selection here
  group_select<G>(k, sel, bitmap, v, g, 0);
  if (a.idx_user)
    for (int t = threadIdx.x; t < a.topk; t += kThreads)
      a.idx_user[((int64_t)v * a.Hkv + g) * a.topk + t] = sel.chosen[t];
}

// Union attention: workgroup (uslot, g, b) attends the uslot-th chunk (in
// ascending order) of the union of the M rows' selections, for the columns of
// the rows that selected it.
template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads) void dec_uattend_kernel(DecKArgs a) {
  __shared__ __align__(16) ItemSmem<T, D> it;
  __shared__ int32_t ulist[16 * 64];
  __shared__ int32_t scan[4];
  __shared__ uint32_t member;
  __shared__ int memslot[16];
  extern __shared__ uint32_t bitmap[];
  const int uslot = blockIdx.x, g = blockIdx.y, br = blockIdx.z;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int M = a.M, kk = a.topk;
  const int64_t ncmax = num_candidates(a.pos.p[br * M + M - 1], a.S, a.W);
  const int nwords = (int)((ncmax + 31) / 32);
  for (int t = threadIdx.x; t < nwords; t += kThreads) bitmap[t] = 0u;
  if (threadIdx.x == 0) member = 0u;
  __syncthreads();
  for (int t = threadIdx.x; t < M * kk; t += kThreads) {
    const int32_t c = a.w.selw[(((int64_t)br * M + t / kk) * a.Hkv + g) * kk + t % kk];
    if (c >= 0) atomicOr(&bitmap[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  // ascending list of the union (block prefix count over the words)
  const int wpt = (nwords + kThreads - 1) / kThreads;
  const int w0 = min(nwords, (int)threadIdx.x * wpt), w1 = min(w0 + wpt, nwords);
  int cnt = 0;
  for (int t = w0; t < w1; ++t) cnt += __popc(bitmap[t]);
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) scan[wave] = incl;
  __syncthreads();
  int pos = incl - cnt, nu = 0;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) {
    pos += w < wave ? scan[w] : 0;
    nu += scan[w];
  }
  for (int t = w0; t < w1; ++t) {
    uint32_t mbits = bitmap[t];
    while (mbits) {
      const int bit = __ffs(mbits) - 1;
      mbits &= mbits - 1u;
      ulist[pos++] = t * 32 + bit;
    }
  }
  __syncthreads();
  if (uslot >= nu) return;   // past the union
  const int32_t c = ulist[uslot];
  for (int t = threadIdx.x; t < M * kk; t += kThreads)
    if (a.w.selw[(((int64_t)br * M + t / kk) * a.Hkv + g) * kk + t % kk] == c) {
      atomicOr(&member, 1u << (t / kk));
      memslot[t / kk] = t % kk;   // ids within a row are distinct: one writer per row
    }
  __syncthreads();
  attend_item_mq<T, D, G>(a, it, br, g, 0, c, false, member, memslot);
}

// Fusion of one (row, head): its selected chunks (slots [0, nsel) of the row) and
// the window chunks of the group (slots kk + w; -inf where the row's window has
// no token of the chunk), weighted by exp(log-weight): one item per thread for
// the weights, waves summing every kFuseWaves-th item (as dec_fuse).
template <typename T, int D, int G>
__global__ __launch_bounds__(64 * kFuseWaves) void dec_mfuse_kernel(DecKArgs a) {
  constexpr int DPL = D / kWave;
  __shared__ float wts[256];
  __shared__ float red[kFuseWaves][D];
  __shared__ float mz[kFuseWaves][2];
  const int h = blockIdx.x, v = blockIdx.y;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int M = a.M;
  const int br = v / M, m = v % M;
  const int g = h / G, hl = h % G;
  const int64_t i = a.pos.p[v];
  const int64_t cfirst = window_left(a.pos.p[br * M], a.S, a.W) / kS;
  const int64_t clast = a.pos.p[br * M + M - 1] / kS;
  const int nsel = (int)min<int64_t>(num_candidates(i, a.S, a.W), a.topk);
  const int nitems = nsel + (int)(clast - cfirst + 1);   // <= 64 + W/S + 3 <= 256 (checked on the host)
  const int64_t bg = (int64_t)br * a.Hkv + g;
  const float* ap = a.w.mpart + (((int64_t)bg * M + m) * a.w.nitems_mq * G + hl) * (D + 2);
  const int kk = a.w.kk;
  auto slot_of = [&](int x) { return x < nsel ? x : kk + (x - nsel); };
  const int it0 = threadIdx.x;
  const float lwi = it0 < nitems ? ap[(int64_t)slot_of(it0) * G * (D + 2) + D] : kNegInf;
  float mx = wave_max(lwi);
  if (lane == 0) mz[wave][0] = mx;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kFuseWaves; ++w) mx = fmaxf(mx, mz[w][0]);
  const float wi = (it0 < nitems && lwi != kNegInf) ? __expf(lwi - mx) : 0.f;
  wts[it0] = wi;
  const float zw = wave_sum(wi);
  if (lane == 0) mz[wave][1] = zw;
  __syncthreads();
  float z = 0.f;
#pragma unroll
  for (int w = 0; w < kFuseWaves; ++w) z += mz[w][1];
  float res[DPL];
#pragma unroll
  for (int t = 0; t < DPL; ++t) res[t] = 0.f;
  constexpr int U = 8;
  for (int itb = wave; itb < nitems; itb += U * kFuseWaves) {
    float x[U][DPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = itb + u * kFuseWaves;
      const float* pp = ap + (int64_t)slot_of(min(it, nitems - 1)) * G * (D + 2) + lane * DPL;
#pragma unroll
      for (int t = 0; t < DPL; ++t) x[u][t] = pp[t];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = itb + u * kFuseWaves;
      const float w = it < nitems ? wts[it] : 0.f;
#pragma unroll
      for (int t = 0; t < DPL; ++t) res[t] = w != 0.f ? fmaf(w, x[u][t], res[t]) : res[t];
    }
  }
#pragma unroll
  for (int t = 0; t < DPL; ++t) red[wave][lane * DPL + t] = res[t];
  __syncthreads();
  if (wave != 0) return;
  const float inv = 1.f / z;
  T* orow = static_cast<T*>(a.out) + ((int64_t)v * a.Hq + h) * D;
#pragma unroll
  for (int t = 0; t < DPL; ++t) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kFuseWaves; ++w) acc += red[w][lane * DPL + t];
    orow[lane * DPL + t] = from_f<T>(acc * inv);
  }
  if (a.lse && lane == 0) a.lse[(int64_t)v * a.Hq + h] = mx + __logf(z);
}

// ---------------------------------------------------------------- host side
template <typename T, int D, int G, int SJ>
hipError_t launch_score_sj(const DecKArgs& k, hipStream_t st) {
  const int nsb = k.B * k.Hq * k.w.nslice;
  KTimer tm(K_DEC_SCORE, st);
  const int nwb = k.B * k.Hkv * k.w.nwin;   // window blocks after the scoring blocks
  hipLaunchKernelGGL((dec_score_kernel<T, D, G, SJ>), dim3((unsigned)(nsb + nwb)), dim3(kThreads), 0, st, k);
  return hipGetLastError();
}

hipError_t launch_headsel(const DecKArgs& k, hipStream_t st) {
  const int nsh = (k.w.nslice + kSPS - 1) / kSPS;
  const dim3 grid(nsh, k.Hq, k.B);
  KTimer tm(K_DEC_SELECT, st);
  switch (k.w.mj) {
    case 1: hipLaunchKernelGGL((dec_headsel_kernel<1>), grid, dim3(64), 0, st, k); break;
    case 2: hipLaunchKernelGGL((dec_headsel_kernel<2>), grid, dim3(64), 0, st, k); break;
    case 4: hipLaunchKernelGGL((dec_headsel_kernel<4>), grid, dim3(64), 0, st, k); break;
    case 8: hipLaunchKernelGGL((dec_headsel_kernel<8>), grid, dim3(64), 0, st, k); break;
    case 16: hipLaunchKernelGGL((dec_headsel_kernel<16>), grid, dim3(64), 0, st, k); break;
    default: hipLaunchKernelGGL((dec_headsel_kernel<32>), grid, dim3(64), 0, st, k); break;
  }
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t launch_decode_tg(const DecKArgs& k, hipStream_t st) {
  hipError_t e;
  switch (k.w.sj) {
    case 1: e = launch_score_sj<T, D, G, 1>(k, st); break;
    default: e = launch_score_sj<T, D, G, 2>(k, st); break;
  }
  if (e != hipSuccess) return e;
  if (k.topk > 0) {
    if (!k.w.direct) {   // else the selection ranks the slice lists itself
      e = launch_headsel(k, st);
      if (e != hipSuccess) return e;
    }
    const size_t lds = (size_t)((k.NCcap + 31) / 32) * 4;
    KTimer tm(K_DEC_ATTEND, st);
    hipLaunchKernelGGL((dec_attend_kernel<T, D, G>), dim3(k.topk, k.Hkv, k.B), dim3(kThreads), lds, st, k);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  KTimer tm(K_DEC_FUSE, st);
  hipLaunchKernelGGL((dec_fuse_kernel<T, D, G>), dim3(k.Hq, k.B), dim3(64 * kFuseWaves), 0, st, k);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_t(const DecKArgs& k, hipStream_t st) {
  switch (k.Hq / k.Hkv) {
    case 1: return launch_decode_tg<T, D, 1>(k, st);
    case 2: return launch_decode_tg<T, D, 2>(k, st);
    case 4: return launch_decode_tg<T, D, 4>(k, st);
    default: return launch_decode_tg<T, D, 8>(k, st);
  }
}

template <typename T, int D, int G, int SJ>
hipError_t launch_mscore_sj(const DecKArgs& k, int Br, hipStream_t st) {
  const int nmg = (k.M + 3) / 4;
  const int nsb = Br * nmg * k.Hq * k.w.nslice;
  const int nwb = Br * k.Hkv * k.w.nwin_mq;
  KTimer tm(K_DEC_SCORE, st);
  hipLaunchKernelGGL((dec_mscore_kernel<T, D, G, SJ>), dim3((unsigned)(nsb + nwb)), dim3(kThreads), 0, st, k);
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t launch_mq_tg(const DecKArgs& k, int Br, hipStream_t st) {
  {
    KTimer tm(K_DEC_APPEND, st);
    hipLaunchKernelGGL((dec_append_kernel<T, D>), dim3(k.Hkv, k.B), dim3(64), 0, st, k);
  }
  hipError_t e = k.w.sj == 1 ? launch_mscore_sj<T, D, G, 1>(k, Br, st) : launch_mscore_sj<T, D, G, 2>(k, Br, st);
  if (e != hipSuccess) return e;
  if (k.topk > 0) {
    if (!k.w.direct) {
      e = launch_headsel(k, st);
      if (e != hipSuccess) return e;
    }
    const size_t lds = (size_t)((k.NCcap + 31) / 32) * 4;
    {
      KTimer tm(K_DEC_GSEL, st);
      hipLaunchKernelGGL((dec_gsel_kernel<G>), dim3(k.Hkv, k.B), dim3(kThreads), lds, st, k);
    }
    KTimer tm(K_DEC_ATTEND, st);
    hipLaunchKernelGGL((dec_uattend_kernel<T, D, G>), dim3(k.M * k.topk, k.Hkv, Br), dim3(kThreads), lds, st, k);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  KTimer tm(K_DEC_FUSE, st);
  hipLaunchKernelGGL((dec_mfuse_kernel<T, D, G>), dim3(k.Hq, k.B), dim3(64 * kFuseWaves), 0, st, k);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_mq_t(const DecKArgs& k, int Br, hipStream_t st) {
  switch (k.Hq / k.Hkv) {
    case 1: return launch_mq_tg<T, D, 1>(k, Br, st);
    case 2: return launch_mq_tg<T, D, 2>(k, Br, st);
    case 4: return launch_mq_tg<T, D, 4>(k, Br, st);
    default: return launch_mq_tg<T, D, 8>(k, Br, st);
  }
}

size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// Candidates of the last cache row (the most any step can see).
int64_t max_candidates(int64_t Lcap, int S, int W) { return Lcap > 0 ? num_candidates(Lcap - 1, S, W) : 0; }

// Candidates per scoring thread SJ (a slice is 256 SJ candidates), keys per
// lane MJ of one share (kSPS slice lists of kk entries) and the number of
// slices; sj = 0 when the shares cannot cover the candidates.  One query per
// sequence takes SJ = 2 once a head has more than 16 slices of 256 (fewer,
// longer workgroups stream k' faster there); several queries per sequence do
// M times the arithmetic per k' row and keep SJ = 1 (twice the workgroups)
// while the shares cover the candidates.
void plan(int64_t NCcap, int kk, int M, int* sj, int* mj, int* nslice) {
  auto slices = [&](int s_) { return (NCcap + 256 * s_ - 1) / (256 * s_); };
  int s = (M == 1 && NCcap > 16 * 256) ? 2 : 1;
  if (s == 1 && slices(1) > (int64_t)kSPS * kMaxShares) s = 2;
  const int64_t ns = slices(s);
  const int m = (kSPS * kk + 63) / 64;
  int j = 1;
  while (j < m) j <<= 1;
  *sj = ns <= (int64_t)kSPS * kMaxShares ? s : 0;
  *mj = j;
  *nslice = (int)(ns > 0 ? ns : 1);
}

// B: sequences; M: queries per sequence (rows B M of the per-row arrays).
void layout(int B, int Hq, int Hkv, int64_t Lcap, int S, int W, int D, int topk, int M, DecWs* w,
            size_t* total, char* base) {
  const int64_t NCcap = Lcap / S;
  const int kk = topk > 0 ? topk : 1;
  int sj = 0, mj = 1, nslice = 1;
  plan(NCcap, kk, M, &sj, &mj, &nslice);
  const int nwin = W / S + 2;
  const int nitems = kk + nwin;
  const int nwin_mq = W / S + 3;   // the union of M <= S windows spans one chunk more
  const int nitems_mq = kk + nwin_mq; // per row: its selection, then the window chunks
  const int G = Hq / Hkv;
  const int Br = B;
  B *= M;
  size_t off = 0;
  auto take = [&](size_t bytes) { char* p = base ? base + off : nullptr; off += a256(bytes); return p; };
  DecWs d{};
  d.shat = reinterpret_cast<float*>(take((size_t)B * Hq * NCcap * 4));
  d.lpart = reinterpret_cast<float2*>(take((size_t)B * Hq * nslice * 8));
  d.lkey = reinterpret_cast<uint32_t*>(take((size_t)B * Hq * nslice * kk * 4));
  d.lid = reinterpret_cast<int32_t*>(take((size_t)B * Hq * nslice * kk * 4));
  d.lk4 = reinterpret_cast<uint32_t*>(take((size_t)B * Hq * nslice * 4 * 4));
  d.hkey = reinterpret_cast<uint32_t*>(take((size_t)B * Hq * kMaxShares * kk * 4));
  d.hid = reinterpret_cast<int32_t*>(take((size_t)B * Hq * kMaxShares * kk * 4));
  d.Lh = reinterpret_cast<float*>(take((size_t)B * Hq * 4));
  if (M == 1) {
    d.apart = reinterpret_cast<float*>(take((size_t)B * Hkv * nitems * G * (D + 2) * 4));
  } else {
    d.mpart = reinterpret_cast<float*>(take((size_t)Br * Hkv * M * nitems_mq * G * (D + 2) * 4));
    d.selw = reinterpret_cast<int32_t*>(take((size_t)B * Hkv * kk * 4));
  }
  d.nslice = nslice;
  d.direct = nslice <= kSPS && nslice * kk <= 64 * kDirectJ;
  d.sj = sj;
  d.mj = mj;
  d.kk = kk;
  d.nwin = nwin;
  d.nitems = nitems;
  d.nwin_mq = nwin_mq;
  d.nitems_mq = nitems_mq;
  if (w) *w = d;
  if (total) *total = off + 256;
}

}  // namespace

bool decode_supported(int64_t Lcap, int S, int W, int topk, int G) {
  int sj = 0, mj = 0, ns = 0;
  (void)G;
  plan(Lcap / S, topk > 0 ? topk : 1, 1, &sj, &mj, &ns);
  // the union bitmap (one bit per candidate) must fit the LDS beside the rest
  return sj > 0 && topk + W / S + 2 <= 256 && (Lcap / S + 31) / 32 * 4 <= 16384;
}

size_t decode_workspace(int B, int Hq, int Hkv, int64_t Lcap, int S, int W, int D, int topk, int M) {
  size_t t = 0;
  layout(B, Hq, Hkv, Lcap, S, W, D, topk, M, nullptr, &t, nullptr);
  return t;
}

hipError_t launch_decode(const DecArgs& d, hipStream_t st) {
  if (d.M > 1) return launch_decode_multi(d, st);
  DecKArgs k{};
  k.M = 1;
  for (int b = 0; b < d.B; ++b) k.pos.p[b] = d.pos[b];
  k.q = d.q; k.qh = d.qh; k.k_new = d.k_new; k.v_new = d.v_new;
  k.kc = d.kc; k.vc = d.vc; k.ksum = d.ksum; k.bsum = d.bsum;
  k.out = d.out; k.lse = d.lse; k.idx_out = d.idx;
  k.B = d.B; k.Hq = d.Hq; k.Hkv = d.Hkv; k.S = d.S; k.W = d.W; k.topk = d.topk;
  k.Lcap = d.Lcap; k.NCcap = d.Lcap / d.S; k.scale = d.scale;
  char* base = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(d.ws) + 255) & ~(uintptr_t)255);
  layout(d.B, d.Hq, d.Hkv, d.Lcap, d.S, d.W, d.D, d.topk, 1, &k.w, nullptr, base);
  hipError_t e;
  if (d.bf16) e = d.D == 128 ? launch_decode_t<bf16_t, 128>(k, st) : launch_decode_t<bf16_t, 64>(k, st);
  else e = d.D == 128 ? launch_decode_t<float, 128>(k, st) : launch_decode_t<float, 64>(k, st);
  if (e != hipSuccess) return e;
  // summaries of chunks completed by this step's token
  SumArgs s{};
  for (int b = 0; b < d.B; ++b) {
    if ((d.pos[b] + 1) % d.S == 0) {
      s.list.b[s.list.n] = b;
      s.list.c[s.list.n] = d.pos[b] / d.S;
      ++s.list.n;
    }
  }
  if (s.list.n > 0) {
    s.k = d.kc; s.ql = d.ql_new; s.ksum = d.ksum; s.bsum = d.bsum;
    s.B = d.B; s.Hq = d.Hq; s.Hkv = d.Hkv; s.D = d.D; s.bf16 = d.bf16;
    s.kT = d.Lcap; s.NCs = d.Lcap / d.S;
    s.ql_sb = (int64_t)d.Hq * d.D; s.ql_sh = d.D; s.ql_sc = 0;
    s.scale = d.scale;
    e = launch_summarize(s, st);
  }
  return e;
}

hipError_t launch_decode_multi(const DecArgs& d, hipStream_t st) {
  DecKArgs k{};
  const int M = d.M;
  for (int b = 0; b < d.B; ++b)
    for (int m = 0; m < M; ++m) k.pos.p[b * M + m] = d.pos[b] + m;
  k.q = d.q; k.qh = d.qh; k.k_new = d.k_new; k.v_new = d.v_new;
  k.kc = d.kc; k.vc = d.vc; k.ksum = d.ksum; k.bsum = d.bsum;
  k.out = d.out; k.lse = d.lse; k.idx_out = nullptr; k.idx_user = d.idx;
  k.B = d.B * M; k.Hq = d.Hq; k.Hkv = d.Hkv; k.S = d.S; k.W = d.W; k.topk = d.topk;
  k.Lcap = d.Lcap; k.NCcap = d.Lcap / d.S; k.scale = d.scale;
  k.M = M;
  char* base = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(d.ws) + 255) & ~(uintptr_t)255);
  layout(d.B, d.Hq, d.Hkv, d.Lcap, d.S, d.W, d.D, d.topk, M, &k.w, nullptr, base);
  hipError_t e;
  if (d.bf16) e = d.D == 128 ? launch_mq_t<bf16_t, 128>(k, d.B, st) : launch_mq_t<bf16_t, 64>(k, d.B, st);
  else e = d.D == 128 ? launch_mq_t<float, 128>(k, d.B, st) : launch_mq_t<float, 64>(k, d.B, st);
  if (e != hipSuccess) return e;
  // summaries of chunks completed by these tokens (at most one per sequence: M <= S)
  SumArgs s{};
  for (int b = 0; b < d.B; ++b) {
    for (int m = 0; m < M; ++m) {
      if ((d.pos[b] + m + 1) % d.S == 0) {
        s.list.b[s.list.n] = b;
        s.list.c[s.list.n] = (d.pos[b] + m) / d.S;
        ++s.list.n;
      }
    }
  }
  if (s.list.n > 0) {
    s.k = d.kc; s.ql = d.ql_new; s.ksum = d.ksum; s.bsum = d.bsum;
    s.B = d.B; s.Hq = d.Hq; s.Hkv = d.Hkv; s.D = d.D; s.bf16 = d.bf16;
    s.kT = d.Lcap; s.NCs = d.Lcap / d.S;
    s.ql_sb = (int64_t)d.Hq * d.D; s.ql_sh = d.D; s.ql_sc = 0;
    s.scale = d.scale;
    e = launch_summarize(s, st);
  }
  return e;
}

}  // namespace hils
