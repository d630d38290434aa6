// decode.hip -- one HiLS decode step per sequence (query at position pos[b]).
//
// The step is the prefill row i = pos[b] of the same definitions (summary page,
// Summary and Methodology; paper-body page, RQ1 and GQA-aware selection).  One
// query has little work per byte, so every kernel here streams memory:
//   dec_score   appends k_new/v_new to the caches and
//               scores every candidate chunk of every head of the group:
//               s_hat = scale * q_hat . k' + b', streaming k' with contiguous
//               whole-wave loads (one k' row per 16-byte lane group) and a
//               butterfly reduction.  Writes s_hat and per-slice (max, sum exp)
//               partials of each head's LSE.  Reading all of k' once dominates
//               the step's bytes.
//   dec_select  one workgroup per (b, group): L_h from the partials, the rank
//               key, per-wave top-k lists in LDS, their merged top-k ascending,
//               and each head's s_hat on it.
//   dec_attend  one workgroup per (b, group, work item), an item being a selected
//               chunk or a window chunk: the G heads are the columns of MFMA
//               tiles for the logits and for o = sum p v; the item's partial is
//               its log-weight (s_hat for a selected chunk, the token-level
//               log-mass for a window chunk) and its normalised output.
//   dec_fuse    one wave per (b, head): the exp(log-weight) average of the
//               items' outputs and L = LSE(s_hat over Sel + {log Z_win}).
//   summarize   (list mode) chunks completed by this step's token.
// Stages hand over through kernel boundaries: a device-wide fence per block (a
// last-block ticket) costs an L2 write-back on a multi-XCD part.
#include "hils_internal.h"
#include "topk.h"

namespace hils {

namespace {

constexpr int kS = 64;
constexpr int kSlice = 256;   // candidates per scoring workgroup (4 waves x 64 lanes)

struct DecPos {
  int64_t p[64];
};

struct DecWs {
  float* shat;        // [B, Hq, NCcap]
  float2* lpart;      // [B, Hq, nslice] (max, sum) in log2 units
  int32_t* idx;       // [B, Hkv, topk]
  float* ssel;        // [B, Hq, topk]
  float* apart;       // [B, Hkv, nitems, G, D + 2] per item: normalised output, log-weight
  int nslice, selj, nitems;
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

// Scoring streams k' with whole-wave contiguous loads: PPR lanes cover one k'
// row (16 bytes each), so one load instruction reads RPI consecutive rows.  Each
// lane multiplies its 16-byte piece by the matching piece of q_hat; a butterfly
// over the PPR lanes of a row (PPR - 1 shuffles for PPR row sets) leaves lane t of
// each row group with the complete dot product of row RPI*t + group.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void dec_score_kernel(DecKArgs a) {
  constexpr int EPV = 16 / sizeof(T);
  constexpr int PPR = D / EPV;        // lanes per k' row
  constexpr int RPI = kWave / PPR;    // rows per load instruction
  constexpr int NI = PPR;             // load instructions per 64 rows (= kWave / RPI)
  __shared__ float red[4][2];
  // one workgroup per (candidate slice, query head, b): a wave's loads are two
  // batches in flight, not one pair per head of the group in turn
  const int slice = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / G;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int64_t i = a.pos.p[b];
  const int64_t nc = num_candidates(i, a.S, a.W);
  const int64_t bg = (int64_t)b * a.Hkv + g;
  if (slice == 0 && h % G == 0) {
    // append this step's key/value row
    const int64_t row = (bg * a.Lcap + i) * D;
    const T* kn = static_cast<const T*>(a.k_new) + bg * D;
    const T* vn = static_cast<const T*>(a.v_new) + bg * D;
    for (int e = threadIdx.x * EPV; e < D; e += blockDim.x * EPV) {
      *reinterpret_cast<uint4*>(static_cast<T*>(a.kc) + row + e) = *reinterpret_cast<const uint4*>(kn + e);
      *reinterpret_cast<uint4*>(static_cast<T*>(a.vc) + row + e) = *reinterpret_cast<const uint4*>(vn + e);
    }
  }
  const int64_t c0 = (int64_t)slice * kSlice;
  float2* lp = a.w.lpart + ((int64_t)b * a.Hq + h) * a.w.nslice + slice;
  if (c0 >= nc) {
    if (threadIdx.x == 0) *lp = make_float2(kNegInf, 0.f);
    return;
  }
  const int pc = lane % PPR, rg = lane / PPR;
  const int64_t cw = c0 + wave * kWave;               // this wave's first candidate
  const int r = RPI * pc + rg;                        // row whose dot product this lane ends with
  const int64_t c = cw + r;
  const bool ok = c < nc;
  float qv[EPV];
  {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.qh) + ((int64_t)b * a.Hq + h) * D + pc * EPV);
    const T* t = reinterpret_cast<const T*>(&u);
#pragma unroll
    for (int e = 0; e < EPV; ++e) qv[e] = to_f<T>(t[e]);
  }
  const T* kb = static_cast<const T*>(a.ksum) + (((int64_t)b * a.Hq + h) * a.NCcap + cw) * D + pc * EPV;
  const float bv = ok ? a.bsum[((int64_t)b * a.Hq + h) * a.NCcap + c] : 0.f;
  float v[NI];
  // two batches of loads keep the live registers within four waves per SIMD
  constexpr int NB = NI >= 8 ? NI / 2 : NI;
#pragma unroll
  for (int t0 = 0; t0 < NI; t0 += NB) {
    uint4 u[NB];
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const int row = RPI * (t0 + t) + rg;
      u[t] = cw + row < nc ? *reinterpret_cast<const uint4*>(kb + (int64_t)row * D) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const T* x = reinterpret_cast<const T*>(&u[t]);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc = fmaf(qv[e], to_f<T>(x[e]), acc);
      v[t0 + t] = acc;
    }
  }
  // butterfly over the PPR lanes of a row: after the step with mask m, lanes
  // with bit m set hold the upper half of the remaining row sets
  butterfly<PPR / 2, NI>(v, lane);
  const float s = fmaf(v[0], a.scale, bv);
  if (ok) a.w.shat[((int64_t)b * a.Hq + h) * a.NCcap + c] = s;
  const float xl = ok ? s * kLog2e : kNegInf;
  const float mw = wave_max(xl);
  const float zw = wave_sum(xl == kNegInf ? 0.f : hw_exp2(xl - mw));
  if (lane == 0) {
    red[wave][0] = mw;
    red[wave][1] = zw;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = kNegInf, Z = 0.f;
    for (int w = 0; w < 4; ++w) lse_merge(M, Z, red[w][0], red[w][1]);
    *lp = make_float2(M, Z);
  }
}

// One workgroup of kSelWaves waves per (b, g).  L_h from the slice partials;
// wave w ranks the candidates [w*64J, (w+1)*64J) (rank key r = max_h(s_hat_h -
// L_h), or s_hat for one head) and keeps its exact top-k in LDS, in ascending
// chunk order; wave 0 then takes the top-k of the concatenated lists (whose
// positions ascend with the chunk index, so ties still go to the lower chunk),
// writes the ids ascending and each head's s_hat on them.  With |C_i| <= k every
// candidate is selected.
constexpr int kSelWaves = 16;

template <int G, int J>
__global__ __launch_bounds__(64 * kSelWaves) void dec_select_kernel(DecKArgs a) {
  constexpr int JM = kSelWaves;     // merge keys per lane: kSelWaves lists of <= 64 entries
  __shared__ float Ls[G];
  __shared__ uint32_t lkey[kSelWaves][64];
  __shared__ int32_t lid[kSelWaves][64];
  __shared__ float lsv[kSelWaves][64][G];   // each listed candidate's s_hat per head
  __shared__ int32_t wsel[kSelWaves][64];
  __shared__ uint32_t sbuf[kSelWaves][64];
  __shared__ int nlist[kSelWaves];
  const int g = blockIdx.y, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int64_t i = a.pos.p[b];
  const int64_t nc = num_candidates(i, a.S, a.W);
  const int topk = a.topk;
  const int64_t bg = (int64_t)b * a.Hkv + g;
  auto shat = [&](int hh, int64_t c) { return a.w.shat[((int64_t)b * a.Hq + g * G + hh) * a.NCcap + c]; };
  // output slot t (< topk) holds chunk c (-1: none) with scores sv[0..G)
  auto emit = [&](int t, int32_t c, const float* sv) {
    a.w.idx[bg * topk + t] = c;
    if (a.idx_out) a.idx_out[bg * topk + t] = c;
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
      a.w.ssel[((int64_t)b * a.Hq + g * G + hh) * topk + t] = c >= 0 ? sv[hh] : kNegInf;
  };
  if (nc <= topk) {
    if (wave == 0 && lane < topk) {
      float sv[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) sv[hh] = lane < nc ? shat(hh, lane) : kNegInf;
      emit(lane, lane < nc ? lane : -1, sv);
    }
    return;
  }
  // this wave's candidates c = cw + lane + 64 j.  With few enough per lane their
  // scores are loaded first, so that the loads overlap the L_h merge below, and
  // stay in registers; otherwise they are loaded in batches after it.
  constexpr bool kHold = J * G <= 64 && J <= 16;
  constexpr int JH = kHold ? J : 1;
  const int64_t cw = (int64_t)wave * 64 * J;
  const int cnt = (int)max<int64_t>(0, min<int64_t>(nc - cw, 64 * J));
  const int jn = (cnt + 63) / 64;
  float sv[G][JH];
  if constexpr (kHold) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int64_t c = min<int64_t>(cw + lane + 64 * j, nc - 1);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) sv[hh][j] = j < jn ? shat(hh, c) : 0.f;
    }
  }
  if (G > 1) {
    if (wave < G) {   // wave hh: L_h from the slice partials, lanes over slices
      const float2* lp = a.w.lpart + ((int64_t)b * a.Hq + g * G + wave) * a.w.nslice;
      float M = kNegInf, Z = 0.f;
      const int ns = (int)((nc + kSlice - 1) / kSlice);
      for (int sl = lane; sl < ns; sl += kWave) lse_merge(M, Z, lp[sl].x, lp[sl].y);
      const float Mw = wave_max(M);
      const float Zw = wave_sum(M == kNegInf ? 0.f : Z * hw_exp2(M - Mw));
      if (lane == 0) Ls[wave] = (Mw + hw_log2(Zw)) * kLn2;
    }
    __syncthreads();
  }
  uint32_t keys[J];
  constexpr int JB = kHold ? J : (32 / G > 0 ? 32 / G : 1);   // keys per batch of loads
#pragma unroll
  for (int j0 = 0; j0 < J; j0 += JB) {
    float xb[G][JB];
    if constexpr (!kHold) {   // the batch's score loads first (clamped in range)
#pragma unroll
      for (int j = 0; j < JB; ++j)
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
          xb[hh][j] = j0 + j < jn ? shat(hh, min<int64_t>(cw + lane + 64 * (j0 + j), nc - 1)) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      float r = kNegInf;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float x = kHold ? sv[hh][j0 + j] : xb[hh][j];
        r = G > 1 ? fmaxf(r, x - Ls[hh]) : x;
      }
      keys[j0 + j] = (j0 + j < jn && cw + lane + 64 * (j0 + j) < nc) ? order_key(r) : 0u;
    }
  }
  // ---- per-wave exact top-k over its candidate range, with the scores of the
  // listed candidates gathered from the lanes that hold them
  int n = 0;
  if (cnt > topk) {
    wave_topk_u32<J>(keys, jn, topk, lane, sbuf[wave], wsel[wave], lkey[wave]);
    n = topk;
    wave_lds_sync();
    const int id = lane < n ? wsel[wave][lane] : 0;
    if constexpr (kHold) {
      const int src = id % 64, jj = id / 64;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float v = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const float x = __shfl(sv[hh][j], src, kWave);
          if (j == jj) v = x;
        }
        if (lane < n) lsv[wave][lane][hh] = v;
      }
    } else if (lane < n) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) lsv[wave][lane][hh] = shat(hh, cw + id);
    }
    if (lane < n) lid[wave][lane] = (int32_t)(cw + id);
  } else if (cnt > 0) {
    n = cnt;
    if (lane < n) {
      lkey[wave][lane] = keys[0];
      lid[wave][lane] = (int32_t)(cw + lane);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        if constexpr (kHold) lsv[wave][lane][hh] = sv[hh][0];
        else lsv[wave][lane][hh] = shat(hh, cw + lane);
      }
    }
  }
  if (lane == 0) nlist[wave] = n;
  __syncthreads();
  if (wave != 0) return;
  // ---- merge: positions w*64 + t, t < nlist[w]; ascending position = ascending chunk
  int total = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) total += nlist[w];
  if (total <= topk) {   // every listed candidate is chosen (lists ascend with the chunk)
    int base = 0;
    for (int w = 0; w < kSelWaves; ++w) {
      const int nw = nlist[w];
      if (lane < nw) emit(base + lane, lid[w][lane], lsv[w][lane]);
      base += nw;
    }
    if (lane >= base && lane < topk) emit(lane, -1, lsv[0][0]);
    return;
  }
  // Each list holds at most TP = topk rounded up to a power of two entries, so
  // lane + 64 j carries entry lane % TP of list LPJ j + lane / TP: with several
  // lists per lane row the lane maxima span more keys, and the first bound of
  // wave_topk_u32 leaves few enough keys for its one-pass path.  The numbering
  // ascends with (list, entry), that is with the chunk.
  const int TP = topk <= 16 ? 16 : (topk <= 32 ? 32 : 64);
  const int LPJ = kWave / TP;
  const int ml = lane / TP, me = lane % TP;
  uint32_t mkeys[JM];
#pragma unroll
  for (int j = 0; j < JM; ++j) {
    const int w = LPJ * j + ml;
    mkeys[j] = (w < kSelWaves && me < nlist[w]) ? lkey[w][me] : 0u;
  }
  wave_topk_u32<JM>(mkeys, (kSelWaves + LPJ - 1) / LPJ, topk, lane, sbuf[0], wsel[0]);
  wave_lds_sync();
  if (lane < topk) {
    const int id = wsel[0][lane];
    const int l = id % 64;
    const int w = LPJ * (id / 64) + l / TP, e = l % TP;
    emit(lane, lid[w][e], lsv[w][e]);
  }
}

// Work item j < nsel: selected chunk idx[j]; else window chunk l_i/S + (j - nsel).
// One workgroup per (b, group, item), so that every item's loads are in flight
// at once.  The G heads of the group are the 16 columns of MFMA tiles
// (zero-padded): wave w takes the logits of tokens 16w .. 16w + 15 (S^T = K Q^T,
// its K fragments loaded straight from HBM), the softmax statistics of each head
// meet in LDS, V goes transposed into LDS, and O^T = V^T P^T gives wave w the
// output dims 16(w + 4t) ...  The item's partial is its log-weight (s_hat for a
// selected chunk, the token-level log-mass for a window chunk) and its
// normalised output.
constexpr int kAttThreads = 256;

template <typename T, int D, int G>
__global__ __launch_bounds__(kAttThreads) void dec_attend_kernel(DecKArgs a) {
  constexpr int EPV = 16 / sizeof(T);
  constexpr int KS = D / 32, MD = D / 16;
  constexpr int PK = D / EPV, PV = kS / EPV;         // 16-byte pieces per K / V^T row
  constexpr int VPW = PK / 4;                        // V pieces per lane (wave w: pieces w*VPW ..)
  constexpr int MDW = MD / 4;                        // output dim tiles per wave
  static_assert(G <= 16 && PK % 4 == 0 && MD % 4 == 0, "tiling");
  __shared__ __align__(16) T vt[D * kS];     // V^T rows, swizzled
  __shared__ __align__(16) T pt[16 * kS];    // P^T as [head][token]
  __shared__ float red[2][4][16];            // per-wave head max and sum
  const int item = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r16 = lane % 16, grp = lane / 16;
  const int64_t i = a.pos.p[b];
  const int64_t lw = window_left(i, a.S, a.W);
  const int64_t nc = lw / kS;
  const int nsel = (int)min<int64_t>(nc, a.topk);
  const int nwin = (int)(i / kS - lw / kS + 1);
  if (item >= nsel + nwin) return;
  const int64_t bg = (int64_t)b * a.Hkv + g;
  const float sl2 = a.scale * kLog2e;
  const bool hcol = r16 < G;                 // this lane's column is a real head
  const int h = g * G + (hcol ? r16 : 0);
  const bool is_win = item >= nsel;
  const int64_t c = is_win ? lw / kS + (item - nsel) : (int64_t)a.w.idx[bg * a.topk + item];
  const T* kc = static_cast<const T*>(a.kc) + (bg * a.Lcap + c * kS) * D;
  const T* vc = static_cast<const T*>(a.vc) + (bg * a.Lcap + c * kS) * D;

  // every load up front: K fragments (row = token 16 wave + r16), V pieces
  // (token = lane), Q^T fragments (column r16 = head)
  Frag<T> kf[KS], bq[KS];
#pragma unroll
  for (int kq = 0; kq < KS; ++kq) load_frag(kf[kq], kc + (int64_t)(16 * wave + r16) * D + 8 * grp + 32 * kq);
  uint4 vr[VPW];
#pragma unroll
  for (int t = 0; t < VPW; ++t) vr[t] = *reinterpret_cast<const uint4*>(vc + (int64_t)lane * D + (wave * VPW + t) * EPV);
  {
    const T* qrow = static_cast<const T*>(a.q) + ((int64_t)b * a.Hq + h) * D + 8 * grp;
#pragma unroll
    for (int kq = 0; kq < KS; ++kq) {
      if (hcol) load_frag(bq[kq], qrow + 32 * kq);
      else zero_frag(bq[kq]);
    }
  }
  const float lnw_sel = (!is_win && hcol) ? a.w.ssel[((int64_t)b * a.Hq + h) * a.topk + item] : 0.f;

  // S^T tile of tokens 16 wave + (4 grp + q4), column r16
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kq = 0; kq < KS; ++kq) mma(acc, kf[kq], bq[kq]);
  float x[4], mx = kNegInf;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int64_t j = c * kS + 16 * wave + 4 * grp + q4;
    const bool ok = !is_win || (j >= lw && j <= i);
    x[q4] = ok ? acc[q4] * sl2 : kNegInf;
    mx = fmaxf(mx, x[q4]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
  mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
  if (grp == 0) red[0][wave][r16] = mx;
  // V transposed into LDS: row d, token = lane
#pragma unroll
  for (int t = 0; t < VPW; ++t) {
    const T* xv = reinterpret_cast<const T*>(&vr[t]);
    const int d0 = (wave * VPW + t) * EPV;
#pragma unroll
    for (int e = 0; e < EPV; ++e) vt[swz<PV>(d0 + e, lane / EPV) * EPV + lane % EPV] = xv[e];
  }
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0][0][r16], red[0][1][r16]), fmaxf(red[0][2][r16], red[0][3][r16]));
  float p[4], ps = 0.f;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    p[q4] = hw_exp2(x[q4] - m);   // every head has an unmasked token in every item
    ps += p[q4];
  }
  ps += __shfl_xor(ps, 16, kWave);
  ps += __shfl_xor(ps, 32, kWave);
  if (grp == 0) red[1][wave][r16] = ps;
  {
    T* prow = pt + r16 * kS + 16 * wave + 4 * grp;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) prow[q4] = from_f<T>(p[q4]);
  }
  __syncthreads();
  const float l = (red[1][0][r16] + red[1][1][r16]) + (red[1][2][r16] + red[1][3][r16]);

  // O^T tiles: dims 16 md + 4 grp + q4, column r16
  f32x4_t o[MDW];
#pragma unroll
  for (int t = 0; t < MDW; ++t) {
    const int md = wave + 4 * t;
    o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k2 = 0; k2 < kS / 32; ++k2) {
      Frag<T> af, pf;
      load_frag_swz<PV>(af, vt, 16 * md + r16, 8 * grp + 32 * k2);
      load_frag(pf, pt + r16 * kS + 8 * grp + 32 * k2);
      mma(o[t], af, pf);
    }
  }
  // partial: log-weight (natural log) and the normalised output
  if (hcol) {
    float* ap = a.w.apart + ((bg * a.w.nitems + item) * G + r16) * (D + 2);
    const float inv = 1.f / l;
#pragma unroll
    for (int t = 0; t < MDW; ++t)
      *reinterpret_cast<float4*>(ap + 16 * (wave + 4 * t) + 4 * grp) =
          make_float4(o[t][0] * inv, o[t][1] * inv, o[t][2] * inv, o[t][3] * inv);
    if (wave == 0 && grp == 0) ap[D] = is_win ? (m + hw_log2(l)) * kLn2 : lnw_sel;
  }
}

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
  // item weights exp(lw_item - max): one item per thread, block max and sum
  const int it0 = threadIdx.x;
  const float lwi = it0 < nitems ? ap[(int64_t)it0 * G * (D + 2) + D] : kNegInf;
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
      const float* pp = ap + (int64_t)min(it, nitems - 1) * G * (D + 2) + lane * DPL;
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

// Candidates per selection wave: 64*J with kSelWaves waves covering every candidate.
int pick_sel_j(int64_t max_nc) {
  for (int J = 1; J <= 64; J <<= 1)
    if ((int64_t)64 * J * kSelWaves >= max_nc) return J;
  return -1;
}

template <int G>
void launch_select_j(const DecKArgs& k, hipStream_t st) {
  const dim3 grid(1, k.Hkv, k.B), block(64 * kSelWaves);
  KTimer tm(K_DEC_SELECT, st);
  switch (k.w.selj) {
    case 1: hipLaunchKernelGGL((dec_select_kernel<G, 1>), grid, block, 0, st, k); break;
    case 2: hipLaunchKernelGGL((dec_select_kernel<G, 2>), grid, block, 0, st, k); break;
    case 4: hipLaunchKernelGGL((dec_select_kernel<G, 4>), grid, block, 0, st, k); break;
    case 8: hipLaunchKernelGGL((dec_select_kernel<G, 8>), grid, block, 0, st, k); break;
    case 16: hipLaunchKernelGGL((dec_select_kernel<G, 16>), grid, block, 0, st, k); break;
    case 32: hipLaunchKernelGGL((dec_select_kernel<G, 32>), grid, block, 0, st, k); break;
    default: hipLaunchKernelGGL((dec_select_kernel<G, 64>), grid, block, 0, st, k); break;
  }
}

template <typename T, int D, int G>
hipError_t launch_decode_tg(const DecKArgs& k, hipStream_t st) {
  {
    KTimer tm(K_DEC_SCORE, st);
    hipLaunchKernelGGL((dec_score_kernel<T, D, G>), dim3(k.w.nslice, k.Hq, k.B), dim3(256), 0, st, k);
  }
  if (k.topk > 0) launch_select_j<G>(k, st);
  {
    KTimer tm(K_DEC_ATTEND, st);
    hipLaunchKernelGGL((dec_attend_kernel<T, D, G>), dim3(k.w.nitems, k.Hkv, k.B), dim3(kAttThreads), 0, st, k);
  }
  {
    KTimer tm(K_DEC_FUSE, st);
    hipLaunchKernelGGL((dec_fuse_kernel<T, D, G>), dim3(k.Hq, k.B), dim3(64 * kFuseWaves), 0, st, k);
  }
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

size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// Candidates of the last cache row (the most any step can see).
int64_t max_candidates(int64_t Lcap, int S, int W) { return Lcap > 0 ? num_candidates(Lcap - 1, S, W) : 0; }

void layout(int B, int Hq, int Hkv, int64_t Lcap, int S, int W, int D, int topk, DecWs* w,
            size_t* total, char* base) {
  const int64_t NCcap = Lcap / S;
  const int nslice = (int)((NCcap + kSlice - 1) / kSlice);
  const int nitems = topk + W / S + 2;
  const int G = Hq / Hkv;
  const int kk = topk > 0 ? topk : 1;
  size_t off = 0;
  auto take = [&](size_t bytes) { char* p = base ? base + off : nullptr; off += a256(bytes); return p; };
  DecWs d{};
  d.shat = reinterpret_cast<float*>(take((size_t)B * Hq * NCcap * 4));
  d.lpart = reinterpret_cast<float2*>(take((size_t)B * Hq * nslice * 8));
  d.idx = reinterpret_cast<int32_t*>(take((size_t)B * Hkv * kk * 4));
  d.ssel = reinterpret_cast<float*>(take((size_t)B * Hq * kk * 4));
  d.apart = reinterpret_cast<float*>(take((size_t)B * Hkv * nitems * G * (D + 2) * 4));
  d.nslice = nslice;
  d.selj = pick_sel_j(max_candidates(Lcap, S, W));
  d.nitems = nitems;
  if (w) *w = d;
  if (total) *total = off + 256;
}

}  // namespace

bool decode_supported(int64_t Lcap, int S, int W, int topk) {
  return pick_sel_j(max_candidates(Lcap, S, W)) > 0 && topk + W / S + 2 <= 256;
}

size_t decode_workspace(int B, int Hq, int Hkv, int64_t Lcap, int S, int W, int D, int topk) {
  size_t t = 0;
  layout(B, Hq, Hkv, Lcap, S, W, D, topk, nullptr, &t, nullptr);
  return t;
}

hipError_t launch_decode(const DecArgs& d, hipStream_t st) {
  DecKArgs k{};
  for (int b = 0; b < d.B; ++b) k.pos.p[b] = d.pos[b];
  k.q = d.q; k.qh = d.qh; k.k_new = d.k_new; k.v_new = d.v_new;
  k.kc = d.kc; k.vc = d.vc; k.ksum = d.ksum; k.bsum = d.bsum;
  k.out = d.out; k.lse = d.lse; k.idx_out = d.idx;
  k.B = d.B; k.Hq = d.Hq; k.Hkv = d.Hkv; k.S = d.S; k.W = d.W; k.topk = d.topk;
  k.Lcap = d.Lcap; k.NCcap = d.Lcap / d.S; k.scale = d.scale;
  char* base = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(d.ws) + 255) & ~(uintptr_t)255);
  layout(d.B, d.Hq, d.Hkv, d.Lcap, d.S, d.W, d.D, d.topk, &k.w, nullptr, base);
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

}  // namespace hils
