// decode.hip -- one HiLS decode step per sequence (query at position pos[b]).
//
// The step is the prefill row i = pos[b] of the same definitions (summary page,
// Summary and Methodology; paper-body page, RQ1 and GQA-aware selection).  One
// query has little work per byte, so every kernel here streams memory:
//   dec_score   appends k_new/v_new to the caches, resets this step's counters,
//               and scores every candidate chunk of every head of the sequence:
//               s_hat = scale * q_hat . k' + b' (16 lanes per k' row, 16-byte
//               loads), writing s_hat and per-slice (max, sum exp) partials.
//               Reading all of k' once dominates the step's bytes.
//   dec_select  per (b, group, slice of candidates): L_h from the partials, the
//               GQA rank key, a wave top-k per 64*J candidates; the last block of
//               the (b, group) (atomic ticket) merges the per-wave lists into the
//               final top-k, ascending, and gathers each head's s_hat.
//   dec_attend  one block per (b, group, work item), an item being a selected
//               chunk or a window chunk; each wave is one head: 64 keys, softmax
//               statistics and o = sum p v.  The last block of the (b, group)
//               fuses: L = LSE(s_hat over Sel + {log Z_win}),
//               out = sum exp(s_hat_c - L) o_c + exp(log Z_win - L) o_win.
//   summarize   (list mode) chunks completed by this step's token.
#include "hils_internal.h"
#include "topk.h"

namespace hils {

namespace {

constexpr int kS = 64;
constexpr int kSlice = 256;   // candidates per scoring block
constexpr int kJ = 32;        // candidates per lane in dec_select (wave: 2048)
constexpr int kSelBlock = 4 * 64 * kJ;  // candidates per select block

struct DecPos {
  int64_t p[64];
};

struct DecWs {
  float* shat;        // [B, Hq, NCcap]
  float2* lpart;      // [B, Hq, nslice] (max2, sum) in log2 units
  uint64_t* cand;     // [B, Hkv, nsel_blocks, 4, topk]
  int32_t* idx;       // [B, Hkv, topk]
  float* ssel;        // [B, Hq, topk]
  float* apart;       // [B, Hkv, nitems, G, D + 2]
  uint32_t* ctr;      // [B, Hkv, 2]
  int nslice, nselb, nitems;
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

template <typename T, int D>
__global__ __launch_bounds__(256) void dec_score_kernel(DecKArgs a) {
  const int slice = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const int64_t i = a.pos.p[b];
  const int64_t nc = num_candidates(i, a.S, a.W);
  if (slice == 0) {
    // append this step's key/value row and reset the step's tickets
    constexpr int EPV = 16 / sizeof(T);
    const int64_t row = (((int64_t)b * a.Hkv + g) * a.Lcap + i) * D;
    const T* kn = static_cast<const T*>(a.k_new) + ((int64_t)b * a.Hkv + g) * D;
    const T* vn = static_cast<const T*>(a.v_new) + ((int64_t)b * a.Hkv + g) * D;
    for (int e = threadIdx.x * EPV; e < D; e += blockDim.x * EPV) {
      *reinterpret_cast<uint4*>(static_cast<T*>(a.kc) + row + e) = *reinterpret_cast<const uint4*>(kn + e);
      *reinterpret_cast<uint4*>(static_cast<T*>(a.vc) + row + e) = *reinterpret_cast<const uint4*>(vn + e);
    }
    if (threadIdx.x < 2) a.w.ctr[((int64_t)b * a.Hkv + g) * 2 + threadIdx.x] = 0u;
  }
  const int64_t c0 = (int64_t)slice * kSlice;
  if (c0 >= nc) {
    // empty slice: neutral LSE partials
    for (int hh = threadIdx.x; hh < G; hh += blockDim.x)
      a.w.lpart[((int64_t)b * a.Hq + g * G + hh) * a.w.nslice + slice] = make_float2(kNegInf, 0.f);
    return;
  }
  constexpr int EPV = 16 / sizeof(T);
  constexpr int LPR = D / EPV;            // lanes per k' row (16 for bf16 d=128)
  constexpr int RPW = kWave / LPR;        // rows per wave step
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int sub = lane % LPR, rsub = lane / LPR;
  __shared__ float red[4][2];
  const int64_t c1 = min(c0 + kSlice, nc);
  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    float qv[EPV];
    {
      const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.qh) +
                                                      ((int64_t)b * a.Hq + h) * D + sub * EPV);
      const T* t = reinterpret_cast<const T*>(&u);
#pragma unroll
      for (int e = 0; e < EPV; ++e) qv[e] = to_f<T>(t[e]);
    }
    const T* kb = static_cast<const T*>(a.ksum) + ((int64_t)b * a.Hq + h) * a.NCcap * D;
    const float* bb = a.bsum + ((int64_t)b * a.Hq + h) * a.NCcap;
    float* sh = a.w.shat + ((int64_t)b * a.Hq + h) * a.NCcap;
    float m2 = kNegInf, s2 = 0.f;
    // rows c = c0 + (wave * RPW + rsub) + 4*RPW*step
    for (int64_t cb = c0 + wave * RPW; cb < c1; cb += 4 * RPW * 4) {
      uint4 u[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t c = cb + rsub + (int64_t)r * 4 * RPW;
        u[r] = c < c1 ? *reinterpret_cast<const uint4*>(kb + c * D + sub * EPV) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t c = cb + rsub + (int64_t)r * 4 * RPW;
        const T* t = reinterpret_cast<const T*>(&u[r]);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc = fmaf(qv[e], to_f<T>(t[e]), acc);
#pragma unroll
        for (int o = 1; o < LPR; o <<= 1) acc += __shfl_xor(acc, o, kWave);
        if (c < c1) {
          const float s = fmaf(acc, a.scale, bb[c]);
          if (sub == 0) sh[c] = s;
          const float x = s * kLog2e;
          const float mn = fmaxf(m2, x);
          s2 = (m2 == mn ? s2 : s2 * exp2f(m2 - mn)) + exp2f(x - mn);
          m2 = mn;
        }
      }
    }
    // combine: lanes with sub == 0 hold partial (m2, s2) for their rows (others duplicate)
    if (sub != 0) { m2 = kNegInf; s2 = 0.f; }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float mo = __shfl_xor(m2, o, kWave), so = __shfl_xor(s2, o, kWave);
      const float mn = fmaxf(m2, mo);
      if (mn != kNegInf)
        s2 = (m2 == kNegInf ? 0.f : s2 * exp2f(m2 - mn)) + (mo == kNegInf ? 0.f : so * exp2f(mo - mn));
      m2 = mn;
    }
    if (lane == 0) { red[wave][0] = m2; red[wave][1] = s2; }
    __syncthreads();
    if (threadIdx.x == 0) {
      float M = kNegInf, Z = 0.f;
      for (int w = 0; w < 4; ++w) {
        const float mo = red[w][0], so = red[w][1];
        const float mn = fmaxf(M, mo);
        if (mn != kNegInf)
          Z = (M == kNegInf ? 0.f : Z * exp2f(M - mn)) + (mo == kNegInf ? 0.f : so * exp2f(mo - mn));
        M = mn;
      }
      a.w.lpart[((int64_t)b * a.Hq + h) * a.w.nslice + slice] = make_float2(M, Z);
    }
    __syncthreads();
  }
}

// Per (b, g, candidate block): wave-local top-k lists; the last block merges.
template <int G>
__global__ __launch_bounds__(256) void dec_select_kernel(DecKArgs a) {
  __shared__ uint64_t sbuf[4][64];
  __shared__ int32_t sids[64];
  __shared__ float Ls[8];
  __shared__ bool last;
  const int blk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t i = a.pos.p[b];
  const int64_t nc = num_candidates(i, a.S, a.W);
  const int topk = a.topk;
  const int64_t bg = (int64_t)b * a.Hkv + g;
  int32_t* idxw = a.w.idx + bg * topk;

  if (nc <= topk) {
    // every candidate is selected; one block writes the result
    if (blk == 0) {
      for (int t = threadIdx.x; t < topk; t += blockDim.x) idxw[t] = t < nc ? t : -1;
      for (int e = threadIdx.x; e < G * topk; e += blockDim.x) {
        const int hh = e / topk, t = e % topk;
        const int h = g * G + hh;
        a.w.ssel[((int64_t)b * a.Hq + h) * topk + t] =
            t < nc ? a.w.shat[((int64_t)b * a.Hq + h) * a.NCcap + t] : kNegInf;
      }
      if (a.idx_out)
        for (int t = threadIdx.x; t < topk; t += blockDim.x) a.idx_out[bg * topk + t] = t < nc ? t : -1;
    }
    return;
  }
  if ((int64_t)blk * kSelBlock >= nc) return;  // no candidates: takes no ticket
  // per-head log-normaliser over C_i from the scoring partials
  if (G > 1 && threadIdx.x < G) {
    const int h = g * G + threadIdx.x;
    const float2* lp = a.w.lpart + ((int64_t)b * a.Hq + h) * a.w.nslice;
    float M = kNegInf, Z = 0.f;
    const int ns = (int)((nc + kSlice - 1) / kSlice);
    for (int s = 0; s < ns; ++s) {
      const float mo = lp[s].x, so = lp[s].y;
      const float mn = fmaxf(M, mo);
      if (mn != kNegInf)
        Z = (M == kNegInf ? 0.f : Z * exp2f(M - mn)) + (mo == kNegInf ? 0.f : so * exp2f(mo - mn));
      M = mn;
    }
    Ls[threadIdx.x] = (M + log2f(Z)) * kLn2;
  }
  __syncthreads();
  const int64_t cbase = (int64_t)blk * kSelBlock + (int64_t)wave * 64 * kJ;
  uint64_t* cand = a.w.cand + (bg * a.w.nselb + blk) * 4 * topk;
  if (cbase < nc) {
    uint64_t keys[kJ];
    int nvalid = 0;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int64_t c = cbase + lane + 64 * j;
      float r = kNegInf;
      if (c < nc) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float s = a.w.shat[((int64_t)b * a.Hq + g * G + hh) * a.NCcap + c];
          r = G > 1 ? fmaxf(r, s - Ls[hh]) : s;
        }
        ++nvalid;
      }
      keys[j] = c < nc ? full_key(order_key(r), c) : 0ull;
    }
    const int nv = wave_sum_i(nvalid);
    if (nv > topk) {
      const uint64_t thr = wave_kth_u64<kJ>(keys, topk, lane, sbuf[wave]);
      int base = 0;
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        const bool sel = keys[j] != 0 && keys[j] >= thr;
        const uint64_t m = __ballot(sel);
        if (sel) cand[wave * topk + base + lane_prefix(m, lane)] = keys[j];
        base += __popcll(m);
      }
    } else {
      int base = 0;
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        const bool sel = keys[j] != 0;
        const uint64_t m = __ballot(sel);
        if (sel) cand[wave * topk + base + lane_prefix(m, lane)] = keys[j];
        base += __popcll(m);
      }
      for (int t = nv + lane; t < topk; t += kWave) cand[wave * topk + t] = 0ull;
    }
  } else {
    for (int t = lane; t < topk; t += kWave) cand[wave * topk + t] = 0ull;
  }
  // ticket: the last block of this (b, g) merges
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int nb = (int)((nc + kSelBlock - 1) / kSelBlock);
    const uint32_t t = atomicAdd(&a.w.ctr[bg * 2 + 0], 1u);
    last = (t == (uint32_t)nb - 1);
  }
  __syncthreads();
  if (!last || wave != 0) return;
  __threadfence();
  const int nb = (int)((nc + kSelBlock - 1) / kSelBlock);
  const int ntot = nb * 4 * topk;  // <= 2048 for supported sizes
  uint64_t v[kJ];
  const uint64_t* call = a.w.cand + bg * a.w.nselb * 4 * topk;
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < ntot ? call[e] : 0ull;
  }
  const uint64_t thr = wave_kth_u64<kJ>(v, topk, lane, sbuf[0]);
  // compact the chosen keys, then sort their chunk ids ascending
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < kJ; ++j) cnt += (v[j] != 0 && v[j] >= thr) ? 1 : 0;
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += x;
  }
  int pos = incl - cnt;
#pragma unroll
  for (int j = 0; j < kJ; ++j)
    if (v[j] != 0 && v[j] >= thr) sids[pos++] = key_chunk(v[j]);
  wave_lds_sync();
  const uint32_t cs = lane < topk ? (uint32_t)sids[lane] : 0xffffffffu;
  const uint32_t srt = bitonic_sort64<uint32_t>(cs, lane, false);
  if (lane < topk) {
    idxw[lane] = (int32_t)srt;
    if (a.idx_out) a.idx_out[bg * topk + lane] = (int32_t)srt;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const int h = g * G + hh;
      a.w.ssel[((int64_t)b * a.Hq + h) * topk + lane] = a.w.shat[((int64_t)b * a.Hq + h) * a.NCcap + srt];
    }
  }
}

// Work item j < nsel: selected chunk idx[j]; else window chunk l_i/S + (j - nsel).
template <typename T, int D, int G>
__global__ __launch_bounds__(64 * G) void dec_attend_kernel(DecKArgs a) {
  constexpr int DPL = D / kWave;  // dims per lane (2 for d=128)
  __shared__ float ps[G][kS];
  __shared__ float qs[G][D];
  __shared__ bool last;
  const int item = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t i = a.pos.p[b];
  const int64_t lw = window_left(i, a.S, a.W);
  const int64_t nc = lw / kS;
  const int nsel = (int)min<int64_t>(nc, a.topk);
  const int nwin = (int)(i / kS - lw / kS + 1);
  const int nitems = nsel + nwin;
  if (item >= nitems) return;
  const int64_t bg = (int64_t)b * a.Hkv + g;
  const int h = g * G + wave;
  int64_t c;
  bool is_win;
  if (item < nsel) {
    c = a.w.idx[bg * a.topk + item];
    is_win = false;
  } else {
    c = lw / kS + (item - nsel);
    is_win = true;
  }
  const T* kc = static_cast<const T*>(a.kc) + (bg * a.Lcap + c * kS) * D;
  const T* vc = static_cast<const T*>(a.vc) + (bg * a.Lcap + c * kS) * D;
  {
    const T* qv = static_cast<const T*>(a.q) + ((int64_t)b * a.Hq + h) * D;
    for (int e = lane; e < D; e += kWave) qs[wave][e] = to_f<T>(qv[e]);
  }
  wave_lds_sync();
  // logits: lane = token
  const int64_t j = c * kS + lane;
  const bool ok = !is_win || (j >= lw && j <= i);
  float s = kNegInf;
  if (ok) {
    constexpr int EPV = 16 / sizeof(T);
    float acc = 0.f;
#pragma unroll
    for (int e0 = 0; e0 < D; e0 += EPV) {
      const uint4 u = *reinterpret_cast<const uint4*>(kc + (int64_t)lane * D + e0);
      const T* t = reinterpret_cast<const T*>(&u);
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc = fmaf(qs[wave][e0 + e], to_f<T>(t[e]), acc);
    }
    s = acc * (a.scale * kLog2e);
  }
  const float m = wave_max(s);
  const float p = ok ? exp2f(s - m) : 0.f;
  const float l = wave_sum(p);
  ps[wave][lane] = p;
  wave_lds_sync();
  float o[DPL];
#pragma unroll
  for (int t = 0; t < DPL; ++t) o[t] = 0.f;
  for (int jj = 0; jj < kS; ++jj) {
    const float pj = ps[wave][jj];
    const T* vr = vc + (int64_t)jj * D + lane * DPL;
#pragma unroll
    for (int t = 0; t < DPL; ++t) o[t] = fmaf(pj, to_f<T>(vr[t]), o[t]);
  }
  float* ap = a.w.apart + ((bg * a.w.nitems + item) * G + wave) * (D + 2);
#pragma unroll
  for (int t = 0; t < DPL; ++t) ap[lane * DPL + t] = o[t];
  if (lane == 0) { ap[D] = m; ap[D + 1] = l; }

  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t t = atomicAdd(&a.w.ctr[bg * 2 + 1], 1u);
    last = (t == (uint32_t)nitems - 1);
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  // fusion for head h (this wave): window items merge at token level
  const float* base = a.w.apart + (bg * a.w.nitems) * G * (D + 2);
  float Mw = kNegInf;
  for (int it = nsel; it < nitems; ++it) Mw = fmaxf(Mw, base[((int64_t)it * G + wave) * (D + 2) + D]);
  float lwin = 0.f, ow[DPL];
#pragma unroll
  for (int t = 0; t < DPL; ++t) ow[t] = 0.f;
  for (int it = nsel; it < nitems; ++it) {
    const float* pp = base + ((int64_t)it * G + wave) * (D + 2);
    const float mi = (pp + D)[0];
    if (mi == kNegInf) continue;
    const float f = exp2f(mi - Mw);
    lwin += f * (pp + D + 1)[0];
#pragma unroll
    for (int t = 0; t < DPL; ++t) ow[t] += f * (pp + lane * DPL + t)[0];
  }
  const float logzw = (Mw + log2f(lwin)) * kLn2;
  const float* ss = a.w.ssel + ((int64_t)b * a.Hq + h) * a.topk;
  float L = logzw;
  for (int it = 0; it < nsel; ++it) {
    const float x = ss[it];
    const float mx = fmaxf(L, x);
    L = mx + __logf(__expf(L - mx) + __expf(x - mx));
  }
  float res[DPL];
  const float fw = __expf(logzw - L) / lwin;
#pragma unroll
  for (int t = 0; t < DPL; ++t) res[t] = ow[t] * fw;
  for (int it = 0; it < nsel; ++it) {
    const float* pp = base + ((int64_t)it * G + wave) * (D + 2);
    const float f = __expf(ss[it] - L) / (pp + D + 1)[0];
#pragma unroll
    for (int t = 0; t < DPL; ++t) res[t] += f * (pp + lane * DPL + t)[0];
  }
  T* orow = static_cast<T*>(a.out) + ((int64_t)b * a.Hq + h) * D;
#pragma unroll
  for (int t = 0; t < DPL; ++t) orow[lane * DPL + t] = from_f<T>(res[t]);
  if (a.lse && lane == 0) a.lse[(int64_t)b * a.Hq + h] = L;
}

template <typename T, int D, int G>
hipError_t launch_decode_tg(const DecKArgs& k, hipStream_t st) {
  hipLaunchKernelGGL((dec_score_kernel<T, D>), dim3(k.w.nslice, k.Hkv, k.B), dim3(256), 0, st, k);
  if (k.topk > 0)
    hipLaunchKernelGGL((dec_select_kernel<G>), dim3(k.w.nselb, k.Hkv, k.B), dim3(256), 0, st, k);
  hipLaunchKernelGGL((dec_attend_kernel<T, D, G>), dim3(k.w.nitems, k.Hkv, k.B), dim3(64 * G), 0, st, k);
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

void layout(int B, int Hq, int Hkv, int64_t Lcap, int S, int W, int D, int topk, DecWs* w,
            size_t* total, char* base) {
  const int64_t NCcap = Lcap / S;
  const int nslice = (int)((NCcap + kSlice - 1) / kSlice);
  const int nselb = (int)((NCcap + kSelBlock - 1) / kSelBlock);
  const int nitems = topk + W / S + 2;
  const int G = Hq / Hkv;
  size_t off = 0;
  auto take = [&](size_t bytes) { char* p = base ? base + off : nullptr; off += a256(bytes); return p; };
  DecWs d{};
  d.shat = reinterpret_cast<float*>(take((size_t)B * Hq * NCcap * 4));
  d.lpart = reinterpret_cast<float2*>(take((size_t)B * Hq * nslice * 8));
  d.cand = reinterpret_cast<uint64_t*>(take((size_t)B * Hkv * nselb * 4 * (topk > 0 ? topk : 1) * 8));
  d.idx = reinterpret_cast<int32_t*>(take((size_t)B * Hkv * (topk > 0 ? topk : 1) * 4));
  d.ssel = reinterpret_cast<float*>(take((size_t)B * Hq * (topk > 0 ? topk : 1) * 4));
  d.apart = reinterpret_cast<float*>(take((size_t)B * Hkv * nitems * G * (D + 2) * 4));
  d.ctr = reinterpret_cast<uint32_t*>(take((size_t)B * Hkv * 2 * 4));
  d.nslice = nslice;
  d.nselb = nselb;
  d.nitems = nitems;
  if (w) *w = d;
  if (total) *total = off + 256;
}

}  // namespace

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
