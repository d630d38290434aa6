// attend.hip -- per-group attention and the hierarchical fusion (prefill).
//
// Summary page, Methodology 2, Eq. 10: w_ij = exp(s_ij)/Z_{i,c(j)} * Zhat_{i,c(j)}/Zhat_i
// with Zhat_{i,c} = exp(s_hat_{i,c}) for a selected chunk and, for the window, its
// true token-level mass Z_{i,win} (paper-body page, implementation: the normaliser
// adds the window's exact mass to the selected chunks' surrogate masses).  So
//   out_i = sum_{c in Sel} exp(s_hat_c - L) o_c + exp(log Z_win - L) o_win,
//   L = LSE({s_hat_c} + {log Z_win}),
// where o_gamma is ordinary softmax attention of q_i over the group's tokens.
//
// The pages' kernel takes adjacent queries together and visits every chunk any
// of them selected once for all of them (paper-body page, implementation,
// kernel design).  That reuse depends on
// adjacent queries picking overlapping chunks; when they do not, every
// (query, chunk) visit re-reads 32 KiB of K/V.  This file instead runs the
// selected part chunk-major: each selected chunk's K/V is staged once in LDS and
// attended by every query that selected it, in MFMA tiles of 16 (query, head)
// rows; each visit writes its weighted output exp(s_hat_c - L_sel) o_c
// (L_sel = LSE over the selected chunks only) to a partial slot.  The window
// part is dense and runs query-major, flash-style; its epilogue fuses, reading
// each row's partials with coalesced loads:
//   out_i = exp(log Z_win - L) o_win + exp(L_sel - L) * sum_slots partial,
//   L = LSE(L_sel, log Z_win).
// The (query, slot) lists per chunk are built deterministically: per tile of
// 256 to 1024 queries each chunk's count (from LDS bitmaps of which of 64
// queries chose it), a column scan over tiles and a scan over chunks give every
// entry a fixed position, in query order within its chunk.
//
// Score tiles are computed transposed, S^T = K Q^T (tokens x rows), so each lane
// holds one row's scores for 16 tokens; the same registers, cast to the operand
// type, are the B operand of O^T = V^T P^T with the reduction order of the
// token axis permuted to match (V is staged transposed in LDS).
#include "attend_tiles.h"
#include "hils_internal.h"
#include "topk.h"

namespace hils {

namespace {

constexpr int kS = 64;  // chunk size


struct IdxArgs {
  const int32_t* idx;
  const float* ssel;
  int32_t* tile_cnt;   // [B, Hkv, ntiles, NCs]: counts, then exclusive offsets
  int32_t* bcount;     // [B, Hkv, NCs]
  int64_t* bbase;      // [B, Hkv, NCs]
  uint32_t* entries;   // i * 64 + slot
  float* wq;           // [B, Hkv, T, topk, G] chunk weights exp(s_hat - L_sel) per head
  float* lsel;         // [B, Hq, T]
  int32_t* nvalid;     // [B, Hkv, T]: selected slots of each row (a prefix of its k)
  int32_t* smap;       // [B, Hkv, sbound]: chunk c | range r << 13 of each chunk-pass workgroup
  int32_t* stot;       // [B, Hkv]: workgroups of (b, g)
  int B, Hq, Hkv, topk;
  int64_t T, NCs, ntiles;
  int tile;            // queries per counting tile (idx_tile)
  int E;               // entries per chunk-pass workgroup (a chunk's list in ranges of E)
  int64_t sbound;      // workgroups per (b, g), an upper bound
};

// Queries per ranking sub-tile (one 64-bit LDS bitmap word per chunk).  A
// counting tile is a multiple of it (idx_tile).
constexpr int kIdxSub = 64;

constexpr size_t kMaxLds = 160 * 1024;   // LDS per workgroup

// Queries per counting tile: 1024, halved down to 256 while the (b, g, tile)
// grid would have fewer than 1024 workgroups.  A workgroup runs its tile's
// sub-tiles one after another, so short sequences want shorter tiles; long ones
// want longer tiles, for fewer per-tile counts to scan and load.
int idx_tile(int B, int Hkv, int64_t T) {
  int tile = 1024;
  while (tile > 256 && (int64_t)B * Hkv * ((T + tile - 1) / tile) < 1024) tile /= 2;
  return tile;
}

// Sets bit ql of chunk c's word for every entry (query i0 + ql, slot) of the
// sub-tile of 64 queries at i0 (a chunk listed twice in a row counts once).
__device__ __forceinline__ void sub_bitmap(const IdxArgs& a, uint64_t* bm, const int32_t* row, int64_t i0) {
  const int n = kIdxSub * a.topk;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const int ql = e / a.topk;
    if (i0 + ql >= a.T) break;
    const int32_t c = row[e];
    if (c >= 0 && c < a.NCs) atomicOr((unsigned long long*)&bm[c], 1ull << ql);
  }
}

// Queries of the counting tile that chose each chunk of (b, g), one
// sub-tile bitmap at a time (eight waves: the sub-tiles form a chain of
// barriers, so more waves per chain beat more workgroups per compute unit).
__global__ __launch_bounds__(512) void idx_count_kernel(IdxArgs a) {
  extern __shared__ uint64_t bm[];
  int32_t* cnt = reinterpret_cast<int32_t*>(bm + a.NCs);
  const int64_t t = blockIdx.x;
  const int g = blockIdx.y, b = blockIdx.z;
  for (int64_t c = threadIdx.x; c < a.NCs; c += blockDim.x) {
    cnt[c] = 0;
    bm[c] = 0ull;
  }
  for (int64_t i0 = t * a.tile; i0 < min<int64_t>((t + 1) * a.tile, a.T); i0 += kIdxSub) {
    __syncthreads();
    sub_bitmap(a, bm, a.idx + (((int64_t)b * a.Hkv + g) * a.T + i0) * a.topk, i0);
    __syncthreads();
    for (int64_t c = threadIdx.x; c < a.NCs; c += blockDim.x) {   // each thread its own chunks
      cnt[c] += __popcll(bm[c]);
      bm[c] = 0ull;
    }
  }
  int32_t* out = a.tile_cnt + (((int64_t)b * a.Hkv + g) * a.ntiles + t) * a.NCs;
  for (int64_t c = threadIdx.x; c < a.NCs; c += blockDim.x) out[c] = cnt[c];
}

// Column scan over tiles: exclusive offsets in place, totals to bcount.  A block
// owns 32 chunk columns of one (b, g); its 32 thread rows split the tiles into
// segments (segment sums, a scan across segments, then the in-place rewrite).
__global__ __launch_bounds__(1024) void idx_scan_tiles_kernel(IdxArgs a) {
  __shared__ int32_t part[32][33];
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;
  const int64_t c = (int64_t)blockIdx.x * 32 + tx;
  const int64_t bg = blockIdx.y;
  const int64_t seg = (a.ntiles + 31) / 32;
  const int64_t t0 = ty * seg, t1 = min(t0 + seg, a.ntiles);
  int32_t* col = a.tile_cnt + bg * a.ntiles * a.NCs + c;
  int32_t s = 0;
  if (c < a.NCs)
    for (int64_t t = t0; t < t1; ++t) s += col[t * a.NCs];
  part[ty][tx] = s;
  __syncthreads();
  int32_t run = 0;
  for (int k = 0; k < ty; ++k) run += part[k][tx];
  if (c < a.NCs) {
    for (int64_t t = t0; t < t1; ++t) {
      const int32_t v = col[t * a.NCs];
      col[t * a.NCs] = run;
      run += v;
    }
    if (ty == 31) a.bcount[bg * a.NCs + c] = run;
  }
}

// Exclusive scan of all bucket counts (one block).
__global__ __launch_bounds__(1024) void idx_scan_buckets_kernel(IdxArgs a) {
  __shared__ int64_t part[1024];
  const int64_t nb = (int64_t)a.B * a.Hkv * a.NCs;
  const int64_t per = (nb + 1023) / 1024;
  const int64_t lo = threadIdx.x * per, hi = min(lo + per, nb);
  int64_t s = 0;
  for (int64_t j = lo; j < hi; ++j) s += a.bcount[j];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int64_t v = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int64_t run = part[threadIdx.x] - s;
  for (int64_t j = lo; j < hi; ++j) {
    a.bbase[j] = run;
    run += a.bcount[j];
  }
}

// The chunk pass's workgroups of (b, g): chunk c's list in ceil(n_c / E) ranges
// of E entries, numbered in chunk order (the early chunks, the longest lists,
// first).  One block per (b, g): per-thread runs of chunks, a block scan of
// their range counts, then each range's (chunk, range) word.
__global__ __launch_bounds__(1024) void split_map_kernel(IdxArgs a) {
  __shared__ int32_t part[1024];
  const int64_t bg = blockIdx.x;
  const int32_t* cnt = a.bcount + bg * a.NCs;
  const int64_t per = (a.NCs + 1023) / 1024;
  const int64_t lo = threadIdx.x * per, hi = min(lo + per, a.NCs);
  int32_t sum = 0;
  for (int64_t c = lo; c < hi; ++c) sum += (cnt[c] + a.E - 1) / a.E;
  part[threadIdx.x] = sum;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int32_t v = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int32_t pos = part[threadIdx.x] - sum;
  int32_t* map = a.smap + bg * a.sbound;
  for (int64_t c = lo; c < hi; ++c) {
    const int32_t nr = (cnt[c] + a.E - 1) / a.E;
    for (int32_t r = 0; r < nr; ++r) map[pos++] = (int32_t)c | (r << 13);
  }
  if (threadIdx.x == 1023) a.stot[bg] = part[1023];
}

// Entries at their final positions, in query order within each bucket.  A
// block takes one counting tile of queries; each chunk's next position (its
// bucket's base relative to the first bucket of (b, g), plus the tile's offset
// in the bucket) sits in LDS, read once with coalesced loads.  The tile's
// sub-tiles of 64 queries run in order: the bitmap of which of the 64 queries
// chose each chunk gives an entry its rank among them, then moves the chunk's
// position on by its count.  (Relative positions fit 32 bits: a (b, g) has
// T * topk entries.)
__global__ __launch_bounds__(256) void idx_fill_kernel(IdxArgs a) {
  extern __shared__ uint64_t bm[];
  int32_t* pos = reinterpret_cast<int32_t*>(bm + a.NCs);
  const int64_t t = blockIdx.x;
  const int g = blockIdx.y, b = blockIdx.z;
  const int32_t* toff = a.tile_cnt + (((int64_t)b * a.Hkv + g) * a.ntiles + t) * a.NCs;
  const int64_t* bbase = a.bbase + ((int64_t)b * a.Hkv + g) * a.NCs;
  const int64_t base0 = bbase[0];
  for (int64_t c = threadIdx.x; c < a.NCs; c += blockDim.x) {
    pos[c] = (int32_t)(bbase[c] - base0) + toff[c];
    bm[c] = 0ull;
  }
  const int n = kIdxSub * a.topk;
  for (int64_t i0 = t * a.tile; i0 < min<int64_t>((t + 1) * a.tile, a.T); i0 += kIdxSub) {
    const int32_t* row = a.idx + (((int64_t)b * a.Hkv + g) * a.T + i0) * a.topk;
    __syncthreads();   // pos and bm as the previous sub-tile left them
    sub_bitmap(a, bm, row, i0);
    __syncthreads();
    for (int e = threadIdx.x; e < n; e += blockDim.x) {
      const int ql = e / a.topk, sl = e % a.topk;
      const int64_t i = i0 + ql;
      if (i >= a.T) break;
      const int32_t c = row[e];
      if (c < 0 || c >= a.NCs) continue;
      const int rank = __popcll(bm[c] & ((1ull << ql) - 1ull));
      a.entries[base0 + pos[c] + rank] = (uint32_t)(i * 64 + sl);
    }
    __syncthreads();
    for (int64_t c = threadIdx.x; c < a.NCs; c += blockDim.x) {   // each thread its own chunks
      pos[c] += __popcll(bm[c]);
      bm[c] = 0ull;
    }
  }
}

// idx_fill_kernel's result, with the tile's entries staged in LDS in chunk
// order and each chunk's run then written with contiguous stores (direct
// 4-byte scatters cost several times their bytes in partial-line writes).  The
// tile's per-chunk counts (the next tile's offsets minus this tile's, or the
// chunk's total after the last tile) are scanned to each chunk's start in the
// stage; the sub-tiles then place their entries there as idx_fill_kernel places
// them in HBM, and run[c] ends as the end of chunk c's run.  LDS: NCs * 12
// bytes + tile * topk * 4 bytes (the host checks that they fit).
__global__ __launch_bounds__(1024) void idx_fill_staged_kernel(IdxArgs a) {
  extern __shared__ uint64_t bm[];
  int32_t* run = reinterpret_cast<int32_t*>(bm + a.NCs);
  uint32_t* stage = reinterpret_cast<uint32_t*>(run + a.NCs);
  __shared__ int32_t wtot[16];
  const int64_t t = blockIdx.x;
  const int g = blockIdx.y, b = blockIdx.z;
  const int64_t bg = (int64_t)b * a.Hkv + g;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int nwaves = blockDim.x / kWave;
  const int32_t* toff = a.tile_cnt + (bg * a.ntiles + t) * a.NCs;
  const int32_t* tnext = t + 1 < a.ntiles ? toff + a.NCs : a.bcount + bg * a.NCs;
  // each thread a contiguous run of chunks: counts, then an exclusive block scan
  const int64_t per = (a.NCs + blockDim.x - 1) / blockDim.x;
  const int64_t c0 = tid * per, c1 = min<int64_t>(c0 + per, a.NCs);
  int32_t sum = 0;
  for (int64_t c = c0; c < c1; ++c) sum += tnext[c] - toff[c];
  int32_t inc = sum;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int32_t v = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += v;
  }
  if (lane == kWave - 1) wtot[wave] = inc;
  __syncthreads();
  int32_t base = inc - sum;
  for (int w = 0; w < wave; ++w) base += wtot[w];
  for (int64_t c = c0; c < c1; ++c) {
    run[c] = base;
    base += tnext[c] - toff[c];
    bm[c] = 0ull;
  }
  const int n = kIdxSub * a.topk;
  for (int64_t i0 = t * a.tile; i0 < min<int64_t>((t + 1) * a.tile, a.T); i0 += kIdxSub) {
    const int32_t* row = a.idx + (bg * a.T + i0) * a.topk;
    __syncthreads();   // run and bm as the previous sub-tile left them
    sub_bitmap(a, bm, row, i0);
    __syncthreads();
    for (int e = tid; e < n; e += blockDim.x) {
      const int ql = e / a.topk, sl = e % a.topk;
      const int64_t i = i0 + ql;
      if (i >= a.T) break;
      const int32_t c = row[e];
      if (c < 0 || c >= a.NCs) continue;
      const int rank = __popcll(bm[c] & ((1ull << ql) - 1ull));
      stage[run[c] + rank] = (uint32_t)(i * 64 + sl);
    }
    __syncthreads();
    for (int64_t c = tid; c < a.NCs; c += blockDim.x) {   // each thread its own chunks
      run[c] += __popcll(bm[c]);
      bm[c] = 0ull;
    }
  }
  __syncthreads();
  // chunk c's run is stage[run[c-1], run[c]) (from 0 for chunk 0); it goes to
  // its bucket at the tile's offset
  const int64_t* bbase = a.bbase + bg * a.NCs;
  for (int64_t c = wave; c < a.NCs; c += nwaves) {
    const int32_t e1 = run[c], e0 = c > 0 ? run[c - 1] : 0;
    if (e1 == e0) continue;
    uint32_t* dst = a.entries + bbase[c] + toff[c];
    for (int32_t j = lane; j < e1 - e0; j += kWave) dst[j] = stage[e0 + j];
  }
}

// The same as lsel_kernel (below) with four slots per lane: lane (r, hh, q) of
// a wave takes slots 4q .. 4q+3 of head hh of row r (NQP lanes per head, G NQP
// per row, 64 / (G NQP) rows per wave), so every score and index load is 16
// bytes.  The slots' exp terms are added in pairs and then across the NQP
// lanes by the same butterfly as lsel_kernel's, so the sums are bit for bit
// the same.  The weights go through a wave-private LDS tile in the record
// layout [row][slot][G] and leave as contiguous 16-byte stores.
template <int G, int NQP>
__global__ __launch_bounds__(256) void lsel4_kernel(IdxArgs a) {
  constexpr int LPR = G * NQP;       // lanes per row
  constexpr int RW = kWave / LPR;    // rows per wave
  __shared__ __align__(16) float wt[4][RW * 4 * NQP * G];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r = lane / LPR, hh = (lane / NQP) % G, q = lane % NQP;
  const int64_t nrows = (int64_t)a.B * a.Hkv * a.T;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * RW;   // this wave's first row
  const int64_t row = row0 + r;
  const bool live = row < nrows;
  const int64_t rr = live ? row : nrows - 1;
  const int64_t i = rr % a.T;
  const int g = (int)((rr / a.T) % a.Hkv);
  const int b = (int)(rr / (a.T * a.Hkv));
  const int topk = a.topk;
  const bool inrow = 4 * q < topk;
  const int64_t rowq = ((int64_t)b * a.Hq + g * G + hh) * a.T + i;
  int4 id = make_int4(-1, -1, -1, -1);
  float4 xs = make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
  if (inrow) {
    id = *reinterpret_cast<const int4*>(a.idx + rr * topk + 4 * q);
    xs = *reinterpret_cast<const float4*>(a.ssel + rowq * topk + 4 * q);
  }
  float x[4] = {id.x >= 0 ? xs.x : kNegInf, id.y >= 0 ? xs.y : kNegInf,
                id.z >= 0 ? xs.z : kNegInf, id.w >= 0 ? xs.w : kNegInf};
  float m = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  if (NQP > 1) m = fmaxf(m, xor_lane<1>(m));
  if (NQP > 2) m = fmaxf(m, xor_lane<2>(m));
  if (NQP > 4) m = fmaxf(m, xor_lane<4>(m));
  if (NQP > 8) m = fmaxf(m, xor_lane<8>(m));
  float e[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) e[j] = (x[j] == kNegInf) ? 0.f : __expf(x[j] - m);
  float z = (e[0] + e[1]) + (e[2] + e[3]);
  if (NQP > 1) z += xor_lane<1>(z);
  if (NQP > 2) z += xor_lane<2>(z);
  if (NQP > 4) z += xor_lane<4>(z);
  if (NQP > 8) z += xor_lane<8>(z);
  const float ls = m == kNegInf ? kNegInf : m + __logf(z);
  if (live && q == 0) a.lsel[rowq] = ls;
  // the row's selected slots (the same for every head), counted over its quarters
  float nsel = (float)((id.x >= 0) + (id.y >= 0) + (id.z >= 0) + (id.w >= 0));
  if (NQP > 1) nsel += xor_lane<1>(nsel);
  if (NQP > 2) nsel += xor_lane<2>(nsel);
  if (NQP > 4) nsel += xor_lane<4>(nsel);
  if (NQP > 8) nsel += xor_lane<8>(nsel);
  if (live && q == 0 && hh == 0) a.nvalid[rr] = (int32_t)nsel;
  float* tw = wt[wave];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int slot = 4 * q + j;
    if (slot < topk) tw[(r * topk + slot) * G + hh] = x[j] == kNegInf ? 0.f : __expf(x[j] - ls);
  }
  wave_lds_sync();
  // the wave's rows are consecutive records: RW * topk * G floats from row0
  const int nf = RW * topk * G;
  float* dst = a.wq + row0 * topk * G;
  const int64_t lim = (nrows - row0) * topk * G;   // floats of live rows
  for (int f = 4 * lane; f < nf; f += 4 * kWave)
    if (f < lim) *reinterpret_cast<float4*>(dst + f) = *reinterpret_cast<const float4*>(tw + f);
}

// L_sel = LSE of each head's s_hat over its selected chunks (-inf if none), and
// each selected chunk's weight exp(s_hat - L_sel) for the G heads of the group,
// stored together ([B, Hkv, T, topk, G]) so the chunk-major pass reads one
// contiguous record per (query, slot).  L lanes per (b, g, i) row (L = smallest
// power of two >= k), lane = slot.
template <int G>
__global__ __launch_bounds__(256) void lsel_kernel(IdxArgs a, int L) {
  const int64_t lane_g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = lane_g / L;                 // (b, g, i)
  const int l = (int)(lane_g % L);
  const int64_t nrows = (int64_t)a.B * a.Hkv * a.T;
  const bool live = row < nrows;
  const int64_t rr = live ? row : nrows - 1;
  const int64_t i = rr % a.T;
  const int g = (int)((rr / a.T) % a.Hkv);
  const int b = (int)(rr / (a.T * a.Hkv));
  // the index and every head's score load together (a slot below k lies inside
  // its row either way); a padding slot is dropped afterwards
  const bool inrow = l < a.topk;
  const int32_t id = inrow ? a.idx[rr * a.topk + l] : -1;
  float xs[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const int64_t rowq = ((int64_t)b * a.Hq + g * G + hh) * a.T + i;
    xs[hh] = inrow ? a.ssel[rowq * a.topk + l] : kNegInf;
  }
  const bool sel = id >= 0;
  {
    float nsel = sel ? 1.f : 0.f;
    if (L > 1) nsel += xor_lane<1>(nsel);
    if (L > 2) nsel += xor_lane<2>(nsel);
    if (L > 4) nsel += xor_lane<4>(nsel);
    if (L > 8) nsel += xor_lane<8>(nsel);
    if (L > 16) nsel += xor_lane<16>(nsel);
    if (L > 32) nsel += xor_lane<32>(nsel);
    if (live && l == 0) a.nvalid[rr] = (int32_t)nsel;
  }
  float w[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const int64_t rowq = ((int64_t)b * a.Hq + g * G + hh) * a.T + i;
    const float x = sel ? xs[hh] : kNegInf;
    float m = x;
    if (L > 1) m = fmaxf(m, xor_lane<1>(m));
    if (L > 2) m = fmaxf(m, xor_lane<2>(m));
    if (L > 4) m = fmaxf(m, xor_lane<4>(m));
    if (L > 8) m = fmaxf(m, xor_lane<8>(m));
    if (L > 16) m = fmaxf(m, xor_lane<16>(m));
    if (L > 32) m = fmaxf(m, xor_lane<32>(m));
    float z = (x == kNegInf) ? 0.f : __expf(x - m);
    if (L > 1) z += xor_lane<1>(z);
    if (L > 2) z += xor_lane<2>(z);
    if (L > 4) z += xor_lane<4>(z);
    if (L > 8) z += xor_lane<8>(z);
    if (L > 16) z += xor_lane<16>(z);
    if (L > 32) z += xor_lane<32>(z);
    const float ls = m == kNegInf ? kNegInf : m + __logf(z);
    if (live && l == 0) a.lsel[rowq] = ls;
    w[hh] = sel ? __expf(x - ls) : 0.f;
  }
  if (live && l < a.topk) {
    float* dst = a.wq + (rr * a.topk + l) * G;
    if constexpr (G % 4 == 0) {
#pragma unroll
      for (int q = 0; q < G; q += 4)
        *reinterpret_cast<float4*>(dst + q) = make_float4(w[q], w[q + 1], w[q + 2], w[q + 3]);
    } else {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) dst[hh] = w[hh];
    }
  }
}

// V^T of every chunk, [B, Hkv, ceil(T/S), D, S] with the tokens of a row in
// vt_token order; tokens past T are zero.  Lets the attention kernels stage V^T
// tiles with plain 16-byte copies.
template <typename T, int D>
__global__ __launch_bounds__(256) void vt_kernel(const T* __restrict__ v, T* __restrict__ vt, int Hkv,
                                                 int64_t T_, int64_t NCf) {
  constexpr int EPV = 16 / sizeof(T);
  constexpr int VP = D + EPV;   // padded LDS row
  __shared__ __align__(16) T tile[kS * VP];
  const int64_t c = blockIdx.x;
  const int g = blockIdx.y, b = blockIdx.z;
  const T* src = v + (((int64_t)b * Hkv + g) * T_ + c * kS) * D;
  for (int e = threadIdx.x; e < kS * D / EPV; e += 256) {
    const int row = e / (D / EPV), pc = e % (D / EPV);
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (c * kS + row < T_) u = *reinterpret_cast<const uint4*>(src + (int64_t)row * D + pc * EPV);
    *reinterpret_cast<uint4*>(tile + row * VP + pc * EPV) = u;
  }
  __syncthreads();
  T* dst = vt + (((int64_t)b * Hkv + g) * NCf + c) * D * kS;
  for (int e = threadIdx.x; e < D * kS / EPV; e += 256) {
    const int drow = e / (kS / EPV), q = e % (kS / EPV);
    T x[EPV];
#pragma unroll
    for (int t = 0; t < EPV; ++t) x[t] = tile[vt_token(q * EPV + t) * VP + drow];
    *reinterpret_cast<uint4*>(dst + (int64_t)drow * kS + q * EPV) = *reinterpret_cast<const uint4*>(x);
  }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct ChunkArgs {
  const void* q;    // [B, Hq, T, D]
  const void* k;
  const void* vt;   // V^T per chunk, [B, Hkv, NCf, D, S]
  const float* wq;  // [B, Hkv, T, topk, G] chunk weights
  const int32_t* bcount;
  const int64_t* bbase;
  const uint32_t* entries;
  void* part;   // [B, Hkv_pass, T, topk, G, D]
  const int32_t* smap;   // the workgroups' (chunk, range) words, sbound per (b, g)
  const int32_t* stot;
  int B, Hq, Hkv, topk, g0, gpass;
  int64_t T, NCs, NCf;
  float scale;
  int E;
  int64_t sbound;
};

// Selected chunks, chunk-major: one workgroup per (b, g, c).  The chunk's K and V
// are staged once; each wave takes 16-row tiles (16/G entries x G heads) of the
// entries that selected the chunk, with the next tile's q rows prefetched.  Each
// tile's weighted output goes through a wave-private LDS tile so that every
// partial row (d values) is written with contiguous 16-byte stores (pieces of
// rows written straight from the accumulators, 32 bytes per row and store,
// run three times slower).  Each wave holds the chunk's K fragments (the A
// operands of its score tiles) in registers for all of its tiles, so per tile
// only the V^T fragments and the output staging pass through LDS.
template <typename T> constexpr int chunk_waves() { return 4; }

template <typename T, int D, int G>
__device__ __forceinline__ void chunk_attend_body(const ChunkArgs& a) {
  constexpr int KS = D / 32, MD = D / 16;
  constexpr int NE = 16 / G;  // entries per 16-row tile
  constexpr int NW = chunk_waves<T>();
  constexpr int OP = D + 16 / (int)sizeof(T);  // padded LDS output row
  __shared__ __align__(16) T ks[kS * D];
  __shared__ __align__(16) T vt[D * kS];
  __shared__ __align__(16) T ot[NW][16 * OP];
  // group by group (one group's q, G rows of every query, fits the last-level
  // cache while its chunks gather them), and within a group the early chunks,
  // candidates of almost every query and so the longest lists, first
  // workgroup = one range of E entries of one chunk's list (long lists split, so
  // that a few of them do not outlast the rest of the grid)
  const int g = a.g0 + (int)(blockIdx.x / a.sbound), b = blockIdx.z;
  const int64_t bg = (int64_t)b * a.Hkv + g;
  const int64_t rr = blockIdx.x % a.sbound;
  if (rr >= a.stot[bg]) return;
  const int32_t word0 = a.smap[bg * a.sbound + rr];
  const int64_t c = word0 & 8191;
  const int e0 = (word0 >> 13) * a.E;
  const int64_t bucket = bg * a.NCs + c;
  const int n = min(a.bcount[bucket] - e0, a.E);
  if (n <= 0) return;
  const int64_t base = a.bbase[bucket] + e0;
  const T* kc = static_cast<const T*>(a.k) + (((int64_t)b * a.Hkv + g) * a.T + c * kS) * D;
  const T* vtc = static_cast<const T*>(a.vt) + (((int64_t)b * a.Hkv + g) * a.NCf + c) * D * kS;
  stage_chunk<T, D, NW * kWave>(kc, vtc, ks, vt, kS);
  __syncthreads();

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r16 = lane % 16, grp = lane / 16;
  const float sl2 = a.scale * kLog2e;
  const T* qbase = static_cast<const T*>(a.q);
  T* part = static_cast<T*>(a.part);
  T* myo = ot[wave];
  const int ntile = (n + NE - 1) / NE;
  const int hh = r16 % G, h = g * G + hh;

  // pipeline over this wave's tiles t, t+NW, ...: the entry word of tile t+3NW,
  // the q rows and weight of tile t+2NW (using the word loaded earlier), the
  // computation of tile t
  auto load_word = [&](int nt) -> uint32_t {
    const int e = nt * NE + r16 / G;
    return (nt < ntile && e < n) ? a.entries[base + e] : 0xffffffffu;
  };
  // A tile's q rows are read row-contiguous (PPR lanes on the 16-byte pieces of
  // a row, RPI rows per load, NI loads), so each load touches few cache lines
  // (one lane per row per load, as the fragments want them, costs a cache-line
  // lookup per lane), and become MFMA fragments through the wave's LDS tile.
  constexpr int EPV = 16 / (int)sizeof(T);
  constexpr int PPR = D / EPV, RPI = kWave / PPR, NI = 16 / RPI;
  const int qp = lane % PPR, qr = lane / PPR;
  auto load_q = [&](uint32_t word, uint4 (&raw)[NI], float& wt) {
    wt = word != 0xffffffffu
             ? a.wq[((((int64_t)b * a.Hkv + g) * a.T + (word >> 6)) * a.topk + (word & 63)) * G + hh]
             : 0.f;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int r = RPI * j + qr;                  // tile row: entry r / G, head r % G
      const uint32_t wr = __shfl(word, r, kWave);  // lanes r (< 16) hold row r's entry
      raw[j] = make_uint4(0u, 0u, 0u, 0u);
      if (wr != 0xffffffffu)
        raw[j] = *reinterpret_cast<const uint4*>(
            qbase + (((int64_t)b * a.Hq + g * G + r % G) * a.T + (wr >> 6)) * D + qp * EPV);
    }
  };
  auto to_frags = [&](const uint4 (&raw)[NI], Frag<T> (&f)[KS]) {
#pragma unroll
    for (int j = 0; j < NI; ++j)
      *reinterpret_cast<uint4*>(myo + (RPI * j + qr) * OP + qp * EPV) = raw[j];
    wave_lds_sync();
#pragma unroll
    for (int kq = 0; kq < KS; ++kq) load_frag(f[kq], myo + r16 * OP + 8 * grp + 32 * kq);
    wave_lds_sync();
  };

  constexpr int PKs = D / (16 / (int)sizeof(T));
  // q rows two of this wave's tiles ahead: the tile after next goes out while
  // this one computes (rb holds the next tile's rows, already in flight)
  Frag<T> bq[KS];
  uint4 ra[NI], rb[NI];
  uint32_t word = load_word(wave), wordn = load_word(wave + NW), wordnn = load_word(wave + 2 * NW);
  float wt, wtn, wtnn;
  load_q(word, ra, wt);
  load_q(wordn, rb, wtn);
  to_frags(ra, bq);
  for (int nt = wave; nt < ntile; nt += NW) {
    load_q(wordnn, ra, wtnn);              // the tile after next, in flight meanwhile
    const uint32_t word3 = load_word(nt + 3 * NW);
    f32x4_t acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      Frag<T> kf[KS];   // K rows 16 mt + r16, dims 32 kq + 8 grp .. + 7
#pragma unroll
      for (int kq = 0; kq < KS; ++kq) load_frag_swz<PKs>(kf[kq], ks, 16 * mt + r16, 8 * grp + 32 * kq);
      acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kq = 0; kq < KS; ++kq) mma(acc[mt], kf[kq], bq[kq]);
    }
    float mx = kNegInf;   // sl2 > 0: the max of the raw logits, scaled once
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) mx = fmaxf(mx, acc[mt][q4]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    mx *= sl2;
    float p[4][4], ls = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        p[mt][q4] = hw_exp2(fmaf(acc[mt][q4], sl2, -mx));
        ls += p[mt][q4];
      }
    ls += __shfl_xor(ls, 16, kWave);
    ls += __shfl_xor(ls, 32, kWave);
    f32x4_t o[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) o[md] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    pv_tile<T, D>(vt, p, o, r16, grp);
    const float w = wt / ls;   // exp(s_hat - L_sel) / Z_c (0 for padding rows)
#pragma unroll
    for (int md = 0; md < MD; ++md) store4<T>(myo + r16 * OP + 16 * md + 4 * grp, o[md], w);
    wave_lds_sync();
    // 16 rows x D values: PPR lanes store the 16-byte pieces of a row, RPI rows
    // per store
#pragma unroll
    for (int r0 = 0; r0 < 16; r0 += RPI) {
      const int r = r0 + qr, piece = qp;
      const uint32_t wr = __shfl(word, r, kWave);  // lanes r (< 16) hold row r's entry
      if (wr != 0xffffffffu) {
        const int rh = r % G;
        const int64_t ri = wr >> 6;
        const int rs = wr & 63;
        T* prow = part + (((((int64_t)b * a.gpass + (g - a.g0)) * a.T + ri) * a.topk + rs) * G + rh) * D;
        // streamed out: the fusion reads each partial row once, much later
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(myo + r * OP + piece * EPV),
                                    reinterpret_cast<u32x4*>(prow + piece * EPV));
      }
    }
    wave_lds_sync();
    to_frags(rb, bq);
#pragma unroll
    for (int j = 0; j < NI; ++j) rb[j] = ra[j];
    word = wordn;
    wordn = wordnn;
    wordnn = word3;
    wt = wtn;
    wtn = wtnn;
  }
}

// bf16 fits 168 VGPRs (three workgroups per compute unit); fp32 operands need
// the full register file.
template <typename T, int D, int G>
__global__ __launch_bounds__(chunk_waves<T>() * kWave) __attribute__((amdgpu_waves_per_eu(3))) void chunk_attend_kernel(ChunkArgs a) {
  chunk_attend_body<T, D, G>(a);
}
template <typename T, int D, int G>
__global__ __launch_bounds__(chunk_waves<T>() * kWave) void chunk_attend_kernel_f32(ChunkArgs a) {
  chunk_attend_body<T, D, G>(a);
}

struct WinArgs {
  const void* q;
  const void* k;
  const void* vt;        // V^T per chunk, [B, Hkv, NCf, D, S]
  const float* lsel;     // [B, Hq, T] L_sel (null: no selection)
  const int32_t* nvalid;  // [B, Hkv, T] selected slots of each row (a prefix)
  const void* part;      // this pass's weighted partials, [B, gpass, T, topk, G, D]
  void* out;             // [B, Hq, T, D]
  float* lse;            // [B, Hq, T] or null
  int B, Hq, Hkv, S, W, topk, g0, gpass;
  int64_t T, NCf;
  float scale;
};

template <int N> using u32v = uint32_t __attribute__((ext_vector_type(N)));

constexpr int kWinWaves = 8;
constexpr int kWinThreads = 64 * kWinWaves;
constexpr float kRefLog2 = -1e30f;   // initial softmax reference (log2 domain)
constexpr float kLazyLog2 = 8.f;     // headroom before the reference must move

// Window attention, query-major and dense (flash style).  A workgroup has 8 waves;
// a wave owns one 16-row MFMA tile of (query, head) rows, the block 128 rows, so
// each staged chunk serves 128 rows.  The next chunk's K and V^T pieces are
// loaded into registers (held as one vector value) while this chunk computes.
// Chunks fully inside every row's window skip the mask.
template <typename T, int D, int G>
__device__ __forceinline__ void window_body(const WinArgs& a) {
  constexpr int KS = D / 32, MD = D / 16;
  constexpr int EPV = 16 / sizeof(T);
  constexpr int PK = D / EPV, PV = kS / EPV;              // 16-byte pieces per K / V^T row
  constexpr int NPK = kS * PK / kWinThreads, NPV = D * PV / kWinThreads;
  constexpr int QW = 16 / G;        // queries per wave
  constexpr int QB = kWinWaves * QW;   // queries per block
  constexpr int NR = kWinWaves * 16;   // (query, head) rows per block
  // K and V^T tiles during the window loop, then the block's normalised window
  // outputs (NR rows of D) for the fusion epilogue
  __shared__ __align__(16) T tiles[2 * kS * D];
  __shared__ float lzs[NR];
  __shared__ float lss[NR];       // each row's L_sel
  __shared__ int32_t nvs[NR];     // each row's selected slots
  T* ks = tiles;
  T* vt = tiles + kS * D;
  const int g = a.g0 + (int)blockIdx.y, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r16 = lane % 16, grp = lane / 16;
  const int64_t T_ = a.T;
  // Consecutive query tiles share most window chunks: give each XCD (blocks are
  // dealt round-robin over the 8 XCDs) a contiguous run of tiles, so those tiles
  // meet in one L2.
  int64_t bx = blockIdx.x;
  if (gridDim.x % 8 == 0) bx = (int64_t)(blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  const int64_t qb0 = bx * QB;
  const int64_t qlast = min(qb0 + QB - 1, T_ - 1);
  const float sl2 = a.scale * kLog2e;

  const int64_t i = qb0 + wave * QW + r16 / G;   // this lane's row: query i, head h
  const int h = g * G + r16 % G;
  const int64_t lw = window_left(i, a.S, a.W);
  Frag<T> bq[KS];
  {
    const T* qrow = static_cast<const T*>(a.q) + (((int64_t)b * a.Hq + h) * T_ + min(i, T_ - 1)) * D + 8 * grp;
#pragma unroll
    for (int kq = 0; kq < KS; ++kq) load_frag(bq[kq], qrow + 32 * kq);
  }
  // Running reference in the log2 domain: finite, far below any logit, so the
  // first chunk with an unmasked token always moves it.
  float m = kRefLog2, ls = 0.f;
  f32x4_t o[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) o[md] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t lw_max = window_left(qlast, a.S, a.W);   // window edges grow with i
  const int64_t c_lo = window_left(qb0, a.S, a.W) / kS;
  const int64_t c_hi = qlast / kS;
  const T* kbase = static_cast<const T*>(a.k) + ((int64_t)b * a.Hkv + g) * T_ * D;
  const T* vtbase = static_cast<const T*>(a.vt) + ((int64_t)b * a.Hkv + g) * a.NCf * D * kS;
  u32v<4 * NPK> pk;
  u32v<4 * NPV> pv;
  auto fetch = [&](int64_t c) {
#pragma unroll
    for (int t = 0; t < NPK; ++t) {
      const int e = t * kWinThreads + threadIdx.x;
      const int row = e / PK, pc = e % PK;
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (c * kS + row < T_) u = *reinterpret_cast<const uint4*>(kbase + (c * kS + row) * D + pc * EPV);
      pk[4 * t] = u.x; pk[4 * t + 1] = u.y; pk[4 * t + 2] = u.z; pk[4 * t + 3] = u.w;
    }
#pragma unroll
    for (int t = 0; t < NPV; ++t) {
      const int e = t * kWinThreads + threadIdx.x;
      const int row = e / PV, pc = e % PV;
      const uint4 u = *reinterpret_cast<const uint4*>(vtbase + (c * D + row) * kS + pc * EPV);
      pv[4 * t] = u.x; pv[4 * t + 1] = u.y; pv[4 * t + 2] = u.z; pv[4 * t + 3] = u.w;
    }
  };
  auto commit = [&]() {
#pragma unroll
    for (int t = 0; t < NPK; ++t) {
      const int e = t * kWinThreads + threadIdx.x;
      *reinterpret_cast<uint4*>(ks + swz<PK>(e / PK, e % PK) * EPV) =
          make_uint4(pk[4 * t], pk[4 * t + 1], pk[4 * t + 2], pk[4 * t + 3]);
    }
#pragma unroll
    for (int t = 0; t < NPV; ++t) {
      const int e = t * kWinThreads + threadIdx.x;
      *reinterpret_cast<uint4*>(vt + swz<PV>(e / PV, e % PV) * EPV) =
          make_uint4(pv[4 * t], pv[4 * t + 1], pv[4 * t + 2], pv[4 * t + 3]);
    }
  };
  fetch(c_lo);
  for (int64_t c = c_lo; c <= c_hi; ++c) {
    __syncthreads();
    commit();
    __syncthreads();
    if (c < c_hi) fetch(c + 1);
    const int64_t j0 = c * kS;
    // no row masks a token of this chunk: its left edge is at or past every row's
    // window edge, and its last token precedes every row's query
    const bool full = j0 >= lw_max && j0 + kS - 1 <= qb0;
    f32x4_t acc[4];
    score_tile<T, D>(ks, bq, acc, r16, grp);
    if (!full) {
      const int lo = (int)max<int64_t>(lw - j0, -1);
      const int hi = i < T_ ? (int)min<int64_t>(i - j0, kS) : -1;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int t = 16 * mt + 4 * grp + q4;
          if (t < lo || t > hi) acc[mt][q4] = kNegInf;
        }
    }
    // Lazy rescaling: the running reference m moves only when some logit of the
    // wave exceeds it by more than kLazyLog2, so p = 2^(x - m) stays below
    // 2^kLazyLog2 and the usual per-chunk max exchange and O rescale are skipped
    // while the row maxima settle.  The final log-mass m + log2(l) is exact for
    // any m.  (sl2 > 0, so the max of the raw logits picks the max of x.)
    float mx = kNegInf;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) mx = fmaxf(mx, acc[mt][q4]);
    mx *= sl2;
    if (__any(mx > m + kLazyLog2)) {
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float mn = fmaxf(m, mx);
      const float alpha = hw_exp2(m - mn);   // 0 while m is still kRefLog2
      ls *= alpha;
#pragma unroll
      for (int md = 0; md < MD; ++md) o[md] *= alpha;
      m = mn;
    }
    float p[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        p[mt][q4] = hw_exp2(fmaf(acc[mt][q4], sl2, -m));   // masked: 2^-inf = 0
        ls += p[mt][q4];
      }
    pv_tile<T, D>(vt, p, o, r16, grp);
  }
  float lsum = ls;
  lsum += __shfl_xor(lsum, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);

  // Fusion (summary page, Methodology 2, Eq. 10, with the window at its
  // token-level log-mass): out = exp(log Z_win - L) o_win + exp(L_sel - L) *
  // (sum of the selected chunks' weighted partials), L = LSE(L_sel, log Z_win).
  // The normalised window rows go through LDS so that the partial rows, read
  // once here, are read with whole-wave contiguous 16-byte loads; meanwhile
  // another workgroup on the compute unit keeps the MFMA busy.
  const int rho = wave * 16 + r16;   // row (query, head) = (rho / G, rho % G) of the block
  __syncthreads();                   // every wave is done with the K / V^T tiles
  {
    const float inv = 1.f / lsum;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      const int d = 16 * md + 4 * grp;
      store4<T>(tiles + swz<PK>(rho, d / EPV) * EPV + d % EPV, o[md], inv);
    }
    if (grp == 0) lzs[rho] = (m + hw_log2(lsum)) * kLn2;
  }
  if (threadIdx.x < NR) {   // the rows' L_sel and selected slots, once per row
    const int rr = threadIdx.x;
    const int64_t iq = min<int64_t>(qb0 + rr / G, T_ - 1);
    lss[rr] = a.lsel ? a.lsel[((int64_t)b * a.Hq + g * G + rr % G) * T_ + iq] : kNegInf;
    nvs[rr] = a.lsel ? a.nvalid[((int64_t)b * a.Hkv + g) * T_ + iq] : 0;
  }
  __syncthreads();
  for (int it = threadIdx.x; it < NR * PK; it += kWinThreads) {
    const int rr = it / PK, pc = it % PK;
    const int64_t iq = qb0 + rr / G;
    if (iq >= T_) continue;
    const int hq = rr % G;
    const int64_t rowq = ((int64_t)b * a.Hq + g * G + hq) * T_ + iq;
    const float lz = lzs[rr];
    const float lsl = lss[rr];
    const float L = lsl == kNegInf ? lz : fmaxf(lsl, lz) + __logf(1.f + __expf(-fabsf(lsl - lz)));
    const float ww = __expf(lz - L);
    const float wsel = lsl == kNegInf ? 0.f : __expf(lsl - L);
    float ows[EPV], acc[EPV];
    {
      const uint4 u = *reinterpret_cast<const uint4*>(tiles + swz<PK>(rr, pc) * EPV);
      const T* t = reinterpret_cast<const T*>(&u);
#pragma unroll
      for (int e = 0; e < EPV; ++e) { ows[e] = to_f<T>(t[e]); acc[e] = 0.f; }
    }
    if (wsel > 0.f) {
      // the row's selected slots are its first nv (padding only at the end)
      const int nv = nvs[rr];
      const T* prow = static_cast<const T*>(a.part) +
                      ((((int64_t)b * a.gpass + (g - a.g0)) * T_ + iq) * a.topk * G + hq) * D + pc * EPV;
      // U slots' partial loads in flight together, with no load waiting on
      // another: a padding slot's partial row lies inside the buffer but holds no
      // value, so it is loaded and then dropped by a select
      constexpr int U = 16;
      for (int s = 0; s < a.topk; s += U) {
        uint4 u[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
          const bool in = s + j < a.topk;
          u32x4 v = u32x4{0u, 0u, 0u, 0u};   // read once: streamed past the caches
          if (in) v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(prow + (int64_t)(s + j) * G * D));
          u[j] = make_uint4(v[0], v[1], v[2], v[3]);
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
          const T* t = reinterpret_cast<const T*>(&u[j]);
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            const float f = to_f<T>(t[e]);
            acc[e] += s + j < nv ? f : 0.f;
          }
        }
      }
    }
    T res[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) res[e] = from_f<T>(ww * ows[e] + wsel * acc[e]);
    *reinterpret_cast<uint4*>(static_cast<T*>(a.out) + rowq * D + pc * EPV) = *reinterpret_cast<const uint4*>(res);
    if (a.lse && pc == 0) a.lse[rowq] = L;
  }
}

// bf16 tiles fit 128 VGPRs, so two workgroups share a compute unit and their
// barriers interleave; fp32 operands need the full register file.
template <typename T, int D, int G>
__global__ __launch_bounds__(kWinThreads) __attribute__((amdgpu_waves_per_eu(4))) void window_kernel(WinArgs a) {
  window_body<T, D, G>(a);
}
template <typename T, int D, int G>
__global__ __launch_bounds__(kWinThreads) void window_kernel_f32(WinArgs a) {
  window_body<T, D, G>(a);
}

template <typename T, int D, int G>
hipError_t launch_attend_tg(const AttArgs& a, const IdxArgs& ia, void* part, void* vt, int gpp,
                            hipStream_t st) {
  const int64_t NCf = (a.T + kS - 1) / kS;
  {
    KTimer tm(K_VT, st);
    hipLaunchKernelGGL((vt_kernel<T, D>), dim3((unsigned)NCf, a.Hkv, a.B), dim3(256), 0, st,
                       static_cast<const T*>(a.v), static_cast<T*>(vt), a.Hkv, a.T, NCf);
  }
  const bool chunks = ia.NCs > 0 && a.topk > 0;
  // per pass of KV groups: the selected chunks (chunk-major), then the window
  // with the fusion of that pass's partials
  for (int g0 = 0; g0 < a.Hkv; g0 += gpp) {
    const int gp = min(gpp, a.Hkv - g0);
    if (chunks) {
      ChunkArgs ca{a.q, a.k, vt, ia.wq, ia.bcount, ia.bbase, ia.entries, part, ia.smap, ia.stot,
                   a.B, a.Hq, a.Hkv, a.topk, g0, gpp, a.T, ia.NCs, NCf, a.scale, ia.E, ia.sbound};
      KTimer tm(K_CHUNK_ATTEND, st);
      const dim3 grid((unsigned)(ia.sbound * gp), 1, a.B);
      if constexpr (sizeof(T) == 2)
        hipLaunchKernelGGL((chunk_attend_kernel<T, D, G>), grid, dim3(chunk_waves<T>() * kWave), 0, st, ca);
      else
        hipLaunchKernelGGL((chunk_attend_kernel_f32<T, D, G>), grid, dim3(chunk_waves<T>() * kWave), 0, st, ca);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    WinArgs wa{a.q, a.k, vt, chunks ? ia.lsel : nullptr, ia.nvalid, part, a.out, a.lse,
               a.B, a.Hq, a.Hkv, a.S, a.W, a.topk, g0, gpp, a.T, NCf, a.scale};
    const int QB = kWinWaves * (16 / G);
    const dim3 grid((unsigned)((a.T + QB - 1) / QB), (unsigned)gp, a.B);
    KTimer tm(K_WINDOW, st);
    if constexpr (sizeof(T) == 2)
      hipLaunchKernelGGL((window_kernel<T, D, G>), grid, dim3(kWinThreads), 0, st, wa);
    else
      hipLaunchKernelGGL((window_kernel_f32<T, D, G>), grid, dim3(kWinThreads), 0, st, wa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int D>
hipError_t launch_attend_t(const AttArgs& a, const IdxArgs& ia, void* part, void* vt, int gpp,
                           hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_attend_tg<T, D, 1>(a, ia, part, vt, gpp, st);
    case 2: return launch_attend_tg<T, D, 2>(a, ia, part, vt, gpp, st);
    case 4: return launch_attend_tg<T, D, 4>(a, ia, part, vt, gpp, st);
    default: return launch_attend_tg<T, D, 8>(a, ia, part, vt, gpp, st);
  }
}

// The fill: staged in LDS when a tile's entries and the per-chunk state fit
// (for example up to 2048 chunks with tiles of 1024 queries and k = 32), else
// with direct scatters.
void launch_idx_fill(const IdxArgs& ia, hipStream_t st) {
  const size_t lds = (size_t)ia.NCs * (sizeof(uint64_t) + sizeof(int32_t));
  const size_t staged = lds + (size_t)ia.tile * ia.topk * sizeof(uint32_t);
  KTimer tm(K_IDX_FILL, st);
  if (staged + 256 <= kMaxLds)   // + the kernel's static LDS
    hipLaunchKernelGGL(idx_fill_staged_kernel, dim3((unsigned)ia.ntiles, ia.Hkv, ia.B), dim3(1024), staged, st,
                       ia);
  else
    hipLaunchKernelGGL(idx_fill_kernel, dim3((unsigned)ia.ntiles, ia.Hkv, ia.B), dim3(256), lds, st, ia);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// The chunk pass's workgroups: each takes one range of E entries of a chunk's
// list, E a multiple of 64, at least 256 and large enough that all (b, g) make
// about 6144 ranges of the T * topk entries each (so long lists cannot outlast
// the grid, and short sequences still fill the chip).  Per (b, g) at most
// sum_c ceil(n_c / E) <= NC + T * topk / E workgroups.
void chunk_split(int B, int Hkv, int64_t T, int64_t NCs, int topk, int* E, int64_t* bound) {
  const int64_t total = (int64_t)B * Hkv * T * topk;
  int64_t e = (total + 6143) / 6144;
  e = (e + 63) / 64 * 64;
  if (e < 256) e = 256;
  *E = (int)e;
  *bound = NCs + (T * topk + e - 1) / e;
}

void attend_workspace(int B, int Hq, int Hkv, int64_t T, int S, int D, int topk, bool bf16,
                      size_t* fixed, size_t* per_kv_head) {
  const int64_t NCs = T / S;
  const int tile = idx_tile(B, Hkv, T);
  const int64_t ntiles = (T + tile - 1) / tile;
  const size_t esz = bf16 ? 2 : 4;
  size_t f = 0;
  f += align256((size_t)B * Hkv * ntiles * NCs * sizeof(int32_t));  // tile_cnt
  f += align256((size_t)B * Hkv * NCs * sizeof(int32_t));           // bcount
  f += align256((size_t)B * Hkv * NCs * sizeof(int64_t));           // bbase
  f += align256((size_t)B * Hkv * T * topk * sizeof(uint32_t));     // entries
  f += align256((size_t)B * Hq * T * topk * sizeof(float));         // chunk weights
  f += align256((size_t)B * Hq * T * sizeof(float));                // lsel
  f += align256((size_t)B * Hkv * T * sizeof(int32_t));             // selected slots per row
  f += align256((size_t)B * Hkv * ((T + kS - 1) / kS) * kS * D * esz);  // V^T per chunk
  int E;
  int64_t sbound;
  chunk_split(B, Hkv, T, NCs, topk > 0 ? topk : 1, &E, &sbound);
  f += align256((size_t)B * Hkv * sbound * sizeof(int32_t));         // chunk-pass workgroup map
  f += align256((size_t)B * Hkv * sizeof(int32_t));                  // its counts
  *fixed = f + 256;
  *per_kv_head = align256((size_t)B * (Hq / Hkv) * T * topk * D * esz);
}

size_t entry_lists_bytes(int B, int Hkv, int64_t T, int S, int topk) {
  const int64_t NCs = T / S;
  const int tile = idx_tile(B, Hkv, T);
  const int64_t ntiles = (T + tile - 1) / tile;
  return align256((size_t)B * Hkv * ntiles * NCs * sizeof(int32_t)) +
         align256((size_t)B * Hkv * NCs * sizeof(int32_t)) + align256((size_t)B * Hkv * NCs * sizeof(int64_t)) +
         align256((size_t)B * Hkv * T * topk * sizeof(uint32_t));
}

hipError_t launch_entry_lists(const int32_t* idx, int B, int Hq, int Hkv, int64_t T, int S, int topk,
                              void* ws, EntryLists* el, hipStream_t st) {
  const int64_t NCs = T / S;
  const int tile = idx_tile(B, Hkv, T);
  const int64_t ntiles = (T + tile - 1) / tile;
  char* w = static_cast<char*>(ws);
  IdxArgs ia{};
  ia.idx = idx;
  ia.tile_cnt = reinterpret_cast<int32_t*>(w);
  w += align256((size_t)B * Hkv * ntiles * NCs * sizeof(int32_t));
  ia.bcount = reinterpret_cast<int32_t*>(w);
  w += align256((size_t)B * Hkv * NCs * sizeof(int32_t));
  ia.bbase = reinterpret_cast<int64_t*>(w);
  w += align256((size_t)B * Hkv * NCs * sizeof(int64_t));
  ia.entries = reinterpret_cast<uint32_t*>(w);
  ia.B = B; ia.Hq = Hq; ia.Hkv = Hkv; ia.topk = topk;
  ia.T = T; ia.NCs = NCs; ia.ntiles = ntiles; ia.tile = tile;
  el->bcount = ia.bcount;
  el->bbase = ia.bbase;
  el->entries = ia.entries;
  el->NCs = NCs;
  if (topk == 0 || NCs == 0) return hipSuccess;
  const size_t lds = (size_t)NCs * sizeof(uint64_t);
  {
    KTimer tm(K_IDX_COUNT, st);
    hipLaunchKernelGGL(idx_count_kernel, dim3((unsigned)ntiles, Hkv, B), dim3(512),
                       lds + (size_t)NCs * sizeof(int32_t), st, ia);
  }
  {
    KTimer tm(K_IDX_SCAN_TILES, st);
    hipLaunchKernelGGL(idx_scan_tiles_kernel, dim3((unsigned)((NCs + 31) / 32), B * Hkv), dim3(1024), 0, st, ia);
  }
  {
    KTimer tm(K_IDX_SCAN_BUCKETS, st);
    hipLaunchKernelGGL(idx_scan_buckets_kernel, dim3(1), dim3(1024), 0, st, ia);
  }
  launch_idx_fill(ia, st);
  return hipGetLastError();
}

hipError_t launch_attend(const AttArgs& a, hipStream_t st) {
  size_t fixed, per;
  attend_workspace(a.B, a.Hq, a.Hkv, a.T, a.S, a.D, a.topk, a.bf16, &fixed, &per);
  const int64_t NCs = a.T / a.S;
  const int tile = idx_tile(a.B, a.Hkv, a.T);
  const int64_t ntiles = (a.T + tile - 1) / tile;
  const size_t esz = a.bf16 ? 2 : 4;
  char* w = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(a.ws) + 255) & ~(uintptr_t)255);
  IdxArgs ia{};
  ia.idx = a.idx;
  ia.ssel = a.ssel;
  ia.tile_cnt = reinterpret_cast<int32_t*>(w);
  w += align256((size_t)a.B * a.Hkv * ntiles * NCs * sizeof(int32_t));
  ia.bcount = reinterpret_cast<int32_t*>(w);
  w += align256((size_t)a.B * a.Hkv * NCs * sizeof(int32_t));
  ia.bbase = reinterpret_cast<int64_t*>(w);
  w += align256((size_t)a.B * a.Hkv * NCs * sizeof(int64_t));
  ia.entries = reinterpret_cast<uint32_t*>(w);
  w += align256((size_t)a.B * a.Hkv * a.T * a.topk * sizeof(uint32_t));
  ia.wq = reinterpret_cast<float*>(w);
  w += align256((size_t)a.B * a.Hq * a.T * a.topk * sizeof(float));
  ia.lsel = reinterpret_cast<float*>(w);
  w += align256((size_t)a.B * a.Hq * a.T * sizeof(float));
  ia.nvalid = reinterpret_cast<int32_t*>(w);
  w += align256((size_t)a.B * a.Hkv * a.T * sizeof(int32_t));
  void* vt = w;
  w += align256((size_t)a.B * a.Hkv * ((a.T + kS - 1) / kS) * kS * a.D * esz);
  chunk_split(a.B, a.Hkv, a.T, NCs, a.topk > 0 ? a.topk : 1, &ia.E, &ia.sbound);
  ia.smap = reinterpret_cast<int32_t*>(w);
  w += align256((size_t)a.B * a.Hkv * ia.sbound * sizeof(int32_t));
  ia.stot = reinterpret_cast<int32_t*>(w);
  w += align256((size_t)a.B * a.Hkv * sizeof(int32_t));
  ia.B = a.B; ia.Hq = a.Hq; ia.Hkv = a.Hkv; ia.topk = a.topk;
  ia.T = a.T; ia.NCs = NCs; ia.ntiles = ntiles; ia.tile = tile;
  void* part = w;
  const size_t avail = a.ws_bytes - fixed;
  int gpp = per > 0 ? (int)(avail / per) : a.Hkv;  // k = 0 needs no partial outputs
  if (gpp > a.Hkv) gpp = a.Hkv;
  if (gpp < 1) gpp = 1;  // the host checked the minimum size

  if (a.topk > 0) {
    int L = 1;
    while (L < a.topk) L <<= 1;
    const int64_t nl = (int64_t)a.B * a.Hkv * a.T * L;
    const dim3 grid((unsigned)((nl + 255) / 256));
    const int G = a.Hq / a.Hkv;
    const int nqp = L / 4;   // lanes per head with four slots each
    const int64_t nrows = (int64_t)a.B * a.Hkv * a.T;
    KTimer tm(K_LSEL, st);
    if (a.topk % 4 == 0 && nqp >= 1 && G * nqp <= kWave) {
      const int rpb = 4 * (kWave / (G * nqp));   // rows per block of four waves
      const dim3 g4((unsigned)((nrows + rpb - 1) / rpb));
      switch (G * 100 + nqp) {
        case 101: hipLaunchKernelGGL((lsel4_kernel<1, 1>), g4, dim3(256), 0, st, ia); break;
        case 102: hipLaunchKernelGGL((lsel4_kernel<1, 2>), g4, dim3(256), 0, st, ia); break;
        case 104: hipLaunchKernelGGL((lsel4_kernel<1, 4>), g4, dim3(256), 0, st, ia); break;
        case 108: hipLaunchKernelGGL((lsel4_kernel<1, 8>), g4, dim3(256), 0, st, ia); break;
        case 116: hipLaunchKernelGGL((lsel4_kernel<1, 16>), g4, dim3(256), 0, st, ia); break;
        case 201: hipLaunchKernelGGL((lsel4_kernel<2, 1>), g4, dim3(256), 0, st, ia); break;
        case 202: hipLaunchKernelGGL((lsel4_kernel<2, 2>), g4, dim3(256), 0, st, ia); break;
        case 204: hipLaunchKernelGGL((lsel4_kernel<2, 4>), g4, dim3(256), 0, st, ia); break;
        case 208: hipLaunchKernelGGL((lsel4_kernel<2, 8>), g4, dim3(256), 0, st, ia); break;
        case 216: hipLaunchKernelGGL((lsel4_kernel<2, 16>), g4, dim3(256), 0, st, ia); break;
        case 401: hipLaunchKernelGGL((lsel4_kernel<4, 1>), g4, dim3(256), 0, st, ia); break;
        case 402: hipLaunchKernelGGL((lsel4_kernel<4, 2>), g4, dim3(256), 0, st, ia); break;
        case 404: hipLaunchKernelGGL((lsel4_kernel<4, 4>), g4, dim3(256), 0, st, ia); break;
        case 408: hipLaunchKernelGGL((lsel4_kernel<4, 8>), g4, dim3(256), 0, st, ia); break;
        case 416: hipLaunchKernelGGL((lsel4_kernel<4, 16>), g4, dim3(256), 0, st, ia); break;
        case 801: hipLaunchKernelGGL((lsel4_kernel<8, 1>), g4, dim3(256), 0, st, ia); break;
        case 802: hipLaunchKernelGGL((lsel4_kernel<8, 2>), g4, dim3(256), 0, st, ia); break;
        case 804: hipLaunchKernelGGL((lsel4_kernel<8, 4>), g4, dim3(256), 0, st, ia); break;
        default: hipLaunchKernelGGL((lsel4_kernel<8, 8>), g4, dim3(256), 0, st, ia); break;
      }
    } else {
      switch (G) {
        case 1: hipLaunchKernelGGL(lsel_kernel<1>, grid, dim3(256), 0, st, ia, L); break;
        case 2: hipLaunchKernelGGL(lsel_kernel<2>, grid, dim3(256), 0, st, ia, L); break;
        case 4: hipLaunchKernelGGL(lsel_kernel<4>, grid, dim3(256), 0, st, ia, L); break;
        default: hipLaunchKernelGGL(lsel_kernel<8>, grid, dim3(256), 0, st, ia, L); break;
      }
    }
  } else {
    ia.lsel = nullptr;  // no selection: the window is the whole normaliser
  }
  if (a.topk > 0 && NCs > 0) {
    const size_t lds = (size_t)NCs * sizeof(uint64_t);
    {
      KTimer tm(K_IDX_COUNT, st);
      hipLaunchKernelGGL(idx_count_kernel, dim3((unsigned)ntiles, a.Hkv, a.B), dim3(512),
                         lds + (size_t)NCs * sizeof(int32_t), st, ia);
    }
    {
      KTimer tm(K_IDX_SCAN_TILES, st);
      hipLaunchKernelGGL(idx_scan_tiles_kernel, dim3((unsigned)((NCs + 31) / 32), a.B * a.Hkv),
                         dim3(1024), 0, st, ia);
    }
    {
      KTimer tm(K_IDX_SCAN_BUCKETS, st);
      hipLaunchKernelGGL(idx_scan_buckets_kernel, dim3(1), dim3(1024), 0, st, ia);
    }
    launch_idx_fill(ia, st);
    KTimer tm(K_IDX_SCAN_BUCKETS, st);
    hipLaunchKernelGGL(split_map_kernel, dim3((unsigned)(a.B * a.Hkv)), dim3(1024), 0, st, ia);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.bf16) return a.D == 128 ? launch_attend_t<bf16_t, 128>(a, ia, part, vt, gpp, st) : launch_attend_t<bf16_t, 64>(a, ia, part, vt, gpp, st);
  return a.D == 128 ? launch_attend_t<float, 128>(a, ia, part, vt, gpp, st) : launch_attend_t<float, 64>(a, ia, part, vt, gpp, st);
}

}  // namespace hils
