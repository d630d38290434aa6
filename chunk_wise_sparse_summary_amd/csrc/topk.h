// topk.h -- wave-level exact top-k over 64-bit keys (gfx950, wave64).
//
// A candidate's key packs its rank key and chunk id as key32 << 32 | ~chunk, so
// distinct candidates have distinct keys and "larger key" means "larger rank key,
// or equal rank key and lower chunk id" -- ties go to the lower chunk.  Key 0
// marks an absent candidate (every real key is larger).  A wave holds J keys per
// lane; the k-th largest key is found as follows:
//   1. theta = the k-th largest of the 64 per-lane maxima.  The k lanes with the
//      largest maxima hold k distinct keys >= theta, so theta is a lower bound of
//      the k-th largest key.
//   2. If at most 64 keys reach theta, they are compacted one per lane and
//      bitonic-sorted across the wave; the k-th of them is the answer.
//   3. Otherwise the answer is found exactly by bisection on the key value,
//      counting keys >= mid with a wave reduction.
#pragma once

#include "hils_common.h"

namespace hils {

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = __shfl((uint32_t)v, src, kWave);
  const uint32_t hi = __shfl((uint32_t)(v >> 32), src, kWave);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  const uint32_t lo = __shfl_xor((uint32_t)v, o, kWave);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// One value per lane, sorted descending (desc = true) or ascending across the wave.
template <typename V>
__device__ __forceinline__ V bitonic_sort64(V v, int lane, bool desc_order) {
#pragma unroll
  for (int kk = 2; kk <= 64; kk <<= 1) {
#pragma unroll
    for (int j = kk >> 1; j > 0; j >>= 1) {
      V p;
      if constexpr (sizeof(V) == 8) p = shfl_xor_u64(v, j);
      else p = __shfl_xor(v, j, kWave);
      const bool seg = ((lane & kk) == 0) == desc_order;
      const bool lower = (lane & j) == 0;
      v = (lower == seg) ? (v > p ? v : p) : (v < p ? v : p);
    }
  }
  return v;
}

__device__ __forceinline__ uint64_t full_key(uint32_t key, int64_t c) {
  return ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - (uint32_t)c);
}
__device__ __forceinline__ int32_t key_chunk(uint64_t v) {
  return (int32_t)(0xffffffffu - (uint32_t)v);
}
__device__ __forceinline__ int lane_prefix(uint64_t mask, int lane) {
  return __popcll(mask & ((1ull << lane) - 1ull));
}
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The topk-th largest of the wave's keys (there must be more than topk present).
// buf: 64 wave-private uint64 in LDS.
template <int J>
__device__ uint64_t wave_kth_u64(const uint64_t (&v)[J], int topk, int lane, uint64_t* buf) {
  uint64_t lm = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) lm = v[j] > lm ? v[j] : lm;
  const uint64_t srt = bitonic_sort64<uint64_t>(lm, lane, true);
  const uint64_t theta = shfl_u64(srt, topk - 1);
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) cnt += (v[j] != 0 && v[j] >= theta) ? 1 : 0;
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += x;
  }
  const int total = __shfl(incl, 63, kWave);
  if (total <= 64) {
    int pos = incl - cnt;
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (v[j] != 0 && v[j] >= theta) buf[pos++] = v[j];
    wave_lds_sync();
    const uint64_t x = lane < total ? buf[lane] : 0ull;
    wave_lds_sync();
    const uint64_t sx = bitonic_sort64<uint64_t>(x, lane, true);
    return shfl_u64(sx, topk - 1);
  }
  // bisection: largest t with count(keys >= t) >= topk
  uint64_t lo = theta > 0 ? theta : 1, hi = shfl_u64(srt, 0);
  while (lo < hi) {
    const uint64_t mid = lo + ((hi - lo + 1) >> 1);
    int c = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) c += v[j] >= mid ? 1 : 0;
    if (wave_sum_i(c) >= topk) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Keys held as candidate lane + 64*j (ascending chunk order): write the chunk ids
// of keys >= thr in ascending order to out[].
template <int J>
__device__ __forceinline__ void emit_ascending(const uint64_t (&v)[J], uint64_t thr, int lane,
                                               int32_t* out) {
  int base = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const bool sel = v[j] != 0 && v[j] >= thr;
    const uint64_t m = __ballot(sel);
    if (sel) out[base + lane_prefix(m, lane)] = key_chunk(v[j]);
    base += __popcll(m);
  }
}

// The topk-th largest of one value per lane (with multiplicity), found bit by
// bit from the top: the largest t with count(x >= t) >= topk.  Only ballots and
// scalar counts, no cross-lane data movement.
__device__ __forceinline__ uint32_t wave_kth_lane_u32(uint32_t x, int topk) {
  uint32_t t = 0;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = t | (1u << bit);
    if (__popcll(__ballot(x >= c)) >= topk) t = c;
  }
  return t;
}

// Exact top-k of 32-bit rank keys held J per lane, candidate id lane + 64*j
// (key 0 = absent; keys[j] for j >= jn are all absent), more than topk present.
// Ties at the k-th key go to the lower ids.  Writes the chosen ids ascending to
// out[0..topk) (and their keys to out_keys, if given).  buf: 64 wave-private
// uint32 in LDS.
//   1. theta = the k-th largest of the 64 per-lane maxima: a lower bound of the
//      k-th largest key K (the k lanes with the largest maxima hold k keys >= theta);
//   2. if at most 64 keys reach theta they are compacted one per lane and K is
//      the k-th largest of those; otherwise K is found over all keys, bit by bit;
//   3. every key above K is chosen, plus the lowest-id keys equal to K up to k.
template <int J>
__device__ void wave_topk_u32(const uint32_t (&keys)[J], int jn, int topk, int lane, uint32_t* buf,
                              int32_t* out, uint32_t* out_keys = nullptr) {
  uint32_t lm = 0;
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (j < jn) lm = keys[j] > lm ? keys[j] : lm;
  const uint32_t theta = wave_kth_lane_u32(lm, topk);   // >= 1: more than topk keys present
  int total = 0;
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (j < jn) total += __popcll(__ballot(keys[j] >= theta));
  uint32_t kstar;
  if (total <= 64) {
    int base = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (j < jn) {
        const bool s = keys[j] >= theta;
        const uint64_t m = __ballot(s);
        if (s) buf[base + lane_prefix(m, lane)] = keys[j];
        base += __popcll(m);
      }
    }
    wave_lds_sync();
    const uint32_t x = lane < total ? buf[lane] : 0u;
    wave_lds_sync();
    kstar = wave_kth_lane_u32(x, topk);
  } else {
    kstar = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = kstar | (1u << bit);
      int n = 0;
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (j < jn) n += __popcll(__ballot(keys[j] >= c));
      if (n >= topk) kstar = c;
    }
  }
  int gt = 0;
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (j < jn) gt += __popcll(__ballot(keys[j] > kstar));
  const int need = topk - gt;   // ties at kstar to take, lowest ids first
  int base = 0, eq_seen = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (j < jn) {
      const bool eq = keys[j] == kstar;
      const uint64_t meq = __ballot(eq);
      const bool sel = keys[j] > kstar || (eq && eq_seen + lane_prefix(meq, lane) < need);
      eq_seen += __popcll(meq);
      const uint64_t m = __ballot(sel);
      if (sel) {
        const int pos = base + lane_prefix(m, lane);
        out[pos] = lane + 64 * j;
        if (out_keys) out_keys[pos] = keys[j];
      }
      base += __popcll(m);
    }
  }
}

}  // namespace hils
