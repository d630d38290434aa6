// topk.h -- exact wave-level top-k of 32-bit rank keys (gfx950, wave64).
//
// A rank key is the order-preserving unsigned image of an fp32 score (larger
// score -> larger key; 0 marks an absent candidate).  A wave holds the keys of
// up to 64*J candidates, J per lane, candidate id lane + 64*j.  The k-th largest
// key K is found with ballot counts only:
//   1. theta = the k-th largest of the 64 lane maxima, bit by bit from the top;
//      the k lanes with the largest maxima hold k keys >= theta, so theta <= K;
//   2. the keys >= theta are compacted one per lane with their ids (through
//      wave-private LDS); when at most 64 reach theta, K is the k-th largest of
//      those, again bit by bit, and the choice is made among them; otherwise K
//      is found the same way over all keys;
//   3. every key above K is chosen, plus the lowest-id keys equal to K up to k,
//      so ties at the k-th key go to the lower chunk id, and the chosen ids are
//      written in ascending order with ballot prefix counts.
#pragma once

#include "hils_common.h"

namespace hils {

__device__ __forceinline__ int lane_prefix(uint64_t mask, int lane) {
  return __popcll(mask & ((1ull << lane) - 1ull));
}
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The topk-th largest of one value per lane (with multiplicity), found bit by
// bit from the top: the largest t with count(x >= t) >= topk.  Only ballots and
// scalar counts, no cross-lane data movement.  (Starting below the bits that the
// wave's smallest and largest values share saves steps but measured slower: the
// two wave reductions and the data-dependent loop cost more than the steps.)
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
// uint32 in LDS; out: 64 entries (it holds the compacted ids on the way).
//   1. theta = the k-th largest of the 64 per-lane maxima: a lower bound of the
//      k-th largest key K (the k lanes with the largest maxima hold k keys >= theta);
//   2. the keys reaching theta are compacted in id order with their ids (the
//      first 64 of them).  If at most 64 reach it, every chosen key is among
//      them: K is their k-th largest and the choice is made on that one lane's
//      worth; otherwise K is found over all keys, bit by bit;
//   3. every key above K is chosen, plus the lowest-id keys equal to K up to k.
template <int J>
__device__ void wave_topk_u32(const uint32_t (&keys)[J], int jn, int topk, int lane, uint32_t* buf,
                              int32_t* out, uint32_t* out_keys = nullptr) {
  if (jn == 1) {   // one key per lane: K directly, no bound needed
    const uint32_t x = keys[0];
    const uint32_t kstar = wave_kth_lane_u32(x, topk);
    const int need = topk - __popcll(__ballot(x > kstar));
    const uint64_t meq = __ballot(x == kstar);
    const bool sel = x > kstar || (x == kstar && lane_prefix(meq, lane) < need);
    const uint64_t m = __ballot(sel);
    if (sel) {
      const int pos = lane_prefix(m, lane);
      out[pos] = lane;
      if (out_keys) out_keys[pos] = x;
    }
    return;
  }
  uint32_t lm = 0;
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (j < jn) lm = keys[j] > lm ? keys[j] : lm;
  const uint32_t theta = wave_kth_lane_u32(lm, topk);   // >= 1: more than topk keys present
  int total = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (j < jn) {
      const bool s = keys[j] >= theta;
      const uint64_t m = __ballot(s);
      if (s) {
        const int pos = total + lane_prefix(m, lane);
        if (pos < kWave) {
          buf[pos] = keys[j];
          out[pos] = lane + 64 * j;
        }
      }
      total += __popcll(m);
    }
  }
  if (total <= kWave) {
    wave_lds_sync();
    const uint32_t x = lane < total ? buf[lane] : 0u;
    const int32_t id = lane < total ? out[lane] : -1;
    wave_lds_sync();
    const uint32_t kstar = wave_kth_lane_u32(x, topk);
    const int need = topk - __popcll(__ballot(x > kstar));   // ties at kstar to take, lowest ids first
    const uint64_t meq = __ballot(x == kstar);
    const bool sel = x > kstar || (x == kstar && lane_prefix(meq, lane) < need);
    const uint64_t m = __ballot(sel);
    if (sel) {
      const int pos = lane_prefix(m, lane);
      out[pos] = id;
      if (out_keys) out_keys[pos] = x;
    }
    return;
  }
  uint32_t kstar = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = kstar | (1u << bit);
    int n = 0;
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (j < jn) n += __popcll(__ballot(keys[j] >= c));
    if (n >= topk) kstar = c;
  }
  int gt = 0;
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (j < jn) gt += __popcll(__ballot(keys[j] > kstar));
  const int need = topk - gt;   // ties at kstar to take, lowest ids first
  int base = 0, eq_seen = 0;
  wave_lds_sync();   // out held compacted ids above
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

// The top-k (lists of at most 64) as keys and positions of n <= 64*J keys held J
// per lane at position lane + 64 j; fewer than or exactly k present: all of them.
// Writes n_out entries ascending by position.
template <int J>
__device__ __forceinline__ int list_topk(const uint32_t (&keys)[J], int jn, int npresent, int topk,
                                         int lane, uint32_t* sbuf, int32_t* opos, uint32_t* okey) {
  if (npresent > topk) {
    wave_topk_u32<J>(keys, jn, topk, lane, sbuf, opos, okey);
    return topk;
  }
  int base = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (j < jn) {
      const bool s = keys[j] != 0u;
      const uint64_t msk = __ballot(s);
      if (s) {
        const int ps = base + lane_prefix(msk, lane);
        opos[ps] = lane + 64 * j;
        okey[ps] = keys[j];
      }
      base += __popcll(msk);
    }
  }
  return base;
}

}  // namespace hils
