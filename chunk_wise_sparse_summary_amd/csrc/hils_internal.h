// hils_internal.h -- launch interfaces between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hils_common.h"

namespace hils {

// Landmark summaries for a contiguous chunk range of every (b, head), or (decode)
// for a list of (b, chunk) pairs whose landmark queries come from a [B, Hq, d] array.
struct SumList {
  int32_t n;
  int32_t b[64];
  int64_t c[64];
};

struct SumArgs {
  const void* k;
  const void* ql;
  void* ksum;
  float* bsum;
  int B, Hq, Hkv, D;
  bool bf16;
  int64_t kT;      // key rows per KV head
  int64_t NCs;     // chunks per head in ksum / bsum
  int64_t ql_sb, ql_sh, ql_sc;  // landmark query strides (elements) per b, head, chunk
  int64_t c0, n_chunks;         // range mode
  float scale;
  SumList list;                 // list mode when list.n > 0
};
hipError_t launch_summarize(const SumArgs& a, hipStream_t st);

// The low-rank query calibration fused into the selection's first scoring pass.
struct QcFuse {
  const void* q;     // [B, Hq, T, D] token queries
  const float* z;    // [B, T, r] W_down h, fp32
  const void* wu;    // [Hq, D, r]
  void* qh;          // [B, Hq, T, D] q_hat, written by the pass (the same buffer as SelArgs::qh)
};

struct SelArgs {
  const void* qh;
  const void* ksum;
  const float* bsum;
  int32_t* idx;
  float* ssel;
  float* L;          // [B, Hq, T] scratch (G > 1)
  float* scratch;    // rank keys of gpass (b, group) pairs, group_words apart:
                     // n_slots rows of slot_stride each
  int B, Hq, Hkv, D, S, W, topk;
  bool bf16;
  int64_t T, NCs;
  float scale;
  int n_slots;
  int64_t slot_stride;  // keys per row
  int gpass;            // (b, group) pairs per launch
  int64_t group_words;  // keys of one (b, group), padded
  QcFuse qc{};          // used when qc_r > 0
  int qc_r = 0;         // rank of the fused Q-Cal, 0: q_hat is an input
};
hipError_t launch_select(const SelArgs& a, hipStream_t st);
// Naive BSA selection: SelArgs with qh = the token query q, ksum = the keys k,
// bsum unused and ssel = nullptr; the same workspace layout as the selection.
hipError_t launch_bsa_select(const SelArgs& a, hipStream_t st);
hipError_t launch_overlap(const int32_t* ia, const int32_t* ib, int32_t* cnt, int64_t nrows, int topk,
                          hipStream_t st);
// Bytes for every (b, group) at once; a workspace of fixed + k * per_group
// bytes (k >= 1) runs the selection k pairs per launch.
size_t select_workspace(int B, int Hq, int Hkv, int64_t T, int S, bool bf16, int* n_slots,
                        int64_t* slot_stride, size_t* fixed = nullptr, size_t* per_group = nullptr);

struct AttArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;
  const float* ssel;
  void* out;
  float* lse;
  int B, Hq, Hkv, D, S, W, topk;
  bool bf16;
  int64_t T;
  float scale;
  void* ws;
  size_t ws_bytes;
};
hipError_t launch_attend(const AttArgs& a, hipStream_t st);
// Bytes for the index structures (fixed part) and for partial outputs of one KV head.
void attend_workspace(int B, int Hq, int Hkv, int64_t T, int S, int D, int topk, bool bf16,
                      size_t* fixed, size_t* per_kv_head);

// Per-(b, group, chunk) lists of the (query, slot) entries that selected the
// chunk (entry word i * 64 + slot), in ascending query order: bucket (b, g, c)
// holds entries[bbase[.] .. bbase[.] + bcount[.]).
struct EntryLists {
  const int32_t* bcount;
  const int64_t* bbase;
  const uint32_t* entries;
  int64_t NCs;
};
size_t entry_lists_bytes(int B, int Hkv, int64_t T, int S, int topk);
hipError_t launch_entry_lists(const int32_t* idx, int B, int Hq, int Hkv, int64_t T, int S, int topk,
                              void* ws, EntryLists* el, hipStream_t st);

// Backward of the prefill attention and fusion (gradients in fp32).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* qh;
  const void* ksum;
  const int32_t* idx;
  const float* ssel;
  const void* out;
  const float* lse;
  const void* dout;
  const float* dlse;
  float* dq;
  float* dk;
  float* dv;
  float* dqh;
  float* dks;
  float* dbs;
  int B, Hq, Hkv, D, S, W, topk;
  bool bf16;
  int64_t T;
  float scale;
  void* ws;
  size_t ws_bytes;
};
hipError_t launch_attend_backward(const BwdArgs& a, hipStream_t st);
// Workspace of the attention backward: `fixed` bytes (entry lists, row
// statistics, d s_hat) plus `per_group` bytes for each KV head whose dq parts are
// held at once (at least one).
void attend_backward_workspace(int B, int Hq, int Hkv, int64_t T, int S, int D, int topk, bool bf16,
                               size_t* fixed, size_t* per_group);

// Backward of the landmark summaries: dk (accumulated) and dq_land.
struct SumBwdArgs {
  const void* k;
  const void* ql;
  const float* dks;
  const float* dbs;
  float* dk;
  float* dql;
  int B, Hq, Hkv, D;
  bool bf16;
  int64_t kT, NCs;
  int64_t c0, n_chunks;
  float scale;
};
hipError_t launch_summarize_backward(const SumBwdArgs& a, hipStream_t st);

// Low-rank query calibration: q_hat = q + W_up (W_down h).
struct QcalArgs {
  const void* q;
  const void* h;    // [B, T, dm]
  const void* wd;   // [r, dm]
  const void* wu;   // [Hq, D, r]
  void* qh;
  int B, Hq, D, dm, r;
  bool bf16;
  int64_t T;
};
hipError_t launch_qcal(const QcalArgs& a, hipStream_t st);
// z = W_down h alone, fp32 [B, T, r], for the selection that fuses the rest.
hipError_t launch_zdown(const QcalArgs& a, float* z, hipStream_t st);

struct DecArgs {
  const int64_t* pos;  // host
  const void* q;
  const void* qh;
  const void* k_new;
  const void* v_new;
  const void* ql_new;
  void* kc;
  void* vc;
  void* ksum;
  float* bsum;
  void* out;
  float* lse;
  int32_t* idx;
  int B, Hq, Hkv, D, S, W, topk;
  bool bf16;
  int64_t Lcap;
  float scale;
  void* ws;
  size_t ws_bytes;
  int M = 1;           // queries per sequence (positions pos[b] .. pos[b] + M - 1)
};
hipError_t launch_decode(const DecArgs& a, hipStream_t st);
hipError_t launch_decode_multi(const DecArgs& a, hipStream_t st);

// Optional per-kernel timing (the C ABI's hils_timing_* calls): a KTimer around
// a launch records a HIP event pair on the launch stream when that kernel is
// selected, and does nothing otherwise.
enum KernelId {
  K_SUMMARIZE, K_SCORE_LSE, K_IDX_COUNT, K_IDX_SCAN_TILES, K_IDX_SCAN_BUCKETS,
  K_IDX_FILL, K_LSEL, K_WINDOW, K_CHUNK_ATTEND, K_DEC_SCORE, K_DEC_SELECT,
  K_DEC_ATTEND, K_DEC_FUSE, K_DEC_SUMMARIZE, K_VT, K_RANK_KEYS, K_TOPK_SCORES,
  K_BWD_ROWSTAT, K_BWD_KV, K_BWD_DQ, K_BWD_QHAT, K_SUM_BWD, K_BSA_KEYS, K_BSA_TOPK,
  K_QCAL, K_DEC_APPEND, K_DEC_GSEL, K_QCAL_ZDOWN, K_COUNT
};
class KTimer {
 public:
  KTimer(KernelId id, hipStream_t st);
  ~KTimer();
  KTimer(const KTimer&) = delete;
  KTimer& operator=(const KTimer&) = delete;

 private:
  KernelId id_;
  hipStream_t st_;
  hipEvent_t e0_;
};
size_t decode_workspace(int B, int Hq, int Hkv, int64_t Lcap, int S, int W, int D, int topk, int M = 1);
// Whether the decode selection can merge its per-span lists in one wave.
bool decode_supported(int64_t Lcap, int S, int W, int topk, int G);

}  // namespace hils
