// hils.cpp -- the C ABI of include/hils.h: validation, workspace sizing, dispatch.
//
// Every check happens here, on the host, before any work is enqueued; a nonzero
// status therefore means nothing was launched and nothing was written.
#include "hils.h"

#include <cmath>
#include <cstdint>

#include "hils_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

enum Mode { kSummarize, kPrefill, kDecode };

hils_status check_shape(const hils_shape* s, Mode mode) {
  if (!s) return HILS_E_NULL;
  if (s->io_dtype != HILS_F32 && s->io_dtype != HILS_BF16) return HILS_E_DTYPE;
  if (s->summary_dtype != HILS_F32 && s->summary_dtype != HILS_BF16) return HILS_E_DTYPE;
  if (s->batch < 1 || s->heads_q < 1 || s->heads_kv < 1 || s->head_dim < 1 || s->chunk < 1 ||
      s->window < 1 || s->top_k < 0 || s->seq_len < 1)
    return HILS_E_SHAPE;
  if (s->heads_q % s->heads_kv != 0) return HILS_E_SHAPE;
  if (!(s->scale >= 0.f) || std::isinf(s->scale)) return HILS_E_SHAPE;
  const int G = s->heads_q / s->heads_kv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return HILS_E_UNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return HILS_E_UNSUPPORTED;
  if (s->chunk != 64) return HILS_E_UNSUPPORTED;
  if (s->top_k > 64) return HILS_E_UNSUPPORTED;
  if (s->summary_dtype != s->io_dtype) return HILS_E_UNSUPPORTED;
  if (mode == kDecode) {
    if (s->batch > 64) return HILS_E_UNSUPPORTED;
    if (s->seq_len % s->chunk != 0) return HILS_E_SHAPE;
    if (!hils::decode_supported(s->seq_len, s->chunk, s->window, s->top_k, G)) return HILS_E_UNSUPPORTED;
    if (s->seq_len > (int64_t(1) << 31)) return HILS_E_UNSUPPORTED;
  } else if (mode == kPrefill) {
    if (s->seq_len / s->chunk > 8192) return HILS_E_UNSUPPORTED;  // <= 8192 chunks per sequence
  }
  return HILS_OK;
}

float eff_scale(const hils_shape* s) {
  return s->scale > 0.f ? s->scale : 1.0f / std::sqrt((float)s->head_dim);
}

hils_status from_hip(hipError_t e) { return e == hipSuccess ? HILS_OK : HILS_E_LAUNCH; }

size_t attend_min_ws(const hils_shape* s, size_t* full) {
  size_t fixed, per;
  hils::attend_workspace(s->batch, s->heads_q, s->heads_kv, s->seq_len, s->chunk, s->head_dim,
                         s->top_k, s->io_dtype == HILS_BF16, &fixed, &per);
  if (full) *full = fixed + per * (size_t)s->heads_kv;
  return fixed + per;
}

}  // namespace

extern "C" {

int hils_abi_version(void) { return HILS_ABI_VERSION; }

const char* hils_status_string(hils_status st) {
  switch (st) {
    case HILS_OK: return "ok";
    case HILS_E_NULL: return "a required pointer is NULL";
    case HILS_E_SHAPE: return "inconsistent or out-of-range sizes";
    case HILS_E_DTYPE: return "unknown dtype code";
    case HILS_E_ALIGN: return "tensor pointer not 16-byte aligned";
    case HILS_E_WORKSPACE: return "workspace missing or too small";
    case HILS_E_POS: return "decode position outside the cache";
    case HILS_E_NEED_QLAND: return "a chunk completes but no landmark query was given";
    case HILS_E_UNSUPPORTED: return "configuration not supported by this build";
    case HILS_E_LAUNCH: return "the HIP runtime refused a launch";
    case HILS_E_SCRATCH: return "the shape needs more than the built-in scratch of the allocation-free decode step";
  }
  return "unknown status";
}

size_t hils_workspace_bytes(const hils_shape* s, hils_op op) {
  const Mode m = op == HILS_OP_DECODE ? kDecode : op == HILS_OP_SUMMARIZE ? kSummarize : kPrefill;
  if (check_shape(s, m) != HILS_OK) return 0;
  switch (op) {
    case HILS_OP_SUMMARIZE: return 0;
    case HILS_OP_SELECT:
      return hils::select_workspace(s->batch, s->heads_q, s->heads_kv, s->seq_len, s->chunk,
                                    s->io_dtype == HILS_BF16, nullptr, nullptr);
    case HILS_OP_ATTEND_FUSE: {
      size_t full = 0;
      attend_min_ws(s, &full);
      return full;
    }
    case HILS_OP_DECODE:
      return hils::decode_workspace(s->batch, s->heads_q, s->heads_kv, s->seq_len, s->chunk,
                                    s->window, s->head_dim, s->top_k);
    case HILS_OP_ATTEND_BACKWARD: {
      size_t fixed, per;
      hils::attend_backward_workspace(s->batch, s->heads_q, s->heads_kv, s->seq_len, s->chunk,
                                      s->head_dim, s->top_k, s->io_dtype == HILS_BF16, &fixed, &per);
      return fixed + per * (size_t)s->heads_kv;
    }
  }
  return 0;
}

hils_status hils_summarize(const hils_shape* s, const void* k, const void* q_land,
                           int64_t chunk_begin, int64_t n_chunks, void* k_sum, float* b_sum,
                           hipStream_t stream) {
  const hils_status st = check_shape(s, kSummarize);
  if (st != HILS_OK) return st;
  if (!k || !q_land || !k_sum || !b_sum) return HILS_E_NULL;
  if (!aligned16(k) || !aligned16(q_land) || !aligned16(k_sum) || !aligned16(b_sum)) return HILS_E_ALIGN;
  const int64_t NC = s->seq_len / s->chunk;
  if (chunk_begin < 0 || n_chunks < 0 || chunk_begin + n_chunks > NC) return HILS_E_SHAPE;
  if (n_chunks > 0x7fffffff) return HILS_E_UNSUPPORTED;
  if (n_chunks == 0) return HILS_OK;
  hils::SumArgs a{};
  a.k = k; a.ql = q_land; a.ksum = k_sum; a.bsum = b_sum;
  a.B = s->batch; a.Hq = s->heads_q; a.Hkv = s->heads_kv; a.D = s->head_dim;
  a.bf16 = s->io_dtype == HILS_BF16;
  a.kT = s->seq_len; a.NCs = NC;
  a.ql_sb = (int64_t)s->heads_q * NC * s->head_dim;
  a.ql_sh = NC * s->head_dim;
  a.ql_sc = s->head_dim;
  a.c0 = chunk_begin; a.n_chunks = n_chunks;
  a.scale = eff_scale(s);
  a.list.n = 0;
  return from_hip(hils::launch_summarize(a, stream));
}

hils_status hils_summarize_shared(const hils_shape* s, const void* k, const void* q_shared,
                                  int64_t chunk_begin, int64_t n_chunks, void* k_sum, float* b_sum,
                                  hipStream_t stream) {
  const hils_status st = check_shape(s, kSummarize);
  if (st != HILS_OK) return st;
  if (!k || !q_shared || !k_sum || !b_sum) return HILS_E_NULL;
  if (!aligned16(k) || !aligned16(q_shared) || !aligned16(k_sum) || !aligned16(b_sum)) return HILS_E_ALIGN;
  const int64_t NC = s->seq_len / s->chunk;
  if (chunk_begin < 0 || n_chunks < 0 || chunk_begin + n_chunks > NC) return HILS_E_SHAPE;
  if (n_chunks > 0x7fffffff) return HILS_E_UNSUPPORTED;
  if (n_chunks == 0) return HILS_OK;
  hils::SumArgs a{};
  a.k = k; a.ql = q_shared; a.ksum = k_sum; a.bsum = b_sum;
  a.B = s->batch; a.Hq = s->heads_q; a.Hkv = s->heads_kv; a.D = s->head_dim;
  a.bf16 = s->io_dtype == HILS_BF16;
  a.kT = s->seq_len; a.NCs = NC;
  a.ql_sb = 0;                 // one query per head, for every sequence and chunk
  a.ql_sh = s->head_dim;
  a.ql_sc = 0;
  a.c0 = chunk_begin; a.n_chunks = n_chunks;
  a.scale = eff_scale(s);
  a.list.n = 0;
  return from_hip(hils::launch_summarize(a, stream));
}

static bool qcal_dims_ok(int32_t d_model, int32_t rank) {
  return d_model >= 32 && d_model % 32 == 0 && d_model <= 65536 &&
         (rank == 16 || rank == 32 || rank == 64 || rank == 128);
}

hils_status hils_qcal(const hils_shape* s, const void* q, const void* h, const void* w_down,
                      const void* w_up, int32_t d_model, int32_t rank, void* q_hat, hipStream_t stream) {
  const hils_status st = check_shape(s, kSummarize);
  if (st != HILS_OK) return st;
  if (!q || !h || !w_down || !w_up || !q_hat) return HILS_E_NULL;
  if (!aligned16(q) || !aligned16(h) || !aligned16(w_down) || !aligned16(w_up) || !aligned16(q_hat))
    return HILS_E_ALIGN;
  if (!qcal_dims_ok(d_model, rank)) return HILS_E_UNSUPPORTED;
  if (q == q_hat) return HILS_E_SHAPE;
  if (s->seq_len > 0x7fffffffLL * 64) return HILS_E_UNSUPPORTED;
  hils::QcalArgs a{};
  a.q = q; a.h = h; a.wd = w_down; a.wu = w_up; a.qh = q_hat;
  a.B = s->batch; a.Hq = s->heads_q; a.D = s->head_dim; a.dm = d_model; a.r = rank;
  a.bf16 = s->io_dtype == HILS_BF16; a.T = s->seq_len;
  return from_hip(hils::launch_qcal(a, stream));
}

// The selection's workspace carve-up and launch arguments (shape checked).
static hils_status select_setup(const hils_shape* s, void* ws, size_t ws_bytes, hils::SelArgs& a) {
  int n_slots = 0;
  int64_t stride = 0;
  size_t fixed = 0, per_group = 0;
  hils::select_workspace(s->batch, s->heads_q, s->heads_kv, s->seq_len, s->chunk,
                         s->io_dtype == HILS_BF16, &n_slots, &stride, &fixed, &per_group);
  if (!ws || ws_bytes < fixed + per_group) return HILS_E_WORKSPACE;
  char* w = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~(uintptr_t)255);
  a.L = reinterpret_cast<float*>(w);
  a.scratch = reinterpret_cast<float*>(w + (fixed - 256));
  const size_t groups = (ws_bytes - fixed) / per_group;
  const int nbg = s->batch * s->heads_kv;
  a.gpass = groups < (size_t)nbg ? (int)groups : nbg;
  a.group_words = (int64_t)(per_group / sizeof(uint32_t));
  a.B = s->batch; a.Hq = s->heads_q; a.Hkv = s->heads_kv; a.D = s->head_dim; a.S = s->chunk;
  a.W = s->window; a.topk = s->top_k; a.bf16 = s->io_dtype == HILS_BF16;
  a.T = s->seq_len; a.NCs = s->seq_len / s->chunk; a.scale = eff_scale(s);
  a.n_slots = n_slots; a.slot_stride = stride;
  return HILS_OK;
}

hils_status hils_select(const hils_shape* s, const void* q_hat, const void* k_sum,
                        const float* b_sum, int32_t* sel_idx, float* sel_score, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  const hils_status st = check_shape(s, kPrefill);
  if (st != HILS_OK) return st;
  const bool has_chunks = s->seq_len / s->chunk > 0;  // no complete chunk: no summaries to read
  if (!q_hat || (has_chunks && (!k_sum || !b_sum)) || (s->top_k > 0 && (!sel_idx || !sel_score)))
    return HILS_E_NULL;
  if (!aligned16(q_hat) || !aligned16(k_sum) || !aligned16(b_sum) || !aligned16(sel_idx) ||
      !aligned16(sel_score))
    return HILS_E_ALIGN;
  if (s->top_k == 0) return HILS_OK;  // nothing to select
  hils::SelArgs a{};
  const hils_status sw = select_setup(s, ws, ws_bytes, a);
  if (sw != HILS_OK) return sw;
  a.qh = q_hat; a.ksum = k_sum; a.bsum = b_sum; a.idx = sel_idx; a.ssel = sel_score;
  return from_hip(hils::launch_select(a, stream));
}

// z = W_down h (fp32 [B, T, rank]) at the workspace's first 256-byte boundary.
static size_t qcal_z_bytes(const hils_shape* s, int32_t rank) {
  return ((size_t)s->batch * (size_t)s->seq_len * (size_t)rank * sizeof(float) + 255) / 256 * 256 + 256;
}

size_t hils_select_qcal_workspace_bytes(const hils_shape* s, int32_t rank) {
  if (check_shape(s, kPrefill) != HILS_OK || !qcal_dims_ok(32, rank)) return 0;
  return qcal_z_bytes(s, rank) + hils_workspace_bytes(s, HILS_OP_SELECT);
}

hils_status hils_select_qcal(const hils_shape* s, const void* q, const void* h, const void* w_down,
                             const void* w_up, int32_t d_model, int32_t rank, const void* k_sum,
                             const float* b_sum, void* q_hat, int32_t* sel_idx, float* sel_score,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  const hils_status st = check_shape(s, kPrefill);
  if (st != HILS_OK) return st;
  const bool has_chunks = s->seq_len / s->chunk > 0;
  if (!q || !h || !w_down || !w_up || !q_hat || (has_chunks && (!k_sum || !b_sum)) ||
      (s->top_k > 0 && (!sel_idx || !sel_score)))
    return HILS_E_NULL;
  if (!aligned16(q) || !aligned16(h) || !aligned16(w_down) || !aligned16(w_up) || !aligned16(q_hat) ||
      !aligned16(k_sum) || !aligned16(b_sum) || !aligned16(sel_idx) || !aligned16(sel_score))
    return HILS_E_ALIGN;
  if (!qcal_dims_ok(d_model, rank)) return HILS_E_UNSUPPORTED;
  if (q == q_hat) return HILS_E_SHAPE;
  if (s->seq_len > 0x7fffffffLL * 64) return HILS_E_UNSUPPORTED;
  hils::QcalArgs qa{};
  qa.q = q; qa.h = h; qa.wd = w_down; qa.wu = w_up; qa.qh = q_hat;
  qa.B = s->batch; qa.Hq = s->heads_q; qa.D = s->head_dim; qa.dm = d_model; qa.r = rank;
  qa.bf16 = s->io_dtype == HILS_BF16; qa.T = s->seq_len;
  if (s->top_k == 0) return from_hip(hils::launch_qcal(qa, stream));   // nothing to select: q_hat alone
  const size_t zb = qcal_z_bytes(s, rank);
  if (!ws || ws_bytes < zb) return HILS_E_WORKSPACE;
  float* z = reinterpret_cast<float*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~(uintptr_t)255);
  hils::SelArgs a{};
  const hils_status sw = select_setup(s, static_cast<char*>(ws) + zb, ws_bytes - zb, a);
  if (sw != HILS_OK) return sw;
  a.qh = q_hat; a.ksum = k_sum; a.bsum = b_sum; a.idx = sel_idx; a.ssel = sel_score;
  a.qc = hils::QcFuse{q, z, w_up, q_hat};
  a.qc_r = rank;
  hipError_t e = hils::launch_zdown(qa, z, stream);
  if (e != hipSuccess) return from_hip(e);
  return from_hip(hils::launch_select(a, stream));
}

hils_status hils_attend_fuse(const hils_shape* s, const void* q, const void* k, const void* v,
                             const int32_t* sel_idx, const float* sel_score, void* out, float* lse,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  const hils_status st = check_shape(s, kPrefill);
  if (st != HILS_OK) return st;
  if (!q || !k || !v || !out || (s->top_k > 0 && (!sel_idx || !sel_score))) return HILS_E_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse) ||
      !aligned16(sel_idx) || !aligned16(sel_score))
    return HILS_E_ALIGN;
  if (s->seq_len > (int64_t(1) << 25)) return HILS_E_UNSUPPORTED;
  const size_t need = attend_min_ws(s, nullptr);
  if (!ws || ws_bytes < need) return HILS_E_WORKSPACE;
  hils::AttArgs a{};
  a.q = q; a.k = k; a.v = v; a.idx = sel_idx; a.ssel = sel_score; a.out = out; a.lse = lse;
  a.B = s->batch; a.Hq = s->heads_q; a.Hkv = s->heads_kv; a.D = s->head_dim; a.S = s->chunk;
  a.W = s->window; a.topk = s->top_k; a.bf16 = s->io_dtype == HILS_BF16;
  a.T = s->seq_len; a.scale = eff_scale(s); a.ws = ws; a.ws_bytes = ws_bytes;
  return from_hip(hils::launch_attend(a, stream));
}

hils_status hils_decode_step(const hils_shape* s, const int64_t* pos, const void* q,
                             const void* q_hat, const void* k_new, const void* v_new,
                             const void* q_land_new, void* k_cache, void* v_cache, void* k_sum,
                             float* b_sum, void* out, float* lse, int32_t* sel_idx, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  const hils_status st = check_shape(s, kDecode);
  if (st != HILS_OK) return st;
  if (!pos || !q || !q_hat || !k_new || !v_new || !k_cache || !v_cache || !k_sum || !b_sum || !out)
    return HILS_E_NULL;
  if (!aligned16(q) || !aligned16(q_hat) || !aligned16(k_new) || !aligned16(v_new) ||
      !aligned16(q_land_new) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_sum) ||
      !aligned16(b_sum) || !aligned16(out) || !aligned16(lse) || !aligned16(sel_idx))
    return HILS_E_ALIGN;
  bool completes = false;
  for (int b = 0; b < s->batch; ++b) {
    if (pos[b] < 0 || pos[b] >= s->seq_len) return HILS_E_POS;
    if ((pos[b] + 1) % s->chunk == 0) completes = true;
  }
  if (completes && !q_land_new) return HILS_E_NEED_QLAND;
  const size_t need = hils::decode_workspace(s->batch, s->heads_q, s->heads_kv, s->seq_len,
                                             s->chunk, s->window, s->head_dim, s->top_k);
  if (!ws || ws_bytes < need) return HILS_E_WORKSPACE;
  hils::DecArgs a{};
  a.pos = pos; a.q = q; a.qh = q_hat; a.k_new = k_new; a.v_new = v_new; a.ql_new = q_land_new;
  a.kc = k_cache; a.vc = v_cache; a.ksum = k_sum; a.bsum = b_sum; a.out = out; a.lse = lse;
  a.idx = sel_idx;
  a.B = s->batch; a.Hq = s->heads_q; a.Hkv = s->heads_kv; a.D = s->head_dim; a.S = s->chunk;
  a.W = s->window; a.topk = s->top_k; a.bf16 = s->io_dtype == HILS_BF16;
  a.Lcap = s->seq_len; a.scale = eff_scale(s); a.ws = ws; a.ws_bytes = ws_bytes;
  return from_hip(hils::launch_decode(a, stream));
}

hils_status hils_bsa_select(const hils_shape* s, const void* q, const void* k, int32_t* sel_idx, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  const hils_status st = check_shape(s, kPrefill);
  if (st != HILS_OK) return st;
  if (!q || !k || (s->top_k > 0 && !sel_idx)) return HILS_E_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(sel_idx)) return HILS_E_ALIGN;
  if (s->top_k == 0) return HILS_OK;
  int n_slots = 0;
  int64_t stride = 0;
  size_t fixed = 0, per_group = 0;
  hils::select_workspace(s->batch, s->heads_q, s->heads_kv, s->seq_len, s->chunk,
                         s->io_dtype == HILS_BF16, &n_slots, &stride, &fixed, &per_group);
  if (!ws || ws_bytes < fixed + per_group) return HILS_E_WORKSPACE;
  hils::SelArgs a{};
  a.qh = q; a.ksum = k; a.bsum = nullptr; a.idx = sel_idx; a.ssel = nullptr;
  char* w = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~(uintptr_t)255);
  a.L = nullptr;
  a.scratch = reinterpret_cast<float*>(w + (fixed - 256));
  const size_t groups = (ws_bytes - fixed) / per_group;
  const int nbg = s->batch * s->heads_kv;
  a.gpass = groups < (size_t)nbg ? (int)groups : nbg;
  a.group_words = (int64_t)(per_group / sizeof(uint32_t));
  a.B = s->batch; a.Hq = s->heads_q; a.Hkv = s->heads_kv; a.D = s->head_dim; a.S = s->chunk;
  a.W = s->window; a.topk = s->top_k; a.bf16 = s->io_dtype == HILS_BF16;
  a.T = s->seq_len; a.NCs = s->seq_len / s->chunk; a.scale = eff_scale(s);
  a.n_slots = n_slots; a.slot_stride = stride;
  return from_hip(hils::launch_bsa_select(a, stream));
}

hils_status hils_selection_overlap(const hils_shape* s, const int32_t* idx_a, const int32_t* idx_b,
                                   int32_t* count, hipStream_t stream) {
  const hils_status st = check_shape(s, kPrefill);
  if (st != HILS_OK) return st;
  if (!count || (s->top_k > 0 && (!idx_a || !idx_b))) return HILS_E_NULL;
  if (!aligned16(idx_a) || !aligned16(idx_b) || !aligned16(count)) return HILS_E_ALIGN;
  const int64_t nrows = (int64_t)s->batch * s->heads_kv * s->seq_len;
  if (s->top_k == 0) return from_hip(hipMemsetAsync(count, 0, (size_t)nrows * sizeof(int32_t), stream));
  return from_hip(hils::launch_overlap(idx_a, idx_b, count, nrows, s->top_k, stream));
}

hils_status hils_attend_fuse_backward(const hils_shape* s, const void* q, const void* k,
                                      const void* v, const void* q_hat, const void* k_sum,
                                      const int32_t* sel_idx, const float* sel_score,
                                      const void* out, const float* lse, const void* dout,
                                      const float* dlse, float* dq, float* dk, float* dv,
                                      float* dq_hat, float* dk_sum, float* db_sum, void* ws,
                                      size_t ws_bytes, hipStream_t stream) {
  const hils_status st = check_shape(s, kPrefill);
  if (st != HILS_OK) return st;
  const bool has_chunks = s->seq_len / s->chunk > 0;
  if (!q || !k || !v || !q_hat || !out || !lse || !dout || !dq || !dk || !dv || !dq_hat)
    return HILS_E_NULL;
  if (s->top_k > 0 && (!sel_idx || !sel_score)) return HILS_E_NULL;
  if (has_chunks && (!k_sum || !dk_sum || !db_sum)) return HILS_E_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_hat) || !aligned16(k_sum) ||
      !aligned16(sel_idx) || !aligned16(sel_score) || !aligned16(out) || !aligned16(lse) ||
      !aligned16(dout) || !aligned16(dlse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      !aligned16(dq_hat) || !aligned16(dk_sum) || !aligned16(db_sum))
    return HILS_E_ALIGN;
  if (s->seq_len > (int64_t(1) << 25)) return HILS_E_UNSUPPORTED;
  size_t fixed, per;
  hils::attend_backward_workspace(s->batch, s->heads_q, s->heads_kv, s->seq_len, s->chunk, s->head_dim,
                                  s->top_k, s->io_dtype == HILS_BF16, &fixed, &per);
  if (!ws || ws_bytes < fixed + per) return HILS_E_WORKSPACE;
  hils::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.qh = q_hat; a.ksum = k_sum; a.idx = sel_idx; a.ssel = sel_score;
  a.out = out; a.lse = lse; a.dout = dout; a.dlse = dlse;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dqh = dq_hat; a.dks = dk_sum; a.dbs = db_sum;
  a.B = s->batch; a.Hq = s->heads_q; a.Hkv = s->heads_kv; a.D = s->head_dim; a.S = s->chunk;
  a.W = s->window; a.topk = s->top_k; a.bf16 = s->io_dtype == HILS_BF16;
  a.T = s->seq_len; a.scale = eff_scale(s); a.ws = ws; a.ws_bytes = ws_bytes;
  return from_hip(hils::launch_attend_backward(a, stream));
}

hils_status hils_summarize_backward(const hils_shape* s, const void* k, const void* q_land,
                                    const float* dk_sum, const float* db_sum, int64_t chunk_begin,
                                    int64_t n_chunks, float* dk, float* dq_land, hipStream_t stream) {
  const hils_status st = check_shape(s, kSummarize);
  if (st != HILS_OK) return st;
  if (!k || !q_land || !dk_sum || !db_sum || !dk || !dq_land) return HILS_E_NULL;
  if (!aligned16(k) || !aligned16(q_land) || !aligned16(dk_sum) || !aligned16(db_sum) ||
      !aligned16(dk) || !aligned16(dq_land))
    return HILS_E_ALIGN;
  const int64_t NC = s->seq_len / s->chunk;
  if (chunk_begin < 0 || n_chunks < 0 || chunk_begin + n_chunks > NC) return HILS_E_SHAPE;
  if (n_chunks > 0x7fffffff) return HILS_E_UNSUPPORTED;
  if (n_chunks == 0) return HILS_OK;
  hils::SumBwdArgs a{};
  a.k = k; a.ql = q_land; a.dks = dk_sum; a.dbs = db_sum; a.dk = dk; a.dql = dq_land;
  a.B = s->batch; a.Hq = s->heads_q; a.Hkv = s->heads_kv; a.D = s->head_dim;
  a.bf16 = s->io_dtype == HILS_BF16;
  a.kT = s->seq_len; a.NCs = NC; a.c0 = chunk_begin; a.n_chunks = n_chunks;
  a.scale = eff_scale(s);
  return from_hip(hils::launch_summarize_backward(a, stream));
}

size_t hils_decode_multi_workspace_bytes(const hils_shape* s, int32_t n_queries) {
  if (check_shape(s, kDecode) != HILS_OK) return 0;
  const int G = s->heads_q / s->heads_kv;
  if (n_queries < 1 || n_queries > 16 || n_queries * G > 16 || n_queries > s->window ||
      s->batch * n_queries > 64 || (n_queries > 1 && s->top_k + s->window / s->chunk + 3 > 256))
    return 0;
  return hils::decode_workspace(s->batch, s->heads_q, s->heads_kv, s->seq_len, s->chunk, s->window,
                                s->head_dim, s->top_k, n_queries);
}

hils_status hils_decode_multi(const hils_shape* s, int32_t n_queries, const int64_t* pos, const void* q,
                              const void* q_hat, const void* k_new, const void* v_new,
                              const void* q_land_new, void* k_cache, void* v_cache, void* k_sum,
                              float* b_sum, void* out, float* lse, int32_t* sel_idx, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  const hils_status st = check_shape(s, kDecode);
  if (st != HILS_OK) return st;
  const int G = s->heads_q / s->heads_kv;
  const int M = n_queries;
  if (M < 1 || M > 16 || M > s->window) return HILS_E_SHAPE;
  // a row fuses its selection and the union of the M windows (one chunk more
  // than one window spans): at most 256 items
  if (M * G > 16 || s->batch * M > 64 || (M > 1 && s->top_k + s->window / s->chunk + 3 > 256))
    return HILS_E_UNSUPPORTED;
  if (!pos || !q || !q_hat || !k_new || !v_new || !k_cache || !v_cache || !k_sum || !b_sum || !out)
    return HILS_E_NULL;
  if (!aligned16(q) || !aligned16(q_hat) || !aligned16(k_new) || !aligned16(v_new) ||
      !aligned16(q_land_new) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_sum) ||
      !aligned16(b_sum) || !aligned16(out) || !aligned16(lse) || !aligned16(sel_idx))
    return HILS_E_ALIGN;
  bool completes = false;
  for (int b = 0; b < s->batch; ++b) {
    if (pos[b] < 0 || pos[b] + M > s->seq_len) return HILS_E_POS;
    for (int m = 0; m < M; ++m)
      if ((pos[b] + m + 1) % s->chunk == 0) completes = true;
  }
  if (completes && !q_land_new) return HILS_E_NEED_QLAND;
  const size_t need = hils::decode_workspace(s->batch, s->heads_q, s->heads_kv, s->seq_len, s->chunk,
                                             s->window, s->head_dim, s->top_k, M);
  if (!ws || ws_bytes < need) return HILS_E_WORKSPACE;
  hils::DecArgs a{};
  a.pos = pos; a.q = q; a.qh = q_hat; a.k_new = k_new; a.v_new = v_new; a.ql_new = q_land_new;
  a.kc = k_cache; a.vc = v_cache; a.ksum = k_sum; a.bsum = b_sum; a.out = out; a.lse = lse;
  a.idx = sel_idx;
  a.B = s->batch; a.Hq = s->heads_q; a.Hkv = s->heads_kv; a.D = s->head_dim; a.S = s->chunk;
  a.W = s->window; a.topk = s->top_k; a.bf16 = s->io_dtype == HILS_BF16;
  a.Lcap = s->seq_len; a.scale = eff_scale(s); a.ws = ws; a.ws_bytes = ws_bytes;
  a.M = M;
  return from_hip(M == 1 ? hils::launch_decode(a, stream) : hils::launch_decode_multi(a, stream));
}

}  // extern "C"
