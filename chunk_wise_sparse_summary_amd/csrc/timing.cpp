// timing.cpp -- optional per-kernel timing with HIP events on the launch stream.
//
// A KTimer placed around a kernel launch records an event before and after it
// when that kernel is selected by hils_timing_enable; hils_timing_get sums the
// recorded durations.  Events are pooled and reused across enables.
#include <cstring>
#include <string>
#include <vector>

#include "hils.h"
#include "hils_internal.h"

namespace hils {
namespace {

const char* const kNames[K_COUNT] = {
    "summarize", "score_lse", "idx_count", "idx_scan_tiles", "idx_scan_buckets",
    "idx_fill", "lsel", "window", "chunk_attend", "dec_score", "dec_select",
    "dec_attend", "dec_fuse", "dec_summarize", "v_transpose", "rank_keys", "topk_scores",
    "bwd_rowstat", "bwd_kv", "bwd_dq", "bwd_qhat", "summarize_bwd", "bsa_keys", "bsa_topk",
    "qcal", "dec_append", "dec_gsel", "qcal_zdown"};

struct Rec {
  int id;
  hipEvent_t e0, e1;
};

struct State {
  uint32_t mask = 0;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<Rec> recs;
};

State& state() {
  static State s;
  return s;
}

hipEvent_t take() {
  State& g = state();
  if (g.used == g.pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g.pool.push_back(e);
  }
  return g.pool[g.used++];
}

int find(const char* name, size_t len) {
  for (int i = 0; i < K_COUNT; ++i)
    if (std::strlen(kNames[i]) == len && std::strncmp(kNames[i], name, len) == 0) return i;
  return -1;
}

}  // namespace

KTimer::KTimer(KernelId id, hipStream_t st) : id_(id), st_(st), e0_(nullptr) {
  if (!((state().mask >> id) & 1u)) return;
  e0_ = take();
  if (e0_ && hipEventRecord(e0_, st) != hipSuccess) e0_ = nullptr;
}

KTimer::~KTimer() {
  if (!e0_) return;
  hipEvent_t e1 = take();
  if (!e1 || hipEventRecord(e1, st_) != hipSuccess) return;
  state().recs.push_back({(int)id_, e0_, e1});
}

}  // namespace hils

extern "C" hils_status hils_timing_enable(const char* kernels) {
  using namespace hils;
  State& g = state();
  for (const Rec& r : g.recs) hipEventSynchronize(r.e1);   // events are reused below
  g.recs.clear();
  g.used = 0;
  g.mask = 0;
  if (!kernels) return HILS_OK;
  uint32_t m = 0;
  if (std::strcmp(kernels, "*") == 0) {
    m = (1u << K_COUNT) - 1u;
  } else {
    const char* p = kernels;
    while (*p) {
      const char* e = std::strchr(p, ',');
      const size_t len = e ? (size_t)(e - p) : std::strlen(p);
      const int id = find(p, len);
      if (id < 0) return HILS_E_UNSUPPORTED;
      m |= 1u << id;
      p += len;
      if (*p == ',') ++p;
    }
  }
  while (g.pool.size() < 256) {   // most timed regions need no event creation
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) break;
    g.pool.push_back(e);
  }
  g.mask = m;
  return HILS_OK;
}

extern "C" hils_status hils_timing_get(const char* kernel, double* total_ms, int64_t* launches) {
  using namespace hils;
  if (!kernel || !total_ms || !launches) return HILS_E_NULL;
  const int id = find(kernel, std::strlen(kernel));
  if (id < 0) return HILS_E_UNSUPPORTED;
  double t = 0.0;
  int64_t n = 0;
  for (const Rec& r : state().recs) {
    if (r.id != id) continue;
    if (hipEventSynchronize(r.e1) != hipSuccess) return HILS_E_LAUNCH;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.e0, r.e1) != hipSuccess) return HILS_E_LAUNCH;
    t += ms;
    ++n;
  }
  *total_ms = t;
  *launches = n;
  return HILS_OK;
}
