// noalloc.hip -- hils_decode_step_noalloc: the decode step with the library's own
// scratch memory, for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The scratch is a file-scope __device__ array; every GPU the library runs on
// holds its own copy until the process ends.  In host code the array's name is
// only a host-side stand-in, so its device address is looked up once per device
// with hipGetSymbolAddress (with that device current) and that address is what
// the kernels get.  The decode step writes every scratch element it later reads
// within the same call, so nothing has to be cleared between calls.
#include <mutex>

#include "hils.h"
#include "hils_internal.h"

namespace {

constexpr size_t kScratchBytes = HILS_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];

// Device address of this device's scratch array (nullptr on failure).
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" hils_status hils_decode_step_noalloc(const hils_shape* s, const int64_t* pos,
                                                const void* q, const void* q_hat,
                                                const void* k_new, const void* v_new,
                                                const void* q_land_new, void* k_cache,
                                                void* v_cache, void* k_sum, float* b_sum,
                                                void* out, float* lse, int32_t* sel_idx,
                                                hipStream_t stream) {
  const size_t need = hils_workspace_bytes(s, HILS_OP_DECODE);
  if (need == 0)   // invalid shape: let the full validation name the reason
    return hils_decode_step(s, pos, q, q_hat, k_new, v_new, q_land_new, k_cache, v_cache, k_sum,
                            b_sum, out, lse, sel_idx, nullptr, 0, stream);
  if (need > kScratchBytes) return HILS_E_SCRATCH;
  void* ws = device_scratch();
  if (!ws) return HILS_E_LAUNCH;
  return hils_decode_step(s, pos, q, q_hat, k_new, v_new, q_land_new, k_cache, v_cache, k_sum,
                          b_sum, out, lse, sel_idx, ws, kScratchBytes, stream);
}
