// etg_logits_topk_noalloc: the top-k call for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Its workspace is a file-scope device array, one copy per
// GPU, that lives until the process ends; nothing is allocated per call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/etg.h"
#include "etg_internal.hpp"

namespace {

// The workspace of every etg_logits_topk_noalloc call on a device.  Host code
// never passes this name to a kernel or a copy (on the host it is only a
// stand-in for the symbol): it uses the device address looked up below.
__device__ __align__(256) unsigned char scratch[ETG_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int32_t etg_logits_topk_noalloc(const etg_table* lm_head, const float* d_residual, int64_t batch,
                                           int32_t k, int32_t* d_topk_ids, float* d_topk_scores, void* stream) {
  // host-only checks first: the table, batch and k, then the scratch limit
  const int64_t need = etg_logits_topk_workspace(lm_head, batch, k);
  if (need < 0) return (int32_t)need;  // the message is set
  if (need > (int64_t)ETG_NOALLOC_SCRATCH_BYTES)
    return etg::set_error(ETG_EWORKSPACE,
                          "batch %lld, k %d needs %lld bytes of workspace, beyond the %lld-byte scratch of "
                          "etg_logits_topk_noalloc (use etg_logits_topk with a workspace)",
                          (long long)batch, k, (long long)need, (long long)ETG_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return etg::set_error(ETG_EHIP, "scratch lookup failed: %s", hipGetErrorString(e));
  return etg_logits_topk(lm_head, d_residual, batch, k, d_topk_ids, d_topk_scores, ws,
                         (size_t)ETG_NOALLOC_SCRATCH_BYTES, stream);
}
