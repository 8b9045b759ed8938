// gpt_fwd_loss_noalloc: gpt_fwd_loss with its workspace in a fixed device array of this library
// (for callers that cannot allocate device memory).
//
// The array below is the workspace of every such call on a device.  Its host-side name is only
// a stand-in for the symbol: host code never passes it to a kernel or a copy.  The device
// address of each GPU's copy is looked up once per device (hipGetSymbolAddress, with that
// device current) and kept here; that address is what the forward pass receives.  The forward
// pass clears what must start at zero (its device error flags) at the start of every call and
// writes every other workspace byte before reading it, so whatever a previous call left there
// does no harm.  Calls that overlap on one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gptfwd.h"

namespace {

__device__ __align__(256) unsigned char scratch[GPT_NOALLOC_MAX_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (looked up on first use), or NULL.
void* scratch_of(int dev) {
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" gpt_status gpt_fwd_loss_noalloc(const gpt_cfg* cfg, const gpt_weights* w,
                                           const int32_t* tokens, const int32_t* targets,
                                           float* loss, float* mean_loss, float* logits,
                                           void* stream) {
  // Size checks first, on the host only: a configuration that does not validate reports why,
  // one whose workspace exceeds the array is refused before any HIP call.
  const size_t need = gpt_workspace_bytes(cfg);
  if (need == 0) {
    const gpt_status st = gpt_validate(cfg);
    return st != GPT_OK ? st : GPT_E_INVALID_ARG;
  }
  if (need > (size_t)GPT_NOALLOC_MAX_BYTES) return GPT_E_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GPT_E_HIP;
  if (dev >= kMaxDevices) return GPT_E_UNSUPPORTED;
  void* ws = scratch_of(dev);
  if (!ws) return GPT_E_HIP;
  return gpt_fwd_loss(cfg, w, tokens, targets, loss, mean_loss, logits, ws,
                      (size_t)GPT_NOALLOC_MAX_BYTES, stream);
}
