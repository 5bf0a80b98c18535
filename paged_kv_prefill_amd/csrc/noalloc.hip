// Fixed device scratch for the entry point that allocates nothing
// (paged_prefill_attention_pieces_noalloc): the split workspace of its calls
// lives in this file-scope device array instead of a hipMalloc'd buffer.
//
// In host code `scratch` names a host-side stand-in, not device memory; its
// device address comes from hipGetSymbolAddress, taken once per device (with
// that device current) on the first call there and kept.  Every call on a
// device shares that device's array: calls that overlap on one device (two
// streams, or two threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "paged_prefill.h"

namespace ppa {
namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

int static_scratch(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PPA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PPA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return PPA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PPA_OK;
}

}  // namespace ppa
