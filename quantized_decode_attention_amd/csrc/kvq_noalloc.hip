// kvq_noalloc.hip — the partials buffer of kvq_decode_attn_noalloc: one
// file-scope device array that every GPU the library runs on holds until the
// process ends.  Host code never uses the array's name as an address (on the
// host it names a stand-in, not device memory): it asks each device once for
// that device's copy through hipGetSymbolAddress and keeps the answer.
#include <mutex>

#include "kvq_internal.h"

namespace kvq {

static __device__ __align__(256) float scratch[KVQ_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // this device's copy
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *ptr = g_scratch_addr[dev];
  *bytes = KVQ_NOALLOC_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace kvq
