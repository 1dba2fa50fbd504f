// Static device scratch of kv_decode_attn_noalloc: the split-K partial results of
// a decode live in one file-scope device array per GPU instead of a caller
// workspace, for callers that cannot allocate device memory.
//
// In host code `scratch` names a host-side stand-in, not device memory: the host
// looks up the array's device address once per device (with that device current)
// and passes that address to the kernels, like any workspace.  The array keeps the
// last call's contents; the decode writes every partial row it reads, so nothing
// needs clearing between calls.
#include <atomic>

#include <hip/hip_runtime.h>

#include "kvq_internal.hpp"

namespace kvq {
namespace {

static __device__ __align__(256) float scratch[KVQ_STATIC_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;

}  // namespace

hipError_t static_scratch(void** ptr) {
  static std::atomic<void*> addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached) {
    void* p = addr[dev].load(std::memory_order_acquire);
    if (p) {
      *ptr = p;
      return hipSuccess;
    }
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!p) return hipErrorInvalidSymbol;
  if (cached) addr[dev].store(p, std::memory_order_release);
  *ptr = p;
  return hipSuccess;
}

}  // namespace kvq
