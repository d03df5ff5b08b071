// The library's one static device buffer: the split partials of
// paged_varlen_attention_noalloc, for callers that cannot allocate device
// memory (code under graph capture, tight serving loops, harnesses that
// forbid hipMalloc). Each device the library runs on holds its own copy
// until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address on the current device comes from hipGetSymbolAddress,
// looked up once per device and kept, and only that address is handed to
// kernels.
#include <atomic>

#include "launch.h"

namespace pkv {
namespace {

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch[kMaxScratchDevices];

}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool keep = dev >= 0 && dev < kMaxScratchDevices;
  if (keep) {
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p != nullptr) {
      *out = p;
      return hipSuccess;
    }
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (p == nullptr) return hipErrorInvalidSymbol;
  if (keep) g_scratch[dev].store(p, std::memory_order_release);
  *out = p;
  return hipSuccess;
}

}  // namespace pkv
