// Scratch memory of the allocation-free entry point (dspark_markov_draft_noalloc):
// one static device array per GPU, used in place of a caller workspace by
// callers that cannot allocate.  Every call on a GPU shares that GPU's array;
// calls that overlap on one GPU race on it.
#include <mutex>

#include "launch.hpp"

namespace dspark {

// 32 MiB.  The draft needs draft_workspace(B, gamma, V, r) bytes of it, the
// larger of its two schedules: 14.1 MiB at B = 256, V = 151936, r = 256 and
// 28.3 MiB at B = 512 (the device-resident loop's summaries).
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

size_t static_scratch_bytes() { return kStaticScratchBytes; }

// The array's device address on the current device.  In host code `scratch`
// names a host-side stand-in, so the address is taken with
// hipGetSymbolAddress, once per device with that device current, and kept.
hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace dspark
