// Static device scratch for the allocation-free decode entry point.
//
// kvevict_decode_step keeps the split decode's per-chunk partials and raw
// logits in the caller's workspace.  kvevict_decode_step_noalloc, for callers
// that cannot allocate device memory at all (code under graph capture, tight
// serving loops, harnesses that forbid it), keeps them in the array below
// instead: one copy per GPU, loaded with the library's code object and held
// until the process ends, shared by every call on that GPU.
//
// Host code never passes the array's name to a kernel or a copy: in host code
// it is a stand-in, not a device address.  Its device address is looked up
// once per device, with that device current, and kept in the table below.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "launch.hpp"

namespace {
constexpr size_t kStaticScratchBytes = size_t(32) << 20;   // 32 MiB per GPU
}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace kve {

size_t static_scratch_bytes() { return kStaticScratchBytes; }

hipError_t static_scratch_address(void** out) {
  static std::mutex mu;
  static std::vector<void*> addr;    // per device, filled on first use
  if (!out) return hipErrorInvalidValue;
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (addr.empty()) {
    int n = 0;
    e = hipGetDeviceCount(&n);
    if (e != hipSuccess) return e;
    addr.assign(n > 0 ? n : 0, nullptr);
  }
  if (dev < 0 || dev >= (int)addr.size()) return hipErrorInvalidDevice;
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace kve
