// Device scratch memory of ep_execute_noalloc, the entry point for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  Its workspace -- the per-M-tile bias-gradient partials of the two-pass
// DRELU_BGRAD / DGELU_BGRAD reduction and the fp32 partial tiles of split-K -- lives in the
// file-scope array below instead of a plan-owned allocation.  Every GPU the library runs on
// holds its own copy for the life of the process; all calls on one GPU share it, so calls
// that overlap on one GPU race.  Nothing in it needs clearing between calls: every call
// writes each partial it later reads.
#include <hip/hip_runtime.h>

#include <mutex>

#include "static_scratch.hpp"

namespace ep {

static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch` per device, once looked up
}  // namespace

// Device address and size of the scratch array on device `dev`, which must be the calling
// thread's current device.  The address is looked up once per device with hipGetSymbolAddress
// (the array's name on the host is only a stand-in for the symbol, not a device address).
hipError_t static_scratch(int dev, void** ptr, size_t* bytes) {
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = kStaticScratchBytes;
  return hipSuccess;
}

}  // namespace ep
