// noalloc.hip — the fixed scratch array of ssm_scan_fwd_noalloc, for callers that cannot allocate.
//
// The time-split prefill needs scratch for its segment aggregates (and, past 16 segments, the carries).
// ssm_scan_fwd takes it from a stream-ordered pool; ssm_scan_fwd_noalloc uses this file-scope device
// array instead. Every GPU that loads the library holds its own copy until the process ends, at its own
// address, which hipGetSymbolAddress returns once per device (with that device current). In host code the
// array's name is only a stand-in for the symbol: kernels receive the address looked up here, never the
// name itself.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace ssm {
namespace {

static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;

}  // namespace

hipError_t noalloc_scratch(float **out) {
    static std::mutex mu;
    static float *addr[kMaxDevices] = {nullptr};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = static_cast<float *>(p);
    }
    *out = addr[dev];
    return hipSuccess;
}

}  // namespace ssm
