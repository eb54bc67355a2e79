// Static device scratch for the chunk forward's entry point that allocates nothing.
//
// The chunk forward needs a workspace (its parallel phase's per-chunk Gram blocks and pivoted
// operands, read back by the scan). muir_chunk_fwd takes it from the caller;
// muir_chunk_fwd_noalloc takes it from the fixed array below instead, for callers that cannot
// allocate device memory. Each GPU the library runs on holds its own copy of the array, at its
// own address, from the library's load on that device until the process ends. In host code
// `scratch` names a host-side stand-in, not device memory: host code uses only the address
// that hipGetSymbolAddress returns for the current device, kept per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

static __device__ __align__(256) unsigned char scratch[muir::kNoAllocScratchBytes];

namespace muir {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void **ptr) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace muir
