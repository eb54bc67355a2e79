// Host-only stand-ins for libmuir's kernel launchers, so that the C ABI layer (api.cpp) and
// the workspace sizes (sizes.cpp) can be built with the address and undefined-behaviour
// sanitizers by a plain host compiler and run without a GPU. Each launcher counts its calls
// and returns g_launch_status; nothing is launched and no pointer is dereferenced.
#include "kernels.hpp"

#include <stdint.h>

int g_launches = 0;
hipError_t g_launch_status = hipSuccess;
bool g_gates_in_kernel = false;

extern "C" const char *hipGetErrorString(hipError_t err) {
    return err == hipSuccess ? "no error" : "launch failed (host stub)";
}

namespace muir {
namespace {
hipError_t launched() {
    ++g_launches;
    return g_launch_status;
}
}  // namespace

hipError_t launch_decode_step(const void *, const void *, const void *, const float *,
                              const float *, const float *, const float *, const float *,
                              float *, void *, int, int, int, bool, hipStream_t) {
    return launched();
}
hipError_t launch_chunk_prepare(const void *, const void *, const float *, const float *,
                                const float *, int, int, int, int, int, bool, void *,
                                hipStream_t) {
    return launched();
}
hipError_t launch_chunk_prepare_lowrank(const void *, const void *, const void *, const void *,
                                        const void *, const float *, const float *,
                                        const float *, int, int, int, int, int, void *,
                                        hipStream_t) {
    return launched();
}
hipError_t launch_chunk_scan(const void *, const float *, const float *, const float *,
                             const float *, void *, float *, int, int, int, int, int, bool,
                             void *, hipStream_t, bool) {
    return launched();
}
hipError_t launch_chunk_scan_split(const void *, const float *, const float *, const float *,
                                   const float *, void *, float *, int, int, int, int, int,
                                   const void *, hipStream_t) {
    return launched();
}
hipError_t launch_chunk_scan_save(const void *, const float *, const float *, const float *,
                                  void *, float *, float *, float *, int, int, int, int, int,
                                  bool, const void *, hipStream_t) {
    return launched();
}
bool scan_gates_in_kernel(int, int, int, int) { return g_gates_in_kernel; }
hipError_t launch_chunk_scan_lowrank(const void *, const void *, const void *, const void *,
                                     const float *, const float *, const void *, const float *,
                                     const float *, void *, float *, int, int, int, int, int,
                                     const void *, hipStream_t) {
    return launched();
}
hipError_t launch_wy_solve(const void *, const float *, const float *, int, int, int, int, int,
                           void *, hipStream_t) {
    return launched();
}
hipError_t launch_wy_scan(const float *, void *, float *, int, int, int, int, int, void *,
                          hipStream_t) {
    return launched();
}
hipError_t launch_lowrank_gates(const void *, const void *, const void *, const void *,
                                const void *, const void *, const float *, const float *,
                                const float *, const float *, const float *, float *, float *,
                                float *, float *, float *, int, int, int, int, hipStream_t, bool) {
    return launched();
}
hipError_t launch_chunk_bwd(const ChunkBwdArgs &, int, int, int, int, bool, void *,
                            hipStream_t) {
    return launched();
}
// A stand-in address for the static scratch, far from the driver's stand-in buffers.
hipError_t noalloc_scratch(void **ptr) {
    *ptr = reinterpret_cast<void *>(uintptr_t(0x700000000000ull));
    return hipSuccess;
}
}  // namespace muir

// Accessors for the driver, which includes no HIP header.
extern "C" int stub_launches(void) { return g_launches; }
extern "C" void stub_fail_launches(int fail) {
    g_launch_status = fail ? hipErrorLaunchFailure : hipSuccess;
}
extern "C" void stub_gates_in_kernel(int on) { g_gates_in_kernel = on != 0; }
