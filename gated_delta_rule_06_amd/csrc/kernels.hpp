// Internal launchers of libmuir's kernels. Arguments are validated by the C ABI layer
// (api.cpp) before any of these is called; each returns the launch's hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace muir {

hipError_t launch_decode_step(const void *q, const void *k, const void *v, const float *a,
                              const float *g, const float *e, const float *w, const float *r,
                              float *state, void *o, int B, int H, int d, bool bf16,
                              hipStream_t stream);

// Bytes of the chunk-forward workspace for these sizes (0 when they overflow).
size_t chunk_workspace_bytes(int B, int T, int H, int d, int chunk, bool bf16);

hipError_t launch_chunk_fwd(const void *q, const void *k, const void *v, const float *a,
                            const float *g, const float *e, const float *w, const float *r,
                            const float *s0, void *o, float *s_out, int B, int T, int H,
                            int d, int chunk, bool bf16, void *workspace,
                            hipStream_t stream);

}  // namespace muir
