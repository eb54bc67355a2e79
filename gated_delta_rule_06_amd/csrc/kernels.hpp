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

// Bytes of the chunk-forward workspace for these sizes (0 when they overflow): the slots the
// prepare writes and, where the split scan runs, its readout region after them.
size_t chunk_workspace_bytes(int B, int T, int H, int d, int chunk, bool bf16);
// Bytes of the slots alone (what a scan that reads nothing out needs).
size_t chunk_slots_bytes(int B, int T, int H, int d, int chunk, bool bf16);

// Phase P: decay products, pivoted operands and intra-chunk Gram blocks -> workspace.
hipError_t launch_chunk_prepare(const void *q, const void *k, const float *a, const float *g,
                                const float *r, int B, int T, int H, int d, int chunk, bool bf16,
                                void *workspace, hipStream_t stream);

// Phase P for a forward that keeps the state and does not read out (bf16 k): M, its fp32
// diagonal blocks, K*gamma, (K*beta')^T and the pair decays, without P and Qh*gamma (q and g are
// not needed; g may still be passed).
hipError_t launch_chunk_prepare_state(const void *k, const float *a, const float *g, const float *r,
                                      int B, int T, int H, int d, int chunk, void *workspace,
                                      hipStream_t stream);

// Phase P with the decay a and the query gate g formed in the kernel from the low-rank gate
// projection (z [B, T, 512], U_a [H, d, 64], U_g [H, d, 128] bf16; c_a, c_g [H, d] fp32),
// bf16 q and k only.
hipError_t launch_chunk_prepare_lowrank(const void *q, const void *k, const void *z,
                                        const void *Ua, const void *Ug, const float *ca,
                                        const float *cg, const float *r, int B, int T, int H,
                                        int d, int chunk, void *workspace, hipStream_t stream);

// Phase S: sequential chunk scan (solve, readout, state carry) from the workspace. A
// non-null og applies the output-gate epilogue o <- o * og. The slots are only read; where
// the split scan runs it writes the readout region after them.
hipError_t launch_chunk_scan(const void *v, const float *e, const float *w, const float *og,
                             const float *s0, void *o, float *s_out, int B, int T, int H, int d,
                             int chunk, bool bf16, void *workspace, hipStream_t stream,
                             bool packed_ew = false);

// Phase S for bf16 operands where split_scan_applies holds (at most one 8-column workgroup
// per compute unit): the sequential part split over four wavefronts per workgroup (chain,
// right-hand side, state carry, hand-over of S0 and U to the readout region), then the
// readout O = (Qh*gamma) S0 + P U (and the output gate) as a parallel kernel over chunks.
// Same results as the other scan, bit for bit.
// packed_ew: e and w come tile-packed, [B*H][d/8][T][8] fp32 (as launch_lowrank_gates writes them
// with packed_ew), which the split scan reads as whole cache lines; only where the split scan runs
// (elsewhere launch_chunk_scan returns hipErrorInvalidValue).
hipError_t launch_chunk_scan_split(const void *v, const float *e, const float *w, const float *og,
                                   const float *s0, void *o, float *s_out, int B, int T, int H,
                                   int d, int chunk, void *workspace, hipStream_t stream,
                                   bool packed_ew = false);

// The split scan's saving instance (bf16, where split_scan_applies holds): what
// launch_chunk_scan_save keeps, bit for bit, and no readout; reads only the workspace's slots.
hipError_t launch_chunk_scan_split_save(const void *v, const float *e, const float *w,
                                        const float *s0, float *s_out, float *u_out, float *states,
                                        int B, int T, int H, int d, int chunk, const void *workspace,
                                        hipStream_t stream);

// Phase S for the backward pass: keeps u_out [B, T, H, d] fp32 (u = w * v - e * p of every
// token) and states [B * H][ceil(T / 64) + 1][d][d] fp32 (the state at every 64-token block
// start, then the final state), and reads nothing out (o is not written and may be null).
// Chunks of 64, 128 or 256.
hipError_t launch_chunk_scan_save(const void *v, const float *e, const float *w, const float *s0,
                                  void *o, float *s_out, float *u_out, float *states, int B,
                                  int T, int H, int d, int chunk, bool bf16,
                                  const void *workspace, hipStream_t stream);

// Phase S with e and w formed inside the kernel from the low-rank gate projection (z,
// U_e, U_w, c_e, c_w as for launch_lowrank_gates; bf16 operands), bit-identical to
// launch_lowrank_gates followed by launch_chunk_scan; with a non-null U_o (and c_o) also the
// output gate and its epilogue. Only where scan_gates_in_kernel holds; elsewhere it returns
// hipErrorNotSupported and the caller makes the gates first.
bool scan_gates_in_kernel(int B, int H, int d, int chunk);
hipError_t launch_chunk_scan_lowrank(const void *v, const void *z, const void *Ue, const void *Uw,
                                     const float *ce, const float *cw, const void *Uo,
                                     const float *co, const float *s0, void *o, float *s_out, int B,
                                     int T, int H, int d, int chunk, const void *workspace,
                                     hipStream_t stream);

// Shared-erase variant (one erase strength per token, e [B, T, H]); bf16 operands only. Its
// workspace is the prepare kernel's slots followed by one region of per-chunk products per
// slot.
size_t wy_workspace_bytes(int B, int T, int H, int d, int chunk);
// Solve: chunk-parallel. Replaces M in a prepared workspace by T = (I + Diag(e) M)^-1, then
// forms each chunk's state operator, state increment, readout operator and readout offset.
hipError_t launch_wy_solve(const void *v, const float *e, const float *w, int B, int T, int H,
                           int d, int chunk, void *workspace, hipStream_t stream);
// Scan: the state recurrence over chunks (leaving each chunk's start state in the workspace),
// then the chunk-parallel readout.
hipError_t launch_wy_scan(const float *s0, void *o, float *s_out, int B, int T, int H, int d,
                          int chunk, void *workspace, hipStream_t stream);

// Gates a, e, w, g and the output gate og [B, T, H, d] fp32 from the fused low-rank gate
// projection: z [B, T, 512] bf16, up-projections U_n [H, d, r_n] bf16, offsets c_n [H, d]
// fp32. A null gate output is not computed.
hipError_t launch_lowrank_gates(const void *z, const void *Ua, const void *Ue, const void *Uw,
                                const void *Ug, const void *Uo, const float *ca, const float *ce,
                                const float *cw, const float *cg, const float *co, float *a,
                                float *e, float *w, float *g, float *og, int B, int T, int H, int d,
                                hipStream_t stream, bool packed_ew = false);

// Backward pass of the chunk forward (chunks of 64). Inputs as for the forward, plus dout
// (dtype of q) and dsT [B, H, d, d] fp32 (NULL: zero); outputs fp32, [B, T, H, d] except
// dr [H, d] and ds0 [B, H, d, d] (NULL: not written). dla is a * dL/da.
struct ChunkBwdArgs {
    const void *q, *k, *v;
    const float *a, *g, *e, *w, *r, *s0;
    const void *dout;
    const float *dsT;
    float *dq, *dk, *dv, *dla, *dg, *de, *dw, *dr, *ds0;
};
size_t chunk_bwd_workspace_bytes(int B, int T, int H, int d, bool bf16);
hipError_t launch_chunk_bwd(const ChunkBwdArgs &args, int B, int T, int H, int d, bool bf16,
                            void *workspace, hipStream_t stream);

// Size of the static device scratch that muir_chunk_fwd_noalloc uses as its workspace, and
// its address on the current device (looked up once per device with hipGetSymbolAddress).
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
hipError_t noalloc_scratch(void **ptr);

}  // namespace muir
