/*
 * muir.h -- C ABI of libmuir: channel-wise gated delta-rule linear attention with
 * matched-filter readout (Muir), hand-written HIP kernels for AMD CDNA4 (gfx950).
 *
 * The method (sources are the pages on "Muir: Linear Attention with Sensitivity-
 * Allocated Gating and Matched-Filter Readout", arXiv 2611.08376):
 *   per head, a dk x dv fp32 state S (rows = key channels). For each token t:
 *     S <- Diag(a_t) S                  channel-wise (per-row) decay, a_t in [0, 1]
 *     p <- S^T k_t                      prediction of the decayed state for k_t
 *     S <- S + k_t (w_t * v_t - e_t * p)^T   erase under the value-channel erase
 *                                       gate e_t, then write under the write gate w_t
 *     o_t <- S^T (r * g_t * q_t)        matched-filter readout: static row scale r
 *                                       times the dynamic query gate g_t
 *   Update order (Muir abstract, "Full text" on the Astral Feed page): each token
 *   first scales the state down by its per-row decay, then removes what the decayed
 *   state predicts for the new key (per value channel, under the erase gate), then adds
 *   the new key's gated value (the write gate is separate from the erase gate), and the
 *   read comes last. Readout: openai-hub news page, section on matched-filter readout (a static
 *   per-row scale from each row's expected energy plus per-token query modulation),
 *   and the liuch.name summary, first bullet (inverse fractional power law plus
 *   per-token query modulation).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a caller-owned DEVICE buffer, contiguous, row-major,
 *     16-byte aligned. The library never allocates or frees device memory.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 *     Buffers must stay live until the stream reaches the call.
 *   - Argument errors are detected on the host, before any launch, and return a
 *     status; nothing is launched then. A failed launch returns MUIR_ERR_HIP.
 *     muir_last_error() gives a human-readable detail for the calling thread.
 *   - No exceptions cross the ABI. Values are not checked for NaN/Inf; non-finite
 *     inputs propagate. Gates are expected in [0, 1] (a), (0, 1) (e, w, g).
 *   - Results are deterministic: reductions use no atomics.
 *   - The library keeps no state across calls and is safe to call from several
 *     threads (the error detail is thread-local).
 */
#ifndef MUIR_H
#define MUIR_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP stream type itself (hipStream_t is this same pointer type), declared here so that
 * C callers need no HIP header; NULL is the default stream. */
typedef struct ihipStream_t *muir_stream_t;

typedef enum {
    MUIR_OK = 0,
    MUIR_ERR_NULL = 1,        /* a required pointer is NULL                      */
    MUIR_ERR_SHAPE = 2,       /* a size is out of range or inconsistent          */
    MUIR_ERR_UNSUPPORTED = 3, /* a valid but unimplemented combination           */
    MUIR_ERR_WORKSPACE = 4,   /* workspace missing, too small or misaligned      */
    MUIR_ERR_ALIAS = 5,       /* an output overlaps an input it must not alias   */
    MUIR_ERR_HIP = 6          /* the HIP runtime reported an error at launch     */
} muir_status_t;

typedef enum {
    MUIR_F32 = 0,             /* q, k, v and o are float32                       */
    MUIR_BF16 = 1             /* q, k, v and o are bfloat16                      */
} muir_dtype_t;

/*
 * Workspace bytes needed by muir_chunk_fwd for these sizes (0 for invalid sizes).
 * The workspace holds, per (batch, head, chunk), what the parallel phase hands to the
 * sequential one: the lower-triangular intra-chunk Gram matrices M and P in 16x16
 * blocks, the decay-scaled operands K*gamma, (r*g*q)*gamma and (K*beta')^T, in the
 * operand precision (bf16 for bf16 q/k/v, fp32 otherwise), and the decay of every
 * 32-token leaf pair in fp32.
 * It must be 256-byte aligned. Its contents are scratch: nothing is expected in it
 * on entry to muir_chunk_fwd or kept from it on return.
 */
size_t muir_chunk_fwd_workspace_size(int B, int T, int H, int dk, int dv, int chunk,
                                     muir_dtype_t qkv);

/*
 * Chunkwise-parallel forward over a whole sequence (training / prefill).
 *
 * The pages' stable large-chunk scheme (liuch.name summary, third bullet; openai-hub
 * page, section on rewriting the long-sequence parallel algorithm for TPU): decays
 * that cross a block boundary are split into two running products pivoted at that
 * boundary, both in (0, 1], so nothing is divided by a cumulative decay; the
 * intra-chunk unit lower-triangular system is solved by recursive block-Neumann
 * halving whose off-diagonal products run on the matrix cores; chunks are chained by
 * carrying the state. With a value-channel erase gate every value column has its own
 * triangular system, so the recursion is applied to each right-hand side.
 *
 *   q, k    [B, T, H, dk]  dtype `qkv`      keys should be L2-normalised by the caller
 *   v       [B, T, H, dv]  dtype `qkv`
 *   a, g    [B, T, H, dk]  float32          per-row decay in [0, 1], query gate
 *   e, w    [B, T, H, dv]  float32          erase and write gates (value channels)
 *   r       [H, dk]        float32          static readout row scale
 *   s0      [B, H, dk, dv] float32 or NULL  initial state (NULL = zeros)
 *   o       [B, T, H, dv]  dtype `qkv`      output, o_t read after token t's update
 *   s_out   [B, H, dk, dv] float32 or NULL  final state; may equal s0 (in place)
 *   chunk   64, 128 or 256; T need not be a multiple (the last chunk is partial)
 *   dk, dv  dk == dv, 64 or 128
 *   T       >= 0 (T == 0 copies s0, or zeros, into s_out and writes no o)
 *   workspace / workspace_bytes: at least muir_chunk_fwd_workspace_size(...) bytes
 *
 * Errors: MUIR_ERR_NULL for a missing q/k/v/a/g/e/w/r/o (when T > 0) or workspace;
 * MUIR_ERR_SHAPE for B < 1, T < 0, H < 1 or size overflow; MUIR_ERR_UNSUPPORTED for
 * dk != dv, d not in {64, 128} or chunk not in {64, 128, 256}, and when one head's
 * tokens (T*H*dv*4 bytes) or one head's workspace exceed 4 GiB (a longer sequence is
 * processed in several calls, the state carried through s0 / s_out); MUIR_ERR_WORKSPACE
 * for a short or misaligned workspace; MUIR_ERR_ALIAS when o overlaps an input or s_out
 * overlaps an input other than s0 (or s0 partially).
 */
muir_status_t muir_chunk_fwd(
    const void *q, const void *k, const void *v,
    const float *a, const float *g, const float *e, const float *w, const float *r,
    const float *s0, void *o, float *s_out,
    int B, int T, int H, int dk, int dv, int chunk, muir_dtype_t qkv,
    void *workspace, size_t workspace_bytes, muir_stream_t stream);

/*
 * muir_chunk_fwd without the workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. The workspace is a static device array inside the library instead, one per
 * GPU (held from the library's first use on that GPU until the process ends), of
 * muir_chunk_fwd_noalloc_max_workspace() bytes (128 MiB). The call allocates and frees
 * nothing; its address on the current device is looked up once per device.
 *
 * Arguments, results and errors are those of muir_chunk_fwd (same kernels, same bits),
 * plus MUIR_ERR_WORKSPACE when muir_chunk_fwd_workspace_size(...) of these sizes exceeds the
 * static scratch (for example 348 KiB per (batch, head, 256-token chunk) at d = 128 in bf16:
 * 16 heads x 16 chunks of 256 tokens fit, the long-context shape's 16 x 128 chunks do not).
 * Every call on one GPU uses the same scratch and leaves its contents there; nothing in it
 * needs clearing (each call's parallel phase writes every byte its scan reads). Calls that
 * overlap on one GPU (on different streams, or from several threads) race on the scratch:
 * order them on one stream or serialise them.
 */
muir_status_t muir_chunk_fwd_noalloc(
    const void *q, const void *k, const void *v,
    const float *a, const float *g, const float *e, const float *w, const float *r,
    const float *s0, void *o, float *s_out,
    int B, int T, int H, int dk, int dv, int chunk, muir_dtype_t qkv, muir_stream_t stream);

size_t muir_chunk_fwd_noalloc_max_workspace(void);

/*
 * The two phases of muir_chunk_fwd as separate calls, for callers that schedule or
 * time them on their own. muir_chunk_fwd(...) is exactly muir_chunk_fwd_prepare(...)
 * followed by muir_chunk_fwd_scan(...) on the same stream with the same workspace.
 *
 * muir_chunk_fwd_prepare: the parallel phase, one work item per (batch, head, chunk):
 *   the decay running products pivoted at 16-token block boundaries (every factor in
 *   [0, 1], no division), the decay-scaled operands K*gamma, (r*g*q)*gamma and
 *   (K*beta')^T (beta' runs to the end of the token's 32-token leaf pair), the decay of
 *   every leaf pair, and the lower-triangular intra-chunk
 *   Gram matrices M (decayed key-key, strictly lower) and P (decayed query-key,
 *   inclusive) in 16x16 blocks on the matrix cores. Writes them into `workspace`.
 *   Arguments as for muir_chunk_fwd (dv is taken equal to dk). T == 0 launches nothing.
 *
 * muir_chunk_fwd_scan: the sequential phase, one work item per (batch, head, 16 value
 *   columns), chunk after chunk: the prediction of the carried state, the recursive
 *   block-Neumann solve of every value column's triangular system, the readout
 *   o = (r*g*q*gamma) S0 + P U and the state carry S = Diag(gamma_C) S0 + (K*beta)^T U,
 *   evaluated pair by pair as S <- Diag(pair decay) S + (K*beta')^T U.
 *   Reads the slots of `workspace` as left by muir_chunk_fwd_prepare for the same sizes
 *   and inputs; they must not be modified between the two calls. With bf16 q, k, v and
 *   B*H*dk/8 <= 256 (at most one 8-column scan work item per compute unit) the scan hands
 *   S0 and U of every chunk to a parallel readout kernel through a region of `workspace`
 *   after the slots, which it writes (muir_chunk_fwd_workspace_size counts it). T == 0
 *   copies s0 (or zeros) into s_out.
 *
 * Errors as for muir_chunk_fwd, restricted to the arguments each phase takes.
 */
muir_status_t muir_chunk_fwd_prepare(
    const void *q, const void *k, const float *a, const float *g, const float *r,
    int B, int T, int H, int dk, int chunk, muir_dtype_t qkv,
    void *workspace, size_t workspace_bytes, muir_stream_t stream);

muir_status_t muir_chunk_fwd_scan(
    const void *v, const float *e, const float *w, const float *s0, void *o, float *s_out,
    int B, int T, int H, int dk, int dv, int chunk, muir_dtype_t qkv,
    void *workspace, size_t workspace_bytes, muir_stream_t stream);

/*
 * The chunk forward with the output-gate epilogue fused into the readout: the stored
 * output is o_t * og_t elementwise, og_t being the output gate that sets how much of
 * the state's readout reaches the network (openai-hub page, section on
 * sensitivity-allocated gating, gate table: the output gate, rank 128).
 *
 *   og: [B, T, H, dv] fp32, the gate values themselves (already through their
 *       activation, like e, w and g), caller-owned device buffer, 16-byte aligned,
 *       required when T > 0, must not overlap o, s_out or the workspace.
 * Everything else is exactly as for muir_chunk_fwd / muir_chunk_fwd_scan; the state and
 * s_out are unaffected by og. Errors as for those calls, plus MUIR_ERR_NULL for a
 * missing og.
 */
muir_status_t muir_chunk_fwd_gated(
    const void *q, const void *k, const void *v,
    const float *a, const float *g, const float *e, const float *w, const float *og,
    const float *r, const float *s0, void *o, float *s_out,
    int B, int T, int H, int dk, int dv, int chunk, muir_dtype_t qkv,
    void *workspace, size_t workspace_bytes, muir_stream_t stream);

muir_status_t muir_chunk_fwd_scan_gated(
    const void *v, const float *e, const float *w, const float *og, const float *s0,
    void *o, float *s_out, int B, int T, int H, int dk, int dv, int chunk, muir_dtype_t qkv,
    void *workspace, size_t workspace_bytes, muir_stream_t stream);

/*
 * The chunk forward with ONE erase strength per token, shared by every value channel:
 * the plain gated delta rule's erase, which GDN-2 and Muir generalise into decoupled
 * per-channel erase gates (Muir abstract, "Full text" on the Astral Feed page). The
 * result is muir_chunk_fwd's with e[b, t, h, j] = e[b, t, h] for every j.
 *
 * With a shared erase the intra-chunk unit lower-triangular system I + Diag(e) M is the
 * same for every value column, so its inverse T is formed once per chunk, in parallel
 * over chunks, by the block recursion of the stable scheme (liuch.name summary, third
 * bullet): 16x16 diagonal inverses by forward substitution, off-diagonal blocks on the
 * matrix cores. Everything that does not depend on the carried state is then formed in
 * parallel over chunks too (the WY form): with W = T Diag(e) (K*gamma), U~ = T (w*v),
 *   A = (K*beta)^T W,  Bc = (K*beta)^T U~,  Q~ = (r*g*q*gamma) - P W,  O~ = P U~,
 * so the sequential part is two d x d products per chunk,
 *   S_next = Diag(gamma_C) S - A S + Bc,
 * and the readout o = Q~ S + O~ runs in parallel over chunks afterwards.
 *
 *   e       [B, T, H]      float32          erase strength per token and head, in (0, 1)
 *   qkv     MUIR_BF16 only (MUIR_ERR_UNSUPPORTED otherwise)
 *   workspace / workspace_bytes: at least
 *           muir_chunk_fwd_scalar_erase_workspace_size(B, T, H, dk, dv, chunk) bytes,
 *           256-byte aligned: the prepare's workspace followed by the per-chunk products
 * Every other argument as for muir_chunk_fwd.
 *
 * The three phases are also separate calls; muir_chunk_fwd_scalar_erase(...) is exactly
 * muir_chunk_fwd_prepare(...) (into the same workspace), muir_chunk_fwd_scalar_erase_solve(...)
 * and muir_chunk_fwd_scalar_erase_scan(...) on one stream:
 *   - solve: chunk-parallel. It overwrites M in the prepared workspace with T, then writes
 *     the per-chunk products; it must run exactly once after each prepare (a second run
 *     would invert T).
 *   - scan: the state recurrence (leaving each chunk's start state in the workspace), then
 *     the readout. It writes only those start states, the same ones on every run, so it
 *     may be repeated.
 *
 * Errors as for muir_chunk_fwd, plus MUIR_ERR_UNSUPPORTED for f32 q/k/v.
 */
size_t muir_chunk_fwd_scalar_erase_workspace_size(int B, int T, int H, int dk, int dv, int chunk);

muir_status_t muir_chunk_fwd_scalar_erase(
    const void *q, const void *k, const void *v,
    const float *a, const float *g, const float *e, const float *w, const float *r,
    const float *s0, void *o, float *s_out,
    int B, int T, int H, int dk, int dv, int chunk, muir_dtype_t qkv,
    void *workspace, size_t workspace_bytes, muir_stream_t stream);

muir_status_t muir_chunk_fwd_scalar_erase_solve(
    const void *v, const float *e, const float *w, int B, int T, int H, int dk, int chunk,
    muir_dtype_t qkv, void *workspace, size_t workspace_bytes, muir_stream_t stream);

muir_status_t muir_chunk_fwd_scalar_erase_scan(
    const float *s0, void *o, float *s_out, int B, int T, int H, int dk, int dv, int chunk,
    muir_dtype_t qkv, void *workspace, size_t workspace_bytes, muir_stream_t stream);

/*
 * The recurrence's gates from the fused low-rank gate projection. The pages fuse all five
 * gates into one projection of total rank 512: one shared down-projection, then one
 * up-projection per gate with its own rank, decay 64, erase 64, output 128, write 128 and
 * dynamic read 128 (openai-hub page, section on sensitivity-allocated gating, gate table;
 * liuch.name summary, second bullet). Per gate n:
 *   y_n = z[b, t, slice_n] . U_n[h, i, :] + c_n[h, i]
 *   a = exp(-exp(y_decay)) (y is the log decay rate),  e, w, g = sigmoid(y)
 *
 *   z        [B, T, 512] bf16: the down-projection's output, rank slices in the table's
 *            order: decay 0..63, erase 64..127, output 128..255, write 256..383,
 *            read 384..511 (the output gate's slice is read by muir_lowrank_output_gate)
 *   Ua, Ue   [H, d, 64]  bf16;  Uw, Ug [H, d, 128] bf16  (rank contiguous per channel)
 *   ca .. cg [H, d] fp32 offsets
 *   a, e, w, g  [B, T, H, d] fp32 outputs; a NULL output is not computed (and its U and c
 *            may be NULL)
 *   d        64 or 128
 *
 * Errors: MUIR_ERR_NULL for a missing z (T > 0) or a requested gate's U or c;
 * MUIR_ERR_SHAPE for B < 1, T < 0, H < 1, size overflow or a misaligned buffer;
 * MUIR_ERR_UNSUPPORTED for other d or a batch row over 4 GiB; MUIR_ERR_ALIAS when an output
 * overlaps an input or another output.
 */
muir_status_t muir_lowrank_gates(
    const void *z, const void *Ua, const void *Ue, const void *Uw, const void *Ug,
    const float *ca, const float *ce, const float *cw, const float *cg,
    float *a, float *e, float *w, float *g, int B, int T, int H, int d, muir_stream_t stream);

/*
 * The chunk forward with its gates made from the fused low-rank gate projection inside the
 * call (the pages' rank-512 projection; see muir_lowrank_gates for the definition). The
 * decay a and the query gate g are formed inside the parallel phase's kernel, from z rows
 * shared by every head, so their fp32 rows are never read from memory. The erase and write
 * gates e, w are formed inside the sequential phase's kernel when it runs 16-column value
 * tiles (B*H*dv/8 > 256) with chunk <= 128; otherwise the gate kernel writes them into
 * the workspace and the scan reads them back. Either way the result is muir_chunk_fwd's on
 * the gates muir_lowrank_gates makes from the same z, U and c (bit for bit).
 *
 *   q, k, v  as for muir_chunk_fwd, bf16 only (MUIR_ERR_UNSUPPORTED otherwise)
 *   z, U*, c*  as for muir_lowrank_gates (all four gates' up-projections and offsets)
 *   r, s0, o, s_out, sizes: as for muir_chunk_fwd
 *   workspace / workspace_bytes: at least muir_chunk_fwd_lowrank_workspace_size(...) bytes
 *            (the chunk forward's workspace, then room for e and w, used only when the
 *            gate kernel makes them)
 *
 * Errors as for muir_chunk_fwd and muir_lowrank_gates.
 */
size_t muir_chunk_fwd_lowrank_workspace_size(int B, int T, int H, int dk, int dv, int chunk);

muir_status_t muir_chunk_fwd_lowrank(
    const void *q, const void *k, const void *v, const void *z,
    const void *Ua, const void *Ue, const void *Uw, const void *Ug,
    const float *ca, const float *ce, const float *cw, const float *cg, const float *r,
    const float *s0, void *o, float *s_out,
    int B, int T, int H, int dk, int dv, int chunk, muir_dtype_t qkv,
    void *workspace, size_t workspace_bytes, muir_stream_t stream);

/*
 * The output gate from the same fused projection (openai-hub page, section on
 * sensitivity-allocated gating, gate table: the output gate has rank 128 of the 512):
 *   og[b, t, h, j] = sigmoid(z[b, t, 128:256] . Uo[h, j, :] + co[h, j])
 * per value channel j; the gated readout is o_t * og_t (as muir_chunk_fwd_gated applies it).
 *
 *   z        [B, T, 512] bf16 as for muir_lowrank_gates
 *   Uo       [H, d, 128] bf16;  co [H, d] fp32
 *   og       [B, T, H, d] fp32 output
 *
 * Errors as for muir_lowrank_gates (og is required when T > 0).
 */
muir_status_t muir_lowrank_output_gate(const void *z, const void *Uo, const float *co, float *og,
                                       int B, int T, int H, int d, muir_stream_t stream);

/*
 * muir_chunk_fwd_lowrank with the output gate as well: all five gates of the fused
 * projection are made inside the call and the readout is stored as o_t * og_t. og is made
 * like e and w: inside the sequential phase's kernel (from z's output slice, one chunk ahead
 * of the readout) where that kernel makes e and w, otherwise by the gate kernel into the
 * workspace. Either way the result is muir_chunk_fwd_gated's on the gates that
 * muir_lowrank_gates and muir_lowrank_output_gate make from the same z, U and c (bit for
 * bit).
 *
 *   arguments as for muir_chunk_fwd_lowrank, plus Uo [H, dv, 128] bf16 and co [H, dv] fp32
 *   workspace / workspace_bytes: at least muir_chunk_fwd_lowrank_gated_workspace_size(...)
 *            bytes (muir_chunk_fwd_lowrank's, plus room for og)
 *
 * Errors as for muir_chunk_fwd_lowrank (Uo and co are required).
 */
size_t muir_chunk_fwd_lowrank_gated_workspace_size(int B, int T, int H, int dk, int dv, int chunk);

muir_status_t muir_chunk_fwd_lowrank_gated(
    const void *q, const void *k, const void *v, const void *z,
    const void *Ua, const void *Ue, const void *Uw, const void *Ug, const void *Uo,
    const float *ca, const float *ce, const float *cw, const float *cg, const float *co,
    const float *r, const float *s0, void *o, float *s_out,
    int B, int T, int H, int dk, int dv, int chunk, muir_dtype_t qkv,
    void *workspace, size_t workspace_bytes, muir_stream_t stream);

/*
 * One recurrent step per (batch, head), updating the state in place (decode).
 * Constant-memory inference against the fixed state (Muir abstract, "Full text";
 * openai-hub page, opening section: the history lives in a fixed 2-D state, so
 * memory does not grow with context).
 *
 *   q, k    [B, H, dk] dtype `qkv`;  v [B, H, dv] dtype `qkv`
 *   a, g    [B, H, dk] float32;      e, w [B, H, dv] float32;  r [H, dk] float32
 *   state   [B, H, dk, dv] float32, read and written in place
 *   o       [B, H, dv] dtype `qkv`
 *   dk, dv  dk == dv, 64 or 128
 *
 * Errors: MUIR_ERR_NULL for any missing pointer; MUIR_ERR_SHAPE for B < 1, H < 1;
 * MUIR_ERR_UNSUPPORTED for other d; MUIR_ERR_ALIAS when o or state overlaps an input
 * or each other.
 */
muir_status_t muir_decode_step(
    const void *q, const void *k, const void *v,
    const float *a, const float *g, const float *e, const float *w, const float *r,
    float *state, void *o,
    int B, int H, int dk, int dv, muir_dtype_t qkv, muir_stream_t stream);

/*
 * Backward pass of muir_chunk_fwd: every input's gradient of a scalar loss L, given
 * dL/do and dL/ds_out. Training runs the chunk form in both directions (Muir abstract,
 * "Full text": chunkwise-parallel training; openai-hub page, section on the chunkwise
 * algorithm). The gradients are the reverse mode of the same recurrence: per chunk, the
 * transposed triangular system per value column, the state adjoint carried from the chunk
 * end to its start, and decayed key/query products for the rest; no decay is divided by.
 *
 *   q, k, v, a, g, e, w, r, s0   as for muir_chunk_fwd (s0 may be NULL: zero state)
 *   dout     [B, T, H, dv] dtype `qkv`: dL/do
 *   ds_out   [B, H, dk, dv] float32: dL/ds_out, or NULL for zero
 *   dq, dk, dv, dg, de, dw   [B, T, H, d] float32: dL/dq, dL/dk, ...
 *   dla      [B, T, H, dk] float32: a * dL/da, the gradient with respect to log a (finite
 *            where a = 0; callers holding a as a function of its logarithm use it as is)
 *   dr       [H, dk] float32: dL/dr, summed over batch and tokens
 *   ds0      [B, H, dk, dv] float32: dL/ds0, or NULL to skip
 *   chunk    64 (the only chunk size of the backward)
 *   workspace / workspace_bytes: at least muir_chunk_bwd_workspace_size(...) bytes, 256-byte
 *            aligned. The call reruns the forward into it (its prepare and scan, keeping u
 *            and every chunk start state), so no forward result needs to be passed in.
 *
 * Every output is written. Errors: as for muir_chunk_fwd; MUIR_ERR_UNSUPPORTED for chunk
 * != 64; MUIR_ERR_NULL for a missing required pointer; MUIR_ERR_ALIAS when an output
 * overlaps an input, another output or the workspace.
 */
size_t muir_chunk_bwd_workspace_size(int B, int T, int H, int dk, int dv, int chunk,
                                     muir_dtype_t qkv);
muir_status_t muir_chunk_bwd(
    const void *q, const void *k, const void *v,
    const float *a, const float *g, const float *e, const float *w, const float *r,
    const float *s0, const void *dout, const float *ds_out,
    float *dq, float *dk, float *dv, float *dla, float *dg, float *de, float *dw,
    float *dr, float *ds0,
    int B, int T, int H, int dk_, int dv_, int chunk, muir_dtype_t qkv,
    void *workspace, size_t workspace_bytes, muir_stream_t stream);

/*
 * Bytes of the recurrent state of B sequences x H heads, one dk x dv fp32 matrix per head:
 * what muir_decode_step reads and writes per layer and what s0 / s_out of the chunk forward
 * hold. It does not depend on the sequence length: inference runs in constant memory
 * (openai-hub news page, opening section, and the liuch.name summary, opening paragraph: the
 * 24 layers of the 1.34B model, 16 heads of d = 128, keep about 25 MB of fp32 state, here
 * 24 x muir_state_bytes(1, 16, 128, 128) = 25,165,824 bytes per sequence).
 * 0 when a size is below 1 or the product overflows.
 */
size_t muir_state_bytes(int B, int H, int dk, int dv);

/* Static, never-NULL name of a status code ("MUIR_OK", ...). */
const char *muir_status_string(muir_status_t s);

/* Detail of the calling thread's last failed call ("" if none). Valid until the next
 * call on this thread. */
const char *muir_last_error(void);

/* Version of the library as major*10000 + minor*100 + patch. */
int muir_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MUIR_H */
