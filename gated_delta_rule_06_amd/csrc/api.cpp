// C ABI of libmuir: argument validation, workspace sizing and dispatch to the kernels.
// Every check runs on the host before anything is launched.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>
#include <vector>

#include "muir.h"
#include "kernels.hpp"
#include "layout.hpp"

namespace {

thread_local char g_last_error[512] = "";

muir_status_t fail(muir_status_t s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

muir_status_t fail(muir_status_t s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

muir_status_t ok() {
    g_last_error[0] = '\0';
    return MUIR_OK;
}

struct Range {
    const char *name;
    uintptr_t lo, hi;  // [lo, hi)
};

Range range(const char *name, const void *p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, p ? lo + bytes : lo};
}

bool overlaps(const Range &x, const Range &y) {
    if (x.lo == x.hi || y.lo == y.hi) return false;
    return x.lo < y.hi && y.lo < x.hi;
}

// size = a*b*c*d with overflow detection (all factors >= 0).
bool mul_size(size_t &out, std::initializer_list<size_t> f) {
    size_t acc = 1;
    for (size_t x : f) {
        if (x != 0 && acc > SIZE_MAX / x) return false;
        acc *= x;
    }
    out = acc;
    return true;
}

bool supported_d(int d) { return d == 64 || d == 128; }
bool supported_chunk(int c) { return c == 64 || c == 128 || c == 256; }

muir_status_t check_hip(hipError_t err, const char *what) {
    if (err != hipSuccess)
        return fail(MUIR_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
    return ok();
}

}  // namespace

extern "C" {

int muir_version(void) { return 10000; }

const char *muir_status_string(muir_status_t s) {
    switch (s) {
        case MUIR_OK: return "MUIR_OK";
        case MUIR_ERR_NULL: return "MUIR_ERR_NULL";
        case MUIR_ERR_SHAPE: return "MUIR_ERR_SHAPE";
        case MUIR_ERR_UNSUPPORTED: return "MUIR_ERR_UNSUPPORTED";
        case MUIR_ERR_WORKSPACE: return "MUIR_ERR_WORKSPACE";
        case MUIR_ERR_ALIAS: return "MUIR_ERR_ALIAS";
        case MUIR_ERR_HIP: return "MUIR_ERR_HIP";
    }
    return "MUIR_STATUS_UNKNOWN";
}

const char *muir_last_error(void) { return g_last_error; }

size_t muir_state_bytes(int B, int H, int dk, int dv) {
    if (B < 1 || H < 1 || dk < 1 || dv < 1) return 0;
    size_t n;
    if (!mul_size(n, {static_cast<size_t>(B), static_cast<size_t>(H), static_cast<size_t>(dk),
                      static_cast<size_t>(dv), sizeof(float)}))
        return 0;
    return n;
}

size_t muir_chunk_fwd_workspace_size(int B, int T, int H, int dk, int dv, int chunk,
                                     muir_dtype_t qkv) {
    if (B < 1 || T < 0 || H < 1 || dk != dv || !supported_d(dk) || !supported_chunk(chunk))
        return 0;
    if (qkv != MUIR_F32 && qkv != MUIR_BF16) return 0;
    return muir::chunk_workspace_bytes(B, T, H, dk, chunk, qkv == MUIR_BF16);
}

}  // extern "C"

namespace {

// One chunk-forward call as seen by the validator. Pointers a phase does not use are
// NULL; `prep` / `scan` say which phase's inputs and outputs are required.
struct ChunkCall {
    const char *fn;
    const void *q, *k, *v;
    const float *a, *g, *e, *w, *og, *r, *s0;
    void *o;
    float *s_out;
    int B, T, H, dk, dv, chunk;
    muir_dtype_t qkv;
    const void *workspace;
    size_t workspace_bytes;
    bool prep, scan, gated;
    bool scalar_e = false;  // e is [B, T, H] (one erase strength per token): the WY path
};

muir_status_t validate(const ChunkCall &c) {
    const char *fn = c.fn;
    if (c.B < 1 || c.T < 0 || c.H < 1)
        return fail(MUIR_ERR_SHAPE, "%s: need B >= 1, T >= 0, H >= 1 (got B=%d T=%d H=%d)", fn,
                    c.B, c.T, c.H);
    if (c.dk < 1 || c.dv < 1)
        return fail(MUIR_ERR_SHAPE, "%s: dk=%d dv=%d must be positive", fn, c.dk, c.dv);
    if (c.qkv != MUIR_F32 && c.qkv != MUIR_BF16)
        return fail(MUIR_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, static_cast<int>(c.qkv));
    if (c.dk != c.dv || !supported_d(c.dk))
        return fail(MUIR_ERR_UNSUPPORTED, "%s: need dk == dv in {64, 128} (got %d, %d)", fn,
                    c.dk, c.dv);
    if (!supported_chunk(c.chunk))
        return fail(MUIR_ERR_UNSUPPORTED, "%s: chunk must be 64, 128 or 256 (got %d)", fn,
                    c.chunk);
    if (c.scalar_e && c.qkv != MUIR_BF16)
        return fail(MUIR_ERR_UNSUPPORTED, "%s: the shared-erase path needs bf16 q, k, v", fn);
    if (c.T > 0 && c.prep && (!c.q || !c.k || !c.a || !c.g))
        return fail(MUIR_ERR_NULL, "%s: q, k, a and g are required", fn);
    if (c.T > 0 && c.scan && (!c.v || !c.e || !c.w || !c.o))
        return fail(MUIR_ERR_NULL, "%s: v, e, w and o are required", fn);
    if (c.T > 0 && c.gated && !c.og) return fail(MUIR_ERR_NULL, "%s: og is required", fn);
    if (c.prep && !c.r) return fail(MUIR_ERR_NULL, "%s: r is required", fn);

    const size_t es = c.qkv == MUIR_BF16 ? 2 : 4;
    size_t n_tok, n_state;
    if (!mul_size(n_tok, {static_cast<size_t>(c.B), static_cast<size_t>(c.T),
                          static_cast<size_t>(c.H), static_cast<size_t>(c.dk)}) ||
        !mul_size(n_state, {static_cast<size_t>(c.B), static_cast<size_t>(c.H),
                            static_cast<size_t>(c.dk), static_cast<size_t>(c.dv)}) ||
        n_tok > SIZE_MAX / 4 || n_state > SIZE_MAX / 4)
        return fail(MUIR_ERR_SHAPE, "%s: sizes overflow", fn);
    // The scan addresses one head's tokens and its workspace chunks with 32-bit offsets.
    const size_t head_span = static_cast<size_t>(c.T) * c.H * c.dk * 4;
    if (head_span > 0xffffffffu)
        return fail(MUIR_ERR_UNSUPPORTED,
                    "%s: T*H*dv*4 = %zu bytes exceeds 4 GiB; split the sequence over several "
                    "calls, carrying the state through s0 / s_out", fn, head_span);

    const size_t need = c.scalar_e
        ? muir::wy_workspace_bytes(c.B, c.T, c.H, c.dk, c.chunk)
        : muir::chunk_workspace_bytes(c.B, c.T, c.H, c.dk, c.chunk, c.qkv == MUIR_BF16);
    if (need == 0 && c.T > 0) return fail(MUIR_ERR_SHAPE, "%s: workspace size overflows", fn);
    if (need / (static_cast<size_t>(c.B) * c.H) > 0xffffffffu)
        return fail(MUIR_ERR_UNSUPPORTED,
                    "%s: the workspace of one head exceeds 4 GiB; split the sequence over "
                    "several calls, carrying the state through s0 / s_out", fn);
    if (need > 0) {
        if (!c.workspace)
            return fail(MUIR_ERR_WORKSPACE, "%s: workspace of %zu bytes required", fn, need);
        if (c.workspace_bytes < need)
            return fail(MUIR_ERR_WORKSPACE, "%s: workspace has %zu bytes, need %zu", fn,
                        c.workspace_bytes, need);
        if (reinterpret_cast<uintptr_t>(c.workspace) % 256 != 0)
            return fail(MUIR_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
    }
    const void *all[] = {c.q, c.k, c.v, c.a, c.g, c.e, c.w, c.og, c.r, c.s0, c.o, c.s_out};
    for (const void *p : all)
        if (p && reinterpret_cast<uintptr_t>(p) % 16 != 0)
            return fail(MUIR_ERR_SHAPE, "%s: every buffer must be 16-byte aligned", fn);

    const Range inputs[] = {
        range("q", c.q, n_tok * es), range("k", c.k, n_tok * es), range("v", c.v, n_tok * es),
        range("a", c.a, n_tok * 4), range("g", c.g, n_tok * 4),
        range("e", c.e, c.scalar_e ? n_tok / static_cast<size_t>(c.dk) * 4 : n_tok * 4),
        range("w", c.w, n_tok * 4), range("og", c.og, n_tok * 4),
        range("r", c.r, static_cast<size_t>(c.H) * c.dk * 4),
        range("s0", c.s0, n_state * 4)};
    const Range ro = range("o", c.o, n_tok * es);
    const Range rs = range("s_out", c.s_out, n_state * 4);
    const Range rw = range("workspace", c.workspace, need);
    for (const Range &x : inputs) {
        if (overlaps(ro, x)) return fail(MUIR_ERR_ALIAS, "%s: o overlaps %s", fn, x.name);
        if (overlaps(rw, x)) return fail(MUIR_ERR_ALIAS, "%s: workspace overlaps %s", fn, x.name);
        if (overlaps(rs, x) && !(x.lo == rs.lo && x.hi == rs.hi && strcmp(x.name, "s0") == 0))
            return fail(MUIR_ERR_ALIAS, "%s: s_out overlaps %s", fn, x.name);
    }
    if (overlaps(ro, rs) || overlaps(ro, rw) || overlaps(rs, rw))
        return fail(MUIR_ERR_ALIAS, "%s: o, s_out and workspace must not overlap", fn);
    return MUIR_OK;
}

muir_status_t chunk_scan_impl(const ChunkCall &c, muir_stream_t stream) {
    const muir_status_t st = validate(c);
    if (st != MUIR_OK) return st;
    if (c.T == 0 && !c.s_out) return ok();
    return check_hip(muir::launch_chunk_scan(c.v, c.e, c.w, c.og, c.s0, c.o, c.s_out, c.B, c.T,
                                             c.H, c.dk, c.chunk, c.qkv == MUIR_BF16,
                                             const_cast<void *>(c.workspace),
                                             static_cast<hipStream_t>(stream)),
                     c.fn);
}

muir_status_t chunk_fwd_impl(const ChunkCall &c, muir_stream_t stream) {
    const muir_status_t st = validate(c);
    if (st != MUIR_OK) return st;
    if (c.T > 0) {
        const muir_status_t sp = check_hip(
            muir::launch_chunk_prepare(c.q, c.k, c.a, c.g, c.r, c.B, c.T, c.H, c.dk, c.chunk,
                                       c.qkv == MUIR_BF16, const_cast<void *>(c.workspace),
                                       static_cast<hipStream_t>(stream)),
            c.fn);
        if (sp != MUIR_OK) return sp;
    }
    return chunk_scan_impl(c, stream);
}

}  // namespace

extern "C" {

muir_status_t muir_chunk_fwd(const void *q, const void *k, const void *v, const float *a,
                             const float *g, const float *e, const float *w, const float *r,
                             const float *s0, void *o, float *s_out, int B, int T, int H,
                             int dk, int dv, int chunk, muir_dtype_t qkv, void *workspace,
                             size_t workspace_bytes, muir_stream_t stream) {
    return chunk_fwd_impl(ChunkCall{"chunk_fwd", q, k, v, a, g, e, w, nullptr, r, s0, o, s_out,
                                    B, T, H, dk, dv, chunk, qkv, workspace, workspace_bytes,
                                    true, true, false},
                          stream);
}

muir_status_t muir_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *a,
                                     const float *g, const float *e, const float *w,
                                     const float *r, const float *s0, void *o, float *s_out, int B,
                                     int T, int H, int dk, int dv, int chunk, muir_dtype_t qkv,
                                     muir_stream_t stream) {
    const char *fn = "chunk_fwd_noalloc";
    const size_t need = muir_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, qkv);
    if (need > muir::kNoAllocScratchBytes)
        return fail(MUIR_ERR_WORKSPACE,
                    "%s: these sizes need %zu bytes of workspace; the static scratch holds %zu "
                    "(call muir_chunk_fwd with a workspace instead)",
                    fn, need, muir::kNoAllocScratchBytes);
    void *scratch = nullptr;
    size_t scratch_bytes = 0;
    if (need > 0) {
        // Invalid sizes give need == 0 and are reported by the validation below.
        const muir_status_t st = check_hip(muir::noalloc_scratch(&scratch), fn);
        if (st != MUIR_OK) return st;
        scratch_bytes = muir::kNoAllocScratchBytes;
    }
    return chunk_fwd_impl(ChunkCall{fn, q, k, v, a, g, e, w, nullptr, r, s0, o, s_out, B, T, H,
                                    dk, dv, chunk, qkv, scratch, scratch_bytes, true, true, false},
                          stream);
}

size_t muir_chunk_fwd_noalloc_max_workspace(void) { return muir::kNoAllocScratchBytes; }

muir_status_t muir_chunk_fwd_gated(const void *q, const void *k, const void *v, const float *a,
                                   const float *g, const float *e, const float *w,
                                   const float *og, const float *r, const float *s0, void *o,
                                   float *s_out, int B, int T, int H, int dk, int dv, int chunk,
                                   muir_dtype_t qkv, void *workspace, size_t workspace_bytes,
                                   muir_stream_t stream) {
    return chunk_fwd_impl(ChunkCall{"chunk_fwd_gated", q, k, v, a, g, e, w, og, r, s0, o, s_out,
                                    B, T, H, dk, dv, chunk, qkv, workspace, workspace_bytes,
                                    true, true, true},
                          stream);
}

muir_status_t muir_chunk_fwd_prepare(const void *q, const void *k, const float *a,
                                     const float *g, const float *r, int B, int T, int H, int dk,
                                     int chunk, muir_dtype_t qkv, void *workspace,
                                     size_t workspace_bytes, muir_stream_t stream) {
    const ChunkCall c{"chunk_fwd_prepare", q, k, nullptr, a, g, nullptr, nullptr, nullptr, r,
                      nullptr, nullptr, nullptr, B, T, H, dk, dk, chunk, qkv, workspace,
                      workspace_bytes, true, false, false};
    const muir_status_t st = validate(c);
    if (st != MUIR_OK) return st;
    if (T == 0) return ok();
    return check_hip(muir::launch_chunk_prepare(q, k, a, g, r, B, T, H, dk, chunk,
                                                qkv == MUIR_BF16, workspace,
                                                static_cast<hipStream_t>(stream)),
                     "chunk_fwd_prepare launch");
}

muir_status_t muir_chunk_fwd_scan(const void *v, const float *e, const float *w, const float *s0,
                                  void *o, float *s_out, int B, int T, int H, int dk, int dv,
                                  int chunk, muir_dtype_t qkv, void *workspace,
                                  size_t workspace_bytes, muir_stream_t stream) {
    return chunk_scan_impl(ChunkCall{"chunk_fwd_scan", nullptr, nullptr, v, nullptr, nullptr, e,
                                     w, nullptr, nullptr, s0, o, s_out, B, T, H, dk, dv, chunk,
                                     qkv, workspace, workspace_bytes, false, true, false},
                           stream);
}

muir_status_t muir_chunk_fwd_scan_gated(const void *v, const float *e, const float *w,
                                        const float *og, const float *s0, void *o, float *s_out,
                                        int B, int T, int H, int dk, int dv, int chunk,
                                        muir_dtype_t qkv, void *workspace,
                                        size_t workspace_bytes, muir_stream_t stream) {
    return chunk_scan_impl(ChunkCall{"chunk_fwd_scan_gated", nullptr, nullptr, v, nullptr,
                                     nullptr, e, w, og, nullptr, s0, o, s_out, B, T, H, dk, dv,
                                     chunk, qkv, workspace, workspace_bytes, false, true, true},
                           stream);
}

size_t muir_chunk_fwd_scalar_erase_workspace_size(int B, int T, int H, int dk, int dv,
                                                   int chunk) {
    if (B < 1 || T < 0 || H < 1 || dk != dv || !supported_d(dk) || !supported_chunk(chunk))
        return 0;
    return muir::wy_workspace_bytes(B, T, H, dk, chunk);
}

muir_status_t muir_chunk_fwd_scalar_erase(const void *q, const void *k, const void *v,
                                          const float *a, const float *g, const float *e,
                                          const float *w, const float *r, const float *s0,
                                          void *o, float *s_out, int B, int T, int H, int dk,
                                          int dv, int chunk, muir_dtype_t qkv, void *workspace,
                                          size_t workspace_bytes, muir_stream_t stream) {
    ChunkCall c{"chunk_fwd_scalar_erase", q, k, v, a, g, e, w, nullptr, r, s0, o, s_out, B, T, H,
                dk, dv, chunk, qkv, workspace, workspace_bytes, true, true, false};
    c.scalar_e = true;
    const muir_status_t st = validate(c);
    if (st != MUIR_OK) return st;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    if (T > 0) {
        muir_status_t sp = check_hip(muir::launch_chunk_prepare(q, k, a, g, r, B, T, H, dk, chunk,
                                                                true, workspace, hs),
                                     "chunk_fwd_scalar_erase prepare");
        if (sp != MUIR_OK) return sp;
        sp = check_hip(muir::launch_wy_solve(v, e, w, B, T, H, dk, chunk, workspace, hs),
                       "chunk_fwd_scalar_erase solve");
        if (sp != MUIR_OK) return sp;
    } else if (!s_out) {
        return ok();
    }
    return check_hip(muir::launch_wy_scan(s0, o, s_out, B, T, H, dk, chunk, workspace, hs),
                     "chunk_fwd_scalar_erase scan");
}

muir_status_t muir_chunk_fwd_scalar_erase_solve(const void *v, const float *e, const float *w,
                                                int B, int T, int H, int dk, int chunk,
                                                muir_dtype_t qkv, void *workspace,
                                                size_t workspace_bytes, muir_stream_t stream) {
    ChunkCall c{"chunk_fwd_scalar_erase_solve", nullptr, nullptr, v, nullptr, nullptr, e, w,
                nullptr, nullptr, nullptr, nullptr, nullptr, B, T, H, dk, dk, chunk, qkv,
                workspace, workspace_bytes, false, false, false};
    c.scalar_e = true;
    const muir_status_t st = validate(c);
    if (st != MUIR_OK) return st;
    if (T > 0 && (!v || !e || !w))
        return fail(MUIR_ERR_NULL, "chunk_fwd_scalar_erase_solve: v, e and w are required");
    if (T == 0) return ok();
    return check_hip(muir::launch_wy_solve(v, e, w, B, T, H, dk, chunk, workspace,
                                           static_cast<hipStream_t>(stream)),
                     "chunk_fwd_scalar_erase_solve launch");
}

muir_status_t muir_chunk_fwd_scalar_erase_scan(const float *s0, void *o, float *s_out, int B,
                                               int T, int H, int dk, int dv, int chunk,
                                               muir_dtype_t qkv, void *workspace,
                                               size_t workspace_bytes, muir_stream_t stream) {
    ChunkCall c{"chunk_fwd_scalar_erase_scan", nullptr, nullptr, nullptr, nullptr, nullptr,
                nullptr, nullptr, nullptr, nullptr, s0, o, s_out, B, T, H, dk, dv, chunk, qkv,
                workspace, workspace_bytes, false, false, false};
    c.scalar_e = true;
    const muir_status_t st = validate(c);
    if (st != MUIR_OK) return st;
    if (T > 0 && !o) return fail(MUIR_ERR_NULL, "chunk_fwd_scalar_erase_scan: o is required");
    if (T == 0 && !s_out) return ok();
    return check_hip(muir::launch_wy_scan(s0, o, s_out, B, T, H, dk, chunk, workspace,
                                          static_cast<hipStream_t>(stream)),
                     "chunk_fwd_scalar_erase_scan launch");
}

}  // extern "C"

namespace {

// Workspace of the fused low-rank forward: the plain forward's, then (256-byte aligned) e and
// w [B, T, H, dv] fp32, and with the output gate og as well.
size_t lowrank_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, bool gated) {
    const size_t base = muir_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, MUIR_BF16);
    if (base == 0 && T > 0) return 0;
    size_t gates;
    if (!mul_size(gates, {static_cast<size_t>(B), static_cast<size_t>(T), static_cast<size_t>(H),
                          static_cast<size_t>(dv), gated ? size_t(12) : size_t(8)}))
        return 0;
    const size_t aligned = (base + 255) & ~size_t(255);
    return aligned + gates < aligned ? 0 : aligned + gates;
}

// The gate entry points: every requested gate (non-null output) of the five from z.
muir_status_t lowrank_gates_impl(const char *fn, const void *z, const void *Ua, const void *Ue,
                                 const void *Uw, const void *Ug, const void *Uo, const float *ca,
                                 const float *ce, const float *cw, const float *cg,
                                 const float *co, float *a, float *e, float *w, float *g,
                                 float *og, int B, int T, int H, int d, muir_stream_t stream) {
    if (B < 1 || T < 0 || H < 1)
        return fail(MUIR_ERR_SHAPE, "%s: need B >= 1, T >= 0, H >= 1 (got B=%d T=%d H=%d)", fn, B, T, H);
    if (!supported_d(d)) return fail(MUIR_ERR_UNSUPPORTED, "%s: d must be 64 or 128 (got %d)", fn, d);
    struct Gate {
        const char *name;
        const void *U;
        const float *c;
        float *out;
        size_t rank;
    } gates[] = {{"a", Ua, ca, a, 64}, {"e", Ue, ce, e, 64}, {"w", Uw, cw, w, 128},
                 {"g", Ug, cg, g, 128}, {"og", Uo, co, og, 128}};
    constexpr size_t NG = sizeof(gates) / sizeof(gates[0]);
    bool any = false;
    for (const Gate &gt : gates) {
        if (!gt.out) continue;
        any = true;
        if (!gt.U || !gt.c)
            return fail(MUIR_ERR_NULL, "%s: gate %s needs its up-projection and offset", fn, gt.name);
    }
    if (any && T > 0 && !z) return fail(MUIR_ERR_NULL, "%s: z is required", fn);
    size_t n_tok, n_z;
    if (!mul_size(n_tok, {static_cast<size_t>(B), static_cast<size_t>(T), static_cast<size_t>(H),
                          static_cast<size_t>(d)}) ||
        !mul_size(n_z, {static_cast<size_t>(B), static_cast<size_t>(T), 512}) || n_tok > SIZE_MAX / 4)
        return fail(MUIR_ERR_SHAPE, "%s: sizes overflow", fn);
    if (static_cast<size_t>(T) * H * d * 4 > 0xffffffffu || static_cast<size_t>(T) * 512 * 2 > 0xffffffffu)
        return fail(MUIR_ERR_UNSUPPORTED, "%s: one batch row's gates or z exceed 4 GiB", fn);
    std::initializer_list<const void *> ptrs = {z, Ua, Ue, Uw, Ug, Uo, ca, ce, cw, cg, co, a, e, w, g, og};
    for (const void *p : ptrs)
        if (p && reinterpret_cast<uintptr_t>(p) % 16 != 0)
            return fail(MUIR_ERR_SHAPE, "%s: every buffer must be 16-byte aligned", fn);
    std::vector<Range> ins = {range("z", z, n_z * 2)};
    for (const Gate &gt : gates) {
        ins.push_back(range(gt.name, gt.U, static_cast<size_t>(H) * d * gt.rank * 2));
        ins.push_back(range(gt.name, gt.c, static_cast<size_t>(H) * d * 4));
    }
    for (size_t i = 0; i < NG; ++i) {
        const Range ro = range(gates[i].name, gates[i].out, n_tok * 4);
        for (const Range &x : ins)
            if (overlaps(ro, x)) return fail(MUIR_ERR_ALIAS, "%s: gate %s overlaps an input", fn, gates[i].name);
        for (size_t j = i + 1; j < NG; ++j)
            if (overlaps(ro, range(gates[j].name, gates[j].out, n_tok * 4)))
                return fail(MUIR_ERR_ALIAS, "%s: gates %s and %s overlap", fn, gates[i].name, gates[j].name);
    }
    if (!any || T == 0) return ok();
    return check_hip(muir::launch_lowrank_gates(z, Ua, Ue, Uw, Ug, Uo, ca, ce, cw, cg, co, a, e, w, g,
                                                og, B, T, H, d, static_cast<hipStream_t>(stream)),
                     fn);
}

// The fused low-rank forward; with Uo the output gate as well (`gated`).
muir_status_t chunk_fwd_lowrank_impl(const char *fn, const void *q, const void *k, const void *v,
                                     const void *z, const void *Ua, const void *Ue, const void *Uw,
                                     const void *Ug, const void *Uo, const float *ca,
                                     const float *ce, const float *cw, const float *cg,
                                     const float *co, const float *r, const float *s0, void *o,
                                     float *s_out, int B, int T, int H, int dk, int dv, int chunk,
                                     muir_dtype_t qkv, void *workspace, size_t workspace_bytes,
                                     muir_stream_t stream, bool gated) {
    if (qkv != MUIR_BF16)
        return fail(MUIR_ERR_UNSUPPORTED, "%s: the fused low-rank gates need bf16 q, k, v", fn);
    // Shape, pointer, alignment and aliasing checks of the plain forward, with the gate
    // tensors standing in as absent: the gates are made inside the call.
    const size_t base = muir::chunk_workspace_bytes(B, T, H, dk, chunk, true);
    const size_t ebase = (base + 255) & ~size_t(255);
    ChunkCall c{fn, q, k, v, nullptr, nullptr, nullptr, nullptr, nullptr, r, s0, o, s_out, B, T, H,
                dk, dv, chunk, qkv, workspace, workspace_bytes, false, false, false};
    muir_status_t st = validate(c);
    if (st != MUIR_OK) return st;
    if (T > 0 && (!q || !k || !v || !o || !z)) return fail(MUIR_ERR_NULL, "%s: q, k, v, z and o are required", fn);
    if (!r || !Ua || !Ue || !Uw || !Ug || !ca || !ce || !cw || !cg || (gated && (!Uo || !co)))
        return fail(MUIR_ERR_NULL, "%s: r and every up-projection and offset are required", fn);
    const size_t need = lowrank_workspace_bytes(B, T, H, dk, dv, chunk, gated);
    if (need == 0 && T > 0) return fail(MUIR_ERR_SHAPE, "%s: workspace size overflows", fn);
    if (T > 0 && (!workspace || workspace_bytes < need))
        return fail(MUIR_ERR_WORKSPACE, "%s: workspace of %zu bytes required", fn, need);
    if (static_cast<size_t>(T) * 512 * 2 > 0xffffffffu)
        return fail(MUIR_ERR_UNSUPPORTED, "%s: one batch row of z exceeds 4 GiB", fn);
    const size_t n_tok = static_cast<size_t>(B) * T * H * dk;
    const Range ins[] = {range("q", q, n_tok * 2), range("k", k, n_tok * 2), range("v", v, n_tok * 2),
                         range("z", z, static_cast<size_t>(B) * T * 512 * 2),
                         range("Ua", Ua, static_cast<size_t>(H) * dk * 64 * 2),
                         range("Ue", Ue, static_cast<size_t>(H) * dv * 64 * 2),
                         range("Uw", Uw, static_cast<size_t>(H) * dv * 128 * 2),
                         range("Ug", Ug, static_cast<size_t>(H) * dk * 128 * 2),
                         range("Uo", gated ? Uo : nullptr, static_cast<size_t>(H) * dv * 128 * 2),
                         range("ca", ca, static_cast<size_t>(H) * dk * 4), range("ce", ce, static_cast<size_t>(H) * dv * 4),
                         range("cw", cw, static_cast<size_t>(H) * dv * 4), range("cg", cg, static_cast<size_t>(H) * dk * 4),
                         range("co", gated ? co : nullptr, static_cast<size_t>(H) * dv * 4)};
    const Range outs[] = {range("o", o, n_tok * 2), range("workspace", workspace, need),
                          range("s_out", s_out, static_cast<size_t>(B) * H * dk * dv * 4)};
    for (const Range &x : ins) {
        if (x.lo % 16 != 0) return fail(MUIR_ERR_SHAPE, "%s: every buffer must be 16-byte aligned", fn);
        for (const Range &y : outs)
            if (overlaps(x, y)) return fail(MUIR_ERR_ALIAS, "%s: %s overlaps %s", fn, y.name, x.name);
    }
    // validate() checked s0 and r against the base forward's workspace only; the gate kernel
    // writes e and w (and og) past it, up to `need`. s0 may still be s_out (the state in place).
    const Range rs0 = range("s0", s0, static_cast<size_t>(B) * H * dk * dv * 4);
    const Range rr = range("r", r, static_cast<size_t>(H) * dk * 4);
    for (const Range &x : {rs0, rr})
        for (int i = 0; i < 2; ++i)
            if (overlaps(x, outs[i]))
                return fail(MUIR_ERR_ALIAS, "%s: %s overlaps %s", fn, outs[i].name, x.name);
    if (T == 0) {
        if (!s_out) return ok();
        return check_hip(muir::launch_chunk_scan(v, nullptr, nullptr, nullptr, s0, o, s_out, B, T, H,
                                                 dk, chunk, true, workspace,
                                                 static_cast<hipStream_t>(stream)),
                         fn);
    }
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    // The gates the scan reads (e, w and og): made inside the scan where its LDS allows, else
    // by the gate kernel into the workspace's tail first, e and w tile-packed where the split
    // scan reads them (whole cache lines per leaf instead of 32-byte row pieces).
    const bool in_scan = muir::scan_gates_in_kernel(B, H, dv, chunk);
    const bool packed = !in_scan && muir::split_scan_applies(B, H, dv);
    float *e = reinterpret_cast<float *>(static_cast<unsigned char *>(workspace) + ebase);
    float *w = e + n_tok;
    float *og = gated ? w + n_tok : nullptr;
    if (!in_scan) {
        st = check_hip(muir::launch_lowrank_gates(z, nullptr, Ue, Uw, nullptr, gated ? Uo : nullptr,
                                                  nullptr, ce, cw, nullptr, gated ? co : nullptr,
                                                  nullptr, e, w, nullptr, og, B, T, H, dv, hs,
                                                  packed),
                       fn);
        if (st != MUIR_OK) return st;
    }
    st = check_hip(muir::launch_chunk_prepare_lowrank(q, k, z, Ua, Ug, ca, cg, r, B, T, H, dk, chunk,
                                                      workspace, hs),
                   fn);
    if (st != MUIR_OK) return st;
    if (in_scan)
        return check_hip(muir::launch_chunk_scan_lowrank(v, z, Ue, Uw, ce, cw, gated ? Uo : nullptr,
                                                         gated ? co : nullptr, s0, o, s_out, B, T,
                                                         H, dk, chunk, workspace, hs),
                         fn);
    return check_hip(muir::launch_chunk_scan(v, e, w, og, s0, o, s_out, B, T, H, dk, chunk, true,
                                             workspace, hs, packed),
                     fn);
}

}  // namespace

extern "C" {

size_t muir_chunk_fwd_lowrank_workspace_size(int B, int T, int H, int dk, int dv, int chunk) {
    return lowrank_workspace_bytes(B, T, H, dk, dv, chunk, false);
}

size_t muir_chunk_fwd_lowrank_gated_workspace_size(int B, int T, int H, int dk, int dv, int chunk) {
    return lowrank_workspace_bytes(B, T, H, dk, dv, chunk, true);
}

muir_status_t muir_chunk_fwd_lowrank(const void *q, const void *k, const void *v, const void *z,
                                     const void *Ua, const void *Ue, const void *Uw,
                                     const void *Ug, const float *ca, const float *ce,
                                     const float *cw, const float *cg, const float *r,
                                     const float *s0, void *o, float *s_out, int B, int T, int H,
                                     int dk, int dv, int chunk, muir_dtype_t qkv, void *workspace,
                                     size_t workspace_bytes, muir_stream_t stream) {
    return chunk_fwd_lowrank_impl("chunk_fwd_lowrank", q, k, v, z, Ua, Ue, Uw, Ug, nullptr, ca, ce,
                                  cw, cg, nullptr, r, s0, o, s_out, B, T, H, dk, dv, chunk, qkv,
                                  workspace, workspace_bytes, stream, false);
}

muir_status_t muir_chunk_fwd_lowrank_gated(
    const void *q, const void *k, const void *v, const void *z, const void *Ua, const void *Ue,
    const void *Uw, const void *Ug, const void *Uo, const float *ca, const float *ce,
    const float *cw, const float *cg, const float *co, const float *r, const float *s0, void *o,
    float *s_out, int B, int T, int H, int dk, int dv, int chunk, muir_dtype_t qkv,
    void *workspace, size_t workspace_bytes, muir_stream_t stream) {
    return chunk_fwd_lowrank_impl("chunk_fwd_lowrank_gated", q, k, v, z, Ua, Ue, Uw, Ug, Uo, ca, ce,
                                  cw, cg, co, r, s0, o, s_out, B, T, H, dk, dv, chunk, qkv,
                                  workspace, workspace_bytes, stream, true);
}

muir_status_t muir_lowrank_gates(const void *z, const void *Ua, const void *Ue, const void *Uw,
                                const void *Ug, const float *ca, const float *ce, const float *cw,
                                const float *cg, float *a, float *e, float *w, float *g, int B,
                                int T, int H, int d, muir_stream_t stream) {
    return lowrank_gates_impl("lowrank_gates", z, Ua, Ue, Uw, Ug, nullptr, ca, ce, cw, cg, nullptr,
                              a, e, w, g, nullptr, B, T, H, d, stream);
}

muir_status_t muir_lowrank_output_gate(const void *z, const void *Uo, const float *co, float *og,
                                       int B, int T, int H, int d, muir_stream_t stream) {
    if (T > 0 && !og) return fail(MUIR_ERR_NULL, "lowrank_output_gate: og is required");
    return lowrank_gates_impl("lowrank_output_gate", z, nullptr, nullptr, nullptr, nullptr, Uo,
                              nullptr, nullptr, nullptr, nullptr, co, nullptr, nullptr, nullptr,
                              nullptr, og, B, T, H, d, stream);
}

muir_status_t muir_decode_step(const void *q, const void *k, const void *v, const float *a,
                               const float *g, const float *e, const float *w, const float *r,
                               float *state, void *o, int B, int H, int dk, int dv,
                               muir_dtype_t qkv, muir_stream_t stream) {
    if (B < 1 || H < 1)
        return fail(MUIR_ERR_SHAPE, "decode_step: need B >= 1, H >= 1 (got B=%d H=%d)", B, H);
    if (dk < 1 || dv < 1)
        return fail(MUIR_ERR_SHAPE, "decode_step: dk=%d dv=%d must be positive", dk, dv);
    if (qkv != MUIR_F32 && qkv != MUIR_BF16)
        return fail(MUIR_ERR_UNSUPPORTED, "decode_step: unknown dtype %d", static_cast<int>(qkv));
    if (dk != dv || !supported_d(dk))
        return fail(MUIR_ERR_UNSUPPORTED, "decode_step: need dk == dv in {64, 128} (got %d, %d)",
                    dk, dv);
    if (!q || !k || !v || !a || !g || !e || !w || !r || !state || !o)
        return fail(MUIR_ERR_NULL, "decode_step: every pointer is required");
    for (const void *p : {q, k, v, static_cast<const void *>(o), static_cast<const void *>(a), static_cast<const void *>(g),
                          static_cast<const void *>(e), static_cast<const void *>(w),
                          static_cast<const void *>(r), static_cast<const void *>(state)})
        if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
            return fail(MUIR_ERR_SHAPE, "decode_step: every buffer must be 16-byte aligned");
    const size_t es = qkv == MUIR_BF16 ? 2 : 4;
    size_t n_vec, n_state;
    if (!mul_size(n_vec, {static_cast<size_t>(B), static_cast<size_t>(H), static_cast<size_t>(dk)}) ||
        !mul_size(n_state, {n_vec, static_cast<size_t>(dv)}) || n_state > SIZE_MAX / 4)
        return fail(MUIR_ERR_SHAPE, "decode_step: sizes overflow");
    const Range inputs[] = {
        range("q", q, n_vec * es), range("k", k, n_vec * es), range("v", v, n_vec * es),
        range("a", a, n_vec * 4), range("g", g, n_vec * 4), range("e", e, n_vec * 4),
        range("w", w, n_vec * 4), range("r", r, static_cast<size_t>(H) * dk * 4)};
    const Range ro = range("o", o, n_vec * es);
    const Range rs = range("state", state, n_state * 4);
    for (const Range &x : inputs) {
        if (overlaps(ro, x)) return fail(MUIR_ERR_ALIAS, "decode_step: o overlaps %s", x.name);
        if (overlaps(rs, x)) return fail(MUIR_ERR_ALIAS, "decode_step: state overlaps %s", x.name);
    }
    if (overlaps(ro, rs)) return fail(MUIR_ERR_ALIAS, "decode_step: o overlaps state");
    return check_hip(muir::launch_decode_step(q, k, v, a, g, e, w, r, state, o, B, H, dk,
                                              qkv == MUIR_BF16, static_cast<hipStream_t>(stream)),
                     "decode_step launch");
}

size_t muir_chunk_bwd_workspace_size(int B, int T, int H, int dk, int dv, int chunk,
                                     muir_dtype_t qkv) {
    if (B < 1 || T < 0 || H < 1 || dk != dv || !supported_d(dk) || chunk != 64) return 0;
    if (qkv != MUIR_F32 && qkv != MUIR_BF16) return 0;
    return muir::chunk_bwd_workspace_bytes(B, T, H, dk, qkv == MUIR_BF16);
}

muir_status_t muir_chunk_bwd(const void *q, const void *k, const void *v, const float *a,
                             const float *g, const float *e, const float *w, const float *r,
                             const float *s0, const void *dout, const float *ds_out, float *dq,
                             float *dk, float *dv, float *dla, float *dg, float *de, float *dw,
                             float *dr, float *ds0, int B, int T, int H, int dk_, int dv_,
                             int chunk, muir_dtype_t qkv, void *workspace,
                             size_t workspace_bytes, muir_stream_t stream) {
    const char *fn = "chunk_bwd";
    if (B < 1 || T < 0 || H < 1)
        return fail(MUIR_ERR_SHAPE, "%s: need B >= 1, T >= 0, H >= 1 (got B=%d T=%d H=%d)", fn,
                    B, T, H);
    if (qkv != MUIR_F32 && qkv != MUIR_BF16)
        return fail(MUIR_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, static_cast<int>(qkv));
    if (dk_ != dv_ || !supported_d(dk_))
        return fail(MUIR_ERR_UNSUPPORTED, "%s: need dk == dv in {64, 128} (got %d, %d)", fn,
                    dk_, dv_);
    if (chunk != 64)
        return fail(MUIR_ERR_UNSUPPORTED, "%s: the backward runs on chunks of 64 (got %d)", fn,
                    chunk);
    if (!r || !dr) return fail(MUIR_ERR_NULL, "%s: r and dr are required", fn);
    if (T > 0 && (!q || !k || !v || !a || !g || !e || !w || !dout || !dq || !dk || !dv ||
                  !dla || !dg || !de || !dw))
        return fail(MUIR_ERR_NULL, "%s: every input and gradient pointer except s0, ds_out "
                    "and ds0 is required", fn);
    const int d = dk_;
    const size_t es = qkv == MUIR_BF16 ? 2 : 4;
    size_t n_tok, n_state;
    if (!mul_size(n_tok, {static_cast<size_t>(B), static_cast<size_t>(T), static_cast<size_t>(H),
                          static_cast<size_t>(d)}) ||
        !mul_size(n_state, {static_cast<size_t>(B), static_cast<size_t>(H), static_cast<size_t>(d),
                            static_cast<size_t>(d)}) ||
        n_tok > SIZE_MAX / 4 || n_state > SIZE_MAX / 4)
        return fail(MUIR_ERR_SHAPE, "%s: sizes overflow", fn);
    const size_t head_span = static_cast<size_t>(T) * H * d * 4;
    if (head_span > 0xffffffffu)
        return fail(MUIR_ERR_UNSUPPORTED, "%s: T*H*d*4 = %zu bytes exceeds 4 GiB", fn, head_span);
    const size_t need = muir::chunk_bwd_workspace_bytes(B, T, H, d, qkv == MUIR_BF16);
    if (need == 0) return fail(MUIR_ERR_SHAPE, "%s: workspace size overflows", fn);
    if (muir::chunk_slots_bytes(B, T, H, d, 64, qkv == MUIR_BF16) /
            (static_cast<size_t>(B) * H) > 0xffffffffu)
        return fail(MUIR_ERR_UNSUPPORTED, "%s: the forward workspace of one head exceeds 4 GiB",
                    fn);
    if (!workspace)
        return fail(MUIR_ERR_WORKSPACE, "%s: workspace of %zu bytes required", fn, need);
    if (workspace_bytes < need)
        return fail(MUIR_ERR_WORKSPACE, "%s: workspace has %zu bytes, need %zu", fn,
                    workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return fail(MUIR_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
    const void *all[] = {q, k, v, a, g, e, w, r, s0, dout, ds_out, dq, dk, dv, dla, dg, de, dw,
                         dr, ds0};
    for (const void *p : all)
        if (p && reinterpret_cast<uintptr_t>(p) % 16 != 0)
            return fail(MUIR_ERR_SHAPE, "%s: every buffer must be 16-byte aligned", fn);
    const Range inputs[] = {
        range("q", q, n_tok * es), range("k", k, n_tok * es), range("v", v, n_tok * es),
        range("a", a, n_tok * 4), range("g", g, n_tok * 4), range("e", e, n_tok * 4),
        range("w", w, n_tok * 4), range("r", r, static_cast<size_t>(H) * d * 4),
        range("s0", s0, n_state * 4), range("dout", dout, n_tok * es),
        range("ds_out", ds_out, n_state * 4)};
    const Range outputs[] = {
        range("dq", dq, n_tok * 4), range("dk", dk, n_tok * 4), range("dv", dv, n_tok * 4),
        range("dla", dla, n_tok * 4), range("dg", dg, n_tok * 4), range("de", de, n_tok * 4),
        range("dw", dw, n_tok * 4), range("dr", dr, static_cast<size_t>(H) * d * 4),
        range("ds0", ds0, n_state * 4), range("workspace", workspace, need)};
    for (const Range &o : outputs) {
        for (const Range &x : inputs)
            if (overlaps(o, x)) return fail(MUIR_ERR_ALIAS, "%s: %s overlaps %s", fn, o.name, x.name);
        for (const Range &y : outputs)
            if (&y != &o && overlaps(o, y))
                return fail(MUIR_ERR_ALIAS, "%s: %s overlaps %s", fn, o.name, y.name);
    }
    const muir::ChunkBwdArgs args{q, k, v, a, g, e, w, r, s0, dout, ds_out,
                                  dq, dk, dv, dla, dg, de, dw, dr, ds0};
    return check_hip(muir::launch_chunk_bwd(args, B, T, H, d, qkv == MUIR_BF16, workspace,
                                            static_cast<hipStream_t>(stream)),
                     fn);
}

}  // extern "C"
