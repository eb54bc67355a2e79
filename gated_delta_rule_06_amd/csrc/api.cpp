// C ABI of libmuir: argument validation, workspace sizing and dispatch to the kernels.
// Every check runs on the host before anything is launched.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "muir.h"
#include "kernels.hpp"

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

size_t muir_chunk_fwd_workspace_size(int B, int T, int H, int dk, int dv, int chunk,
                                     muir_dtype_t qkv) {
    if (B < 1 || T < 0 || H < 1 || dk != dv || !supported_d(dk) || !supported_chunk(chunk))
        return 0;
    if (qkv != MUIR_F32 && qkv != MUIR_BF16) return 0;
    return muir::chunk_workspace_bytes(B, T, H, dk, chunk, qkv == MUIR_BF16);
}

muir_status_t muir_chunk_fwd(const void *q, const void *k, const void *v, const float *a,
                             const float *g, const float *e, const float *w, const float *r,
                             const float *s0, void *o, float *s_out, int B, int T, int H,
                             int dk, int dv, int chunk, muir_dtype_t qkv, void *workspace,
                             size_t workspace_bytes, muir_stream_t stream) {
    if (B < 1 || T < 0 || H < 1)
        return fail(MUIR_ERR_SHAPE, "chunk_fwd: need B >= 1, T >= 0, H >= 1 (got B=%d T=%d H=%d)",
                    B, T, H);
    if (dk < 1 || dv < 1)
        return fail(MUIR_ERR_SHAPE, "chunk_fwd: dk=%d dv=%d must be positive", dk, dv);
    if (qkv != MUIR_F32 && qkv != MUIR_BF16)
        return fail(MUIR_ERR_UNSUPPORTED, "chunk_fwd: unknown dtype %d", static_cast<int>(qkv));
    if (dk != dv || !supported_d(dk))
        return fail(MUIR_ERR_UNSUPPORTED, "chunk_fwd: need dk == dv in {64, 128} (got %d, %d)",
                    dk, dv);
    if (!supported_chunk(chunk))
        return fail(MUIR_ERR_UNSUPPORTED, "chunk_fwd: chunk must be 64, 128 or 256 (got %d)",
                    chunk);
    if (T > 0 && (!q || !k || !v || !a || !g || !e || !w || !o))
        return fail(MUIR_ERR_NULL, "chunk_fwd: q, k, v, a, g, e, w and o are required");
    if (!r) return fail(MUIR_ERR_NULL, "chunk_fwd: r is required");

    const size_t es = qkv == MUIR_BF16 ? 2 : 4;
    size_t n_tok, n_state;
    if (!mul_size(n_tok, {static_cast<size_t>(B), static_cast<size_t>(T),
                          static_cast<size_t>(H), static_cast<size_t>(dk)}) ||
        !mul_size(n_state, {static_cast<size_t>(B), static_cast<size_t>(H),
                            static_cast<size_t>(dk), static_cast<size_t>(dv)}) ||
        n_tok > SIZE_MAX / 4 || n_state > SIZE_MAX / 4)
        return fail(MUIR_ERR_SHAPE, "chunk_fwd: sizes overflow");

    const size_t need = muir::chunk_workspace_bytes(B, T, H, dk, chunk, qkv == MUIR_BF16);
    if (need == 0 && T > 0) return fail(MUIR_ERR_SHAPE, "chunk_fwd: workspace size overflows");
    if (need > 0) {
        if (!workspace)
            return fail(MUIR_ERR_WORKSPACE, "chunk_fwd: workspace of %zu bytes required", need);
        if (workspace_bytes < need)
            return fail(MUIR_ERR_WORKSPACE, "chunk_fwd: workspace has %zu bytes, need %zu",
                        workspace_bytes, need);
        if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
            return fail(MUIR_ERR_WORKSPACE, "chunk_fwd: workspace must be 256-byte aligned");
    }
    for (const void *p : {q, k, v, static_cast<const void *>(o), static_cast<const void *>(a), static_cast<const void *>(g),
                          static_cast<const void *>(e), static_cast<const void *>(w),
                          static_cast<const void *>(r), static_cast<const void *>(s0),
                          static_cast<const void *>(s_out)})
        if (p && reinterpret_cast<uintptr_t>(p) % 16 != 0)
            return fail(MUIR_ERR_SHAPE, "chunk_fwd: every buffer must be 16-byte aligned");

    const Range inputs[] = {
        range("q", q, n_tok * es), range("k", k, n_tok * es), range("v", v, n_tok * es),
        range("a", a, n_tok * 4), range("g", g, n_tok * 4), range("e", e, n_tok * 4),
        range("w", w, n_tok * 4), range("r", r, static_cast<size_t>(H) * dk * 4),
        range("s0", s0, n_state * 4)};
    const Range ro = range("o", o, n_tok * es);
    const Range rs = range("s_out", s_out, n_state * 4);
    const Range rw = range("workspace", workspace, need);
    for (const Range &x : inputs) {
        if (overlaps(ro, x)) return fail(MUIR_ERR_ALIAS, "chunk_fwd: o overlaps %s", x.name);
        if (overlaps(rw, x))
            return fail(MUIR_ERR_ALIAS, "chunk_fwd: workspace overlaps %s", x.name);
        if (overlaps(rs, x) && !(x.lo == rs.lo && x.hi == rs.hi && strcmp(x.name, "s0") == 0))
            return fail(MUIR_ERR_ALIAS, "chunk_fwd: s_out overlaps %s", x.name);
    }
    if (overlaps(ro, rs) || overlaps(ro, rw) || overlaps(rs, rw))
        return fail(MUIR_ERR_ALIAS, "chunk_fwd: o, s_out and workspace must not overlap");

    if (T == 0 && !s_out) return ok();
    return check_hip(muir::launch_chunk_fwd(q, k, v, a, g, e, w, r, s0, o, s_out, B, T, H, dk,
                                            chunk, qkv == MUIR_BF16, workspace,
                                            static_cast<hipStream_t>(stream)),
                     "chunk_fwd launch");
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

}  // extern "C"
