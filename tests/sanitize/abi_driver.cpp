// Drives every entry point of libmuir's C ABI through its host-side logic (argument checks,
// workspace sizes, alias checks, error paths) against stub launchers, for a build with the
// address and undefined-behaviour sanitizers. Buffers are stand-in addresses that the host
// code only compares, never dereferences. Exit status 0 when every call returned the status
// the header documents.
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "muir.h"

extern "C" int stub_launches(void);
extern "C" void stub_fail_launches(int fail);
extern "C" void stub_gates_in_kernel(int on);

namespace {

int g_failures = 0;

void expect(muir_status_t got, muir_status_t want, const char *what) {
    if (got != want) {
        ++g_failures;
        printf("FAIL %s: got %s, want %s (%s)\n", what, muir_status_string(got),
               muir_status_string(want), muir_last_error());
    }
}

void expect_true(bool ok, const char *what) {
    if (!ok) {
        ++g_failures;
        printf("FAIL %s\n", what);
    }
}

// Stand-in device addresses: disjoint, 256-byte aligned, never dereferenced.
struct Arena {
    uintptr_t next = uintptr_t(0x100000000000ull);
    template <typename P = void>
    P *take(size_t bytes) {
        const uintptr_t p = next;
        next += (bytes + 4095) / 4096 * 4096 + 4096;
        return reinterpret_cast<P *>(p);
    }
};

struct Shape {
    int B, T, H, d, chunk;
    muir_dtype_t qkv;
};

void run_shape(const Shape &s) {
    char what[256];
    Arena ar;
    const size_t es = s.qkv == MUIR_BF16 ? 2 : 4;
    const size_t ntok = size_t(s.B) * s.T * s.H * s.d, nst = size_t(s.B) * s.H * s.d * s.d;
    void *q = ar.take(ntok * es), *k = ar.take(ntok * es), *v = ar.take(ntok * es);
    float *a = ar.take<float>(ntok * 4), *g = ar.take<float>(ntok * 4);
    float *e = ar.take<float>(ntok * 4), *w = ar.take<float>(ntok * 4);
    float *og = ar.take<float>(ntok * 4), *r = ar.take<float>(size_t(s.H) * s.d * 4);
    float *s0 = ar.take<float>(nst * 4), *s_out = ar.take<float>(nst * 4);
    void *o = ar.take(ntok * es);
    const size_t need = muir_chunk_fwd_workspace_size(s.B, s.T, s.H, s.d, s.d, s.chunk, s.qkv);
    void *ws = ar.take(need + 256);
    const int T = s.T;
#define SHAPE_TAG(name) (snprintf(what, sizeof what, "%s B=%d T=%d H=%d d=%d C=%d %s", name, s.B, \
                                  s.T, s.H, s.d, s.chunk, s.qkv == MUIR_BF16 ? "bf16" : "f32"), what)

    expect_true(T == 0 || need > 0, SHAPE_TAG("workspace size"));
    int before = stub_launches();
    expect(muir_chunk_fwd(q, k, v, a, g, e, w, r, s0, o, s_out, s.B, T, s.H, s.d, s.d, s.chunk,
                          s.qkv, ws, need, nullptr), MUIR_OK, SHAPE_TAG("chunk_fwd"));
    expect_true(T == 0 || stub_launches() > before, SHAPE_TAG("chunk_fwd launches"));
    expect(muir_chunk_fwd(q, k, v, a, g, e, w, r, s0, o, s0, s.B, T, s.H, s.d, s.d, s.chunk,
                          s.qkv, ws, need, nullptr), MUIR_OK, SHAPE_TAG("chunk_fwd in place"));
    expect(muir_chunk_fwd(q, k, v, a, g, e, w, r, nullptr, o, nullptr, s.B, T, s.H, s.d, s.d,
                          s.chunk, s.qkv, ws, need, nullptr), MUIR_OK, SHAPE_TAG("chunk_fwd no state"));
    if (T > 0) {
        expect(muir_chunk_fwd(nullptr, k, v, a, g, e, w, r, s0, o, s_out, s.B, T, s.H, s.d, s.d,
                              s.chunk, s.qkv, ws, need, nullptr), MUIR_ERR_NULL, SHAPE_TAG("null q"));
        expect(muir_chunk_fwd(q, k, v, a, g, e, w, r, s0, o, s_out, s.B, T, s.H, s.d, s.d, s.chunk,
                              s.qkv, ws, need - 1, nullptr), MUIR_ERR_WORKSPACE, SHAPE_TAG("short ws"));
        expect(muir_chunk_fwd(q, k, v, a, g, e, w, r, s0, o, s_out, s.B, T, s.H, s.d, s.d, s.chunk,
                              s.qkv, static_cast<char *>(ws) + 16, need, nullptr),
               MUIR_ERR_WORKSPACE, SHAPE_TAG("misaligned ws"));
        expect(muir_chunk_fwd(q, k, v, a, g, e, w, r, s0, q, s_out, s.B, T, s.H, s.d, s.d, s.chunk,
                              s.qkv, ws, need, nullptr), MUIR_ERR_ALIAS, SHAPE_TAG("o aliases q"));
        expect(muir_chunk_fwd(q, k, v, a, g, e, w, r, s0, o, s_out, s.B, T, s.H, s.d, s.d, s.chunk,
                              s.qkv, a, need, nullptr), MUIR_ERR_ALIAS, SHAPE_TAG("ws aliases a"));
        stub_fail_launches(1);
        expect(muir_chunk_fwd(q, k, v, a, g, e, w, r, s0, o, s_out, s.B, T, s.H, s.d, s.d, s.chunk,
                              s.qkv, ws, need, nullptr), MUIR_ERR_HIP, SHAPE_TAG("launch failure"));
        expect_true(strlen(muir_last_error()) > 0, SHAPE_TAG("error detail"));
        stub_fail_launches(0);
    }
    // The two phases, the gated forms and the allocation-free form.
    expect(muir_chunk_fwd_prepare(q, k, a, g, r, s.B, T, s.H, s.d, s.chunk, s.qkv, ws, need,
                                  nullptr), MUIR_OK, SHAPE_TAG("prepare"));
    expect(muir_chunk_fwd_scan(v, e, w, s0, o, s_out, s.B, T, s.H, s.d, s.d, s.chunk, s.qkv, ws,
                               need, nullptr), MUIR_OK, SHAPE_TAG("scan"));
    expect(muir_chunk_fwd_gated(q, k, v, a, g, e, w, og, r, s0, o, s_out, s.B, T, s.H, s.d, s.d,
                                s.chunk, s.qkv, ws, need, nullptr), MUIR_OK, SHAPE_TAG("gated"));
    expect(muir_chunk_fwd_scan_gated(v, e, w, og, s0, o, s_out, s.B, T, s.H, s.d, s.d, s.chunk,
                                     s.qkv, ws, need, nullptr), MUIR_OK, SHAPE_TAG("scan gated"));
    if (T > 0)
        expect(muir_chunk_fwd_gated(q, k, v, a, g, e, w, nullptr, r, s0, o, s_out, s.B, T, s.H, s.d,
                                    s.d, s.chunk, s.qkv, ws, need, nullptr), MUIR_ERR_NULL,
               SHAPE_TAG("gated without og"));
    expect(muir_chunk_fwd_noalloc(q, k, v, a, g, e, w, r, s0, o, s_out, s.B, T, s.H, s.d, s.d,
                                  s.chunk, s.qkv, nullptr),
           need <= muir_chunk_fwd_noalloc_max_workspace() ? MUIR_OK : MUIR_ERR_WORKSPACE,
           SHAPE_TAG("noalloc"));

    // Shared erase: e is [B, T, H]; bf16 operands only.
    const size_t wyn = muir_chunk_fwd_scalar_erase_workspace_size(s.B, T, s.H, s.d, s.d, s.chunk);
    void *wyws = ar.take(wyn + 256);
    float *es1 = ar.take<float>(size_t(s.B) * T * s.H * 4);
    const muir_status_t want_se = s.qkv == MUIR_BF16 ? MUIR_OK : MUIR_ERR_UNSUPPORTED;
    expect(muir_chunk_fwd_scalar_erase(q, k, v, a, g, es1, w, r, s0, o, s_out, s.B, T, s.H, s.d,
                                       s.d, s.chunk, s.qkv, wyws, wyn, nullptr), want_se,
           SHAPE_TAG("scalar erase"));
    if (s.qkv == MUIR_BF16) {
        expect(muir_chunk_fwd_scalar_erase_solve(v, es1, w, s.B, T, s.H, s.d, s.chunk, s.qkv, wyws,
                                                 wyn, nullptr), MUIR_OK, SHAPE_TAG("scalar erase solve"));
        expect(muir_chunk_fwd_scalar_erase_scan(s0, o, s_out, s.B, T, s.H, s.d, s.d, s.chunk, s.qkv,
                                                wyws, wyn, nullptr), MUIR_OK, SHAPE_TAG("scalar erase scan"));
    }

    // Low-rank gates: z [B, T, 512], ranks 64 / 64 / 128 / 128, offsets [H, d].
    void *z = ar.take(size_t(s.B) * T * 512 * 2);
    void *Ua = ar.take(size_t(s.H) * s.d * 64 * 2), *Ue = ar.take(size_t(s.H) * s.d * 64 * 2);
    void *Uw = ar.take(size_t(s.H) * s.d * 128 * 2), *Ug = ar.take(size_t(s.H) * s.d * 128 * 2);
    float *ca = ar.take<float>(size_t(s.H) * s.d * 4), *ce = ar.take<float>(size_t(s.H) * s.d * 4);
    float *cw = ar.take<float>(size_t(s.H) * s.d * 4), *cg = ar.take<float>(size_t(s.H) * s.d * 4);
    expect(muir_lowrank_gates(z, Ua, Ue, Uw, Ug, ca, ce, cw, cg, a, e, w, g, s.B, T, s.H, s.d,
                              nullptr), MUIR_OK, SHAPE_TAG("lowrank gates"));
    const size_t lrn = muir_chunk_fwd_lowrank_workspace_size(s.B, T, s.H, s.d, s.d, s.chunk);
    void *lrws = ar.take(lrn + 256);
    for (int in_kernel = 0; in_kernel < 2; ++in_kernel) {
        stub_gates_in_kernel(in_kernel);
        expect(muir_chunk_fwd_lowrank(q, k, v, z, Ua, Ue, Uw, Ug, ca, ce, cw, cg, r, s0, o, s_out,
                                      s.B, T, s.H, s.d, s.d, s.chunk, s.qkv, lrws, lrn, nullptr),
               s.qkv == MUIR_BF16 ? MUIR_OK : MUIR_ERR_UNSUPPORTED, SHAPE_TAG("lowrank fwd"));
    }
    // The output gate, alone and in the fused forward.
    void *Uo = ar.take(size_t(s.H) * s.d * 128 * 2);
    float *co = ar.take<float>(size_t(s.H) * s.d * 4);
    float *og2 = ar.take<float>(ntok * 4);
    expect(muir_lowrank_output_gate(z, Uo, co, og2, s.B, T, s.H, s.d, nullptr), MUIR_OK,
           SHAPE_TAG("output gate"));
    if (T > 0)
        expect(muir_lowrank_output_gate(z, Uo, co, nullptr, s.B, T, s.H, s.d, nullptr), MUIR_ERR_NULL,
               SHAPE_TAG("output gate without og"));
    const size_t lgn = muir_chunk_fwd_lowrank_gated_workspace_size(s.B, T, s.H, s.d, s.d, s.chunk);
    expect_true(T == 0 || lgn > lrn, SHAPE_TAG("gated low-rank workspace"));
    void *lgws = ar.take(lgn + 256);
    for (int in_kernel = 0; in_kernel < 2; ++in_kernel) {
        stub_gates_in_kernel(in_kernel);
        expect(muir_chunk_fwd_lowrank_gated(q, k, v, z, Ua, Ue, Uw, Ug, Uo, ca, ce, cw, cg, co, r, s0,
                                            o, s_out, s.B, T, s.H, s.d, s.d, s.chunk, s.qkv, lgws, lgn,
                                            nullptr),
               s.qkv == MUIR_BF16 ? MUIR_OK : MUIR_ERR_UNSUPPORTED, SHAPE_TAG("lowrank gated fwd"));
    }
    if (T > 0 && s.qkv == MUIR_BF16)
        expect(muir_chunk_fwd_lowrank_gated(q, k, v, z, Ua, Ue, Uw, Ug, nullptr, ca, ce, cw, cg, co, r,
                                            s0, o, s_out, s.B, T, s.H, s.d, s.d, s.chunk, s.qkv, lgws,
                                            lgn, nullptr),
               MUIR_ERR_NULL, SHAPE_TAG("lowrank gated fwd without Uo"));
    stub_gates_in_kernel(0);

    // Decode step on [B, H, d] tokens against a [B, H, d, d] state.
    float *state = ar.take<float>(nst * 4);
    expect(muir_decode_step(q, k, v, a, g, e, w, r, state, o, s.B, s.H, s.d, s.d, s.qkv, nullptr),
           MUIR_OK, SHAPE_TAG("decode"));
    expect(muir_decode_step(q, k, v, a, g, e, w, r, state, q, s.B, s.H, s.d, s.d, s.qkv, nullptr),
           MUIR_ERR_ALIAS, SHAPE_TAG("decode o aliases q"));

    // Backward (64-token chunks).
    const size_t bn = muir_chunk_bwd_workspace_size(s.B, T, s.H, s.d, s.d, 64, s.qkv);
    void *bws = ar.take(bn + 256), *dout = ar.take(ntok * es);
    float *ds_out = ar.take<float>(nst * 4);
    float *grads[8];
    for (float *&p : grads) p = ar.take<float>(ntok * 4);
    float *dr = ar.take<float>(size_t(s.H) * s.d * 4), *ds0 = ar.take<float>(nst * 4);
    expect(muir_chunk_bwd(q, k, v, a, g, e, w, r, s0, dout, ds_out, grads[0], grads[1], grads[2],
                          grads[3], grads[4], grads[5], grads[6], dr, ds0, s.B, T, s.H, s.d, s.d,
                          64, s.qkv, bws, bn, nullptr), MUIR_OK, SHAPE_TAG("bwd"));
#undef SHAPE_TAG
}

}  // namespace

int main() {
    const Shape shapes[] = {
        {1, 256, 2, 64, 64, MUIR_BF16}, {2, 300, 3, 128, 256, MUIR_BF16},
        {1, 65, 1, 64, 128, MUIR_F32},  {3, 1, 2, 128, 64, MUIR_F32},
        {1, 0, 2, 64, 256, MUIR_BF16},  {1, 32768, 16, 128, 256, MUIR_BF16},
    };
    for (const Shape &s : shapes) run_shape(s);

    // Sizes and codes the header calls invalid.
    expect_true(muir_chunk_fwd_workspace_size(0, 256, 2, 64, 64, 64, MUIR_BF16) == 0, "B = 0 size");
    expect_true(muir_chunk_fwd_workspace_size(1, 256, 2, 96, 96, 64, MUIR_BF16) == 0, "d = 96 size");
    expect_true(muir_chunk_fwd_workspace_size(1, 256, 2, 64, 128, 64, MUIR_BF16) == 0, "dk != dv size");
    expect_true(muir_chunk_fwd_workspace_size(1, 256, 2, 64, 64, 32, MUIR_BF16) == 0, "chunk 32 size");
    expect_true(muir_chunk_fwd_workspace_size(1, 256, 2, 64, 64, 64, (muir_dtype_t)7) == 0, "dtype 7");
    expect_true(muir_chunk_fwd_workspace_size(INT_MAX, INT_MAX, INT_MAX, 128, 128, 64, MUIR_F32) == 0,
                "overflowing size");
    Arena ar;
    void *p = ar.take(1 << 20), *ws = ar.take(1 << 20);
    float *f = ar.take<float>(1 << 20), *o = ar.take<float>(1 << 20);
    expect(muir_chunk_fwd(p, p, p, f, f, f, f, f, nullptr, o, nullptr, 0, 256, 2, 64, 64, 64,
                          MUIR_BF16, ws, 1 << 20, nullptr), MUIR_ERR_SHAPE, "B = 0");
    expect(muir_chunk_fwd(p, p, p, f, f, f, f, f, nullptr, o, nullptr, 1, 256, 2, 96, 96, 64,
                          MUIR_BF16, ws, 1 << 20, nullptr), MUIR_ERR_UNSUPPORTED, "d = 96");
    expect(muir_chunk_fwd(p, p, p, f, f, f, f, f, nullptr, o, nullptr, 1, 256, 2, 64, 64, 32,
                          MUIR_BF16, ws, 1 << 20, nullptr), MUIR_ERR_UNSUPPORTED, "chunk 32");
    expect(muir_chunk_fwd(p, p, p, f, f, f, f, f, nullptr, o, nullptr, 1, INT_MAX, 16, 128, 128,
                          256, MUIR_BF16, ws, 1 << 20, nullptr), MUIR_ERR_UNSUPPORTED,
           "one head past 4 GiB");
    expect(muir_chunk_fwd(p, p, p, f, f, f, f, f, nullptr, o, nullptr, INT_MAX, INT_MAX, INT_MAX,
                          128, 128, 256, MUIR_BF16, ws, 1 << 20, nullptr), MUIR_ERR_SHAPE,
           "overflowing sizes");
    expect(muir_chunk_bwd(p, p, p, f, f, f, f, f, nullptr, p, nullptr, f, f, f, f, f, f, f,
                          nullptr, nullptr, 1, 256, 2, 64, 64, 128, MUIR_BF16, ws, 1 << 20, nullptr),
           MUIR_ERR_UNSUPPORTED, "bwd chunk 128");
    for (int c = 0; c <= 7; ++c)
        expect_true(strlen(muir_status_string(static_cast<muir_status_t>(c))) > 0, "status string");
    expect_true(muir_version() > 0, "version");
    expect_true(24 * muir_state_bytes(1, 16, 128, 128) == 25165824, "state bytes");
    expect_true(muir_state_bytes(INT_MAX, INT_MAX, INT_MAX, INT_MAX) == 0, "state bytes overflow");
    expect_true(muir_state_bytes(1, 0, 128, 128) == 0, "state bytes H = 0");
    printf("%d failures, %d launches\n", g_failures, stub_launches());
    return g_failures == 0 ? 0 : 1;
}
