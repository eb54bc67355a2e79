// Workspace sizes of every entry point, from the layouts in layout.hpp. Host code only: the
// library builds it with the kernels, and it also builds with a plain host compiler.
#include <stdint.h>

#include "kernels.hpp"
#include "layout.hpp"

namespace muir {

namespace {

template <int OB, int D, int C>
size_t slot_bytes() { return SlotLayout<OB, D, C>::BYTES; }

// Bytes of one (batch, head, chunk) slot of the chunk forward: bf16 or fp32 operands.
size_t slot_bytes_rt(bool bf16, int d, int chunk) {
#define MUIR_SLOT(D, C) \
    if (d == D && chunk == C) return bf16 ? slot_bytes<2, D, C>() : slot_bytes<4, D, C>();
    MUIR_SLOT(64, 64) MUIR_SLOT(64, 128) MUIR_SLOT(64, 256)
    MUIR_SLOT(128, 64) MUIR_SLOT(128, 128) MUIR_SLOT(128, 256)
#undef MUIR_SLOT
    return 0;
}

// The shared-erase form: the chunk forward's bf16 slot and its own per-chunk products.
template <int D, int C>
size_t wy_bytes() { return SlotLayout<2, D, C>::BYTES + XSlot<D, C>::BYTES; }

}  // namespace

size_t chunk_slots_bytes(int B, int T, int H, int d, int chunk, bool bf16) {
    const size_t slot = slot_bytes_rt(bf16, d, chunk);
    if (slot == 0 || B < 1 || H < 1 || T < 0) return 0;
    const size_t nchunks = (size_t(T) + chunk - 1) / chunk;
    const size_t n = size_t(B) * size_t(H) * nchunks;
    if (n != 0 && slot > SIZE_MAX / n) return 0;
    return n * slot;
}

size_t chunk_workspace_bytes(int B, int T, int H, int d, int chunk, bool bf16) {
    const size_t slots = chunk_slots_bytes(B, T, H, d, chunk, bf16);
    if (slots == 0 || !bf16 || !split_scan_applies(B, H, d)) return slots;
    // The split scan's readout region (bf16 only), after the slots (a multiple of 256 bytes).
    const size_t n = size_t(B) * size_t(H) * ((size_t(T) + chunk - 1) / chunk);
    const size_t per = readout_chunk_bytes(d, chunk);
    if (per > (SIZE_MAX - slots) / n) return 0;
    return slots + n * per;
}

size_t wy_workspace_bytes(int B, int T, int H, int d, int chunk) {
    size_t per = 0;
#define MUIR_WY(D, C) \
    if (d == D && chunk == C) per = wy_bytes<D, C>();
    MUIR_WY(64, 64) MUIR_WY(64, 128) MUIR_WY(64, 256)
    MUIR_WY(128, 64) MUIR_WY(128, 128) MUIR_WY(128, 256)
#undef MUIR_WY
    if (per == 0 || B < 1 || H < 1 || T < 0) return 0;
    const size_t nchunks = (size_t(T) + chunk - 1) / chunk;
    const size_t n = size_t(B) * size_t(H) * nchunks;
    if (n != 0 && per > SIZE_MAX / n) return 0;
    return n * per;
}

int bwd_fwd_chunk(int, int T, int, int) { return T >= 256 ? 128 : kBwdChunk; }

bool bwd_layout(int B, int T, int H, int d, bool bf16, BwdLayout &L) {
    constexpr int kC = kBwdChunk;
    const size_t fwd = chunk_slots_bytes(B, T, H, d, bwd_fwd_chunk(B, T, H, d), bf16);
    if (fwd == 0 && T > 0) return false;
    const size_t nc = (size_t(T) + kC - 1) / kC;
    const size_t BH = size_t(B) * H, tok = size_t(B) * T * H * d;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align256(bytes);
        return at;
    };
    L.fwd = take(fwd);
    L.u = take(tok * 4);
    L.states = take(BH * (nc + 1) * d * d * 4);
    L.kb = take(BH * nc * kC * d * 4);
    L.kg = take(BH * nc * kC * d * 4);
    L.qg = take(BH * nc * kC * d * 4);
    L.gC = take(BH * nc * d * 4);
    L.M = take(BH * nc * kC * kC * 4);
    L.P = take(BH * nc * kC * kC * 4);
    L.pred = take(tok * 4);
    L.dU = take(tok * 4);
    L.lamC = take(BH * nc * d * d * 4);
    L.drp = take(BH * nc * d * 4);
    L.total = off;
    return true;
}

size_t chunk_bwd_workspace_bytes(int B, int T, int H, int d, bool bf16) {
    if (B < 1 || H < 1 || T < 0 || (d != 64 && d != 128)) return 0;
    BwdLayout L;
    if (!bwd_layout(B, T, H, d, bf16, L)) return 0;
    return L.total;
}

}  // namespace muir
