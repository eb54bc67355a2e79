// Workspace layouts of the chunk kernels: constexpr offset arithmetic only, shared by the
// kernels and by the host-side size queries (sizes.cpp), so that both the device compiler and
// a plain host C++ compiler take it.
#pragma once

#include <stddef.h>

namespace muir {

constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace slot of one (batch, head, chunk). M and P blocks are 16x16 row-major
// (row = later token t, column = earlier token s), lower-triangular block order; the
// diagonal blocks of M are kept apart in fp32 (MD) for the leaf solve, and M's own slots
// for them hold zeros.
//
// The matrix-core operands are stored in the order the scan consumes them. Within every
// group of 32 positions, position 8g + 4h + i holds index 16h + 4g + i of the group
// (g < 4, h < 2, i < 4): lane group g then finds, in one 8-element load, the indices
// 4g..4g+3 of both 16-halves. Kg and Qg ([C][D]) are permuted along channels, KbT
// ([D][C]) along tokens.
template <int OB, int D, int C> struct SlotLayout {
    static constexpr int NB = C / 16;
    static constexpr int NPAIR = (NB / 2) * (NB / 2 + 1);  // block-pair slots of M (and of P)
    static constexpr size_t M_BYTES = size_t(NPAIR) * 512 * size_t(OB);
    static constexpr size_t M_OFF = 0;
    static constexpr size_t PP_OFF = align256(M_OFF + M_BYTES);       // pair decays [NB/2][D]
    static constexpr size_t P_OFF = align256(PP_OFF + size_t(NB / 2) * D * 4);
    static constexpr size_t KG_OFF = align256(P_OFF + M_BYTES);
    static constexpr size_t QG_OFF = align256(KG_OFF + size_t(C) * D * size_t(OB));
    static constexpr size_t KBT_OFF = align256(QG_OFF + size_t(C) * D * size_t(OB));
    static constexpr size_t MD_OFF = align256(KBT_OFF + size_t(C) * D * size_t(OB));
    static constexpr size_t BYTES = align256(MD_OFF + size_t(NB) * 256 * 4);
    // First block-pair slot of block row bt; the row has bt / 2 + 1 of them.
    static constexpr int prow(int bt) {
        return (bt >> 1) * ((bt >> 1) + 1) + (bt & 1) * ((bt >> 1) + 1);
    }
    // Element w = 16 t + s of block (bt, bs). Blocks 2j and 2j + 1 of a row share one
    // slot, interleaved four elements at a time, so that one 8-element load gives a lane
    // the same four elements of both (the two halves of a K = 32 operand).
    static constexpr size_t blk(int bt, int bs, int w) {
        return size_t(prow(bt) + (bs >> 1)) * 512 + ((w >> 2) * 2 + (bs & 1)) * 4 + (w & 3);
    }
};

// The split scan (bf16 operands, at most one 8-column scan workgroup per compute unit, so
// B * H * d / 8 <= 256) leaves the readout to a kernel of its own. It hands over, in a region
// after the slots, per (batch, head, chunk) and per 16-column value tile:
//   S0: the chunk's start state as d/32 K = 32 operand fragments (rows = the tile's value
//       columns, contraction = channels), [d/32][64 lanes][8] bf16;
//   U:  the chunk's solved values as C/32 leaf-pair fragments (rows = value columns,
//       contraction = the pair's 32 tokens), [C/32][64 lanes][8] bf16.
// Fragment lane 16 G + x holds row x: value column 2 (x / 4) + (x % 4) of the tile's first
// eight for x % 4 < 2, column 8 + 2 (x / 4) + (x % 4 - 2) for x % 4 >= 2 (the two 8-column scan
// tiles of a 16-column tile each fill half of the rows).
constexpr bool split_scan_applies(int B, int H, int d) { return size_t(B) * H * (d / 8) <= 256; }
constexpr size_t readout_tile_bytes(int d, int chunk) { return size_t(d / 32 + chunk / 32) * 1024; }
constexpr size_t readout_chunk_bytes(int d, int chunk) { return size_t(d / 16) * readout_tile_bytes(d, chunk); }

// Per (batch, head, chunk) products of the shared-erase form, kept in a workspace region
// after the prepare kernel's slots (same (b, h, chunk) order). With W = T Diag(e) (K*gamma)
// and U~ = T (w*v) (never stored):
//   AT: A~ = (K*beta)^T W as the state scan's A operand (rows = channels i, positions =
//       channels j in the 32-group order), [D/16][D/32][64 lanes][8] bf16
//   BC: (K*beta)^T U~ in accumulator layout per (channel tile, value tile), [D/16][D/16][64][4] fp32
//   GC: gamma_C, the chunk's whole decay per channel, [D] fp32
//   QT: Q~ = (Qh*gamma) - P W, A operand like Qg (rows = tokens), [C/16][D/32][64][8] bf16
//   OT: O~ = P U~ in accumulator layout per (leaf, value tile), [C/16][D/16][64][4] bf16
//   SC: the chunk's start state as B operand per (value tile, channel group), [D/16][D/32][64][8] bf16
// so that for a chunk with start state S:  S_next = Diag(gamma_C) S - A~ S + BC  and
// O = Q~ S + O~.
template <int D, int C> struct XSlot {
    static constexpr size_t AT_OFF = 0;
    static constexpr size_t BC_OFF = AT_OFF + size_t(D) * D * 2;
    static constexpr size_t GC_OFF = BC_OFF + size_t(D) * D * 4;
    static constexpr size_t QT_OFF = align256(GC_OFF + size_t(D) * 4);
    static constexpr size_t OT_OFF = QT_OFF + size_t(C) * D * 2;
    static constexpr size_t SC_OFF = OT_OFF + size_t(C) * D * 2;
    static constexpr size_t BYTES = align256(SC_OFF + size_t(D) * D * 2);
};

// The backward pass runs 64-token chunks. Its workspace: the forward's, then fp32 and
// operand-precision regions, each 256-byte aligned.
constexpr int kBwdChunk = 64;
struct BwdLayout {
    size_t fwd, u, states, kb, kg, qg, gC, M, P, pred, dU, lamC, drp, total;
};
// Offsets of the backward workspace for these sizes; false when the forward's workspace size
// is invalid.
bool bwd_layout(int B, int T, int H, int d, bool bf16, BwdLayout &L);
// Chunk size of the forward that the backward pass reruns (it saves the state every 64
// tokens whatever its own chunk size).
int bwd_fwd_chunk(int B, int T, int H, int d);

}  // namespace muir
