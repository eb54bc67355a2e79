// Chunkwise forward of the gated delta rule with one erase strength per token, shared by
// every value channel.
//
// This is the plain gated delta rule's erase, the one GDN-2 and Muir generalise into
// decoupled per-channel erase gates (the Muir abstract, "Full text" on the Astral Feed
// page). Decay stays channel-wise; the write gate, the query gate and the matched-filter
// readout are unchanged. The token recurrence is the channel-wise one with e_{t,j} = e_t
// for every value column j.
//
// With a shared erase, the unit lower-triangular system of a chunk is one matrix for all
// value columns, so its inverse exists per chunk and the sequential part becomes dense
// products (the WY form of the delta rule):
//   T = (I + Diag(e) M)^-1                                   chunk-parallel
//   U = T (W*V - Diag(e) (K*gamma) S0)                       per chunk, all columns
//   O = (Qh*gamma) S0 + P U
//   S_C = Diag(gamma_C) S0 + (K*beta)^T U                    Horner form over leaf pairs
// M, P, K*gamma, Qh*gamma, (K*beta')^T and the pair decays come from the channel-wise
// path's prepare kernel, pivoted at block boundaries so that no cumulative decay is ever
// divided (the stable large-chunk scheme: liuch.name summary, third bullet; openai-hub
// news page, section on rewriting the long-sequence parallel algorithm). The inverse is
// the block recursion of that scheme, one 16-token row block at a time:
//   T_ii = (I + Diag(e_i) M_ii)^-1                    forward substitution, fp32
//   T_ij = -T_ii Diag(e_i) sum_{j<=k<i} M_ik T_kj     (j < i) on the matrix cores
// and it replaces M in the workspace.
#include "chunk_layout.hpp"
#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace muir {

namespace {

// LDS of the inverse kernel (bytes). Diagonal blocks are fp32 [16][TDS] (row pitch padded
// so the 16-lane groups of one wavefront hit different banks).
template <int C> struct InvLds {
    static constexpr int NB = C / 16, NP = NB / 2, TDS = 260;
    static constexpr size_t E_OFF = 0;                                     // [C] erase strengths
    static constexpr size_t MD_OFF = E_OFF + size_t(C) * 4;                // [NB][TDS] M_ii
    static constexpr size_t TD_OFF = MD_OFF + size_t(NB) * TDS * 4;        // [NB][TDS] T_ii
    static constexpr size_t TA_OFF = TD_OFF + size_t(NB) * TDS * 4;        // [NB][64] T_ii, A operand
    static constexpr size_t TB_OFF = TA_OFF + size_t(NB) * 64 * 8;         // [NP(NP+1)][64] B operand
    static constexpr size_t BYTES = TB_OFF + size_t(NP) * (NP + 1) * 64 * 16;
};

// Wavefronts of the inverse kernel: eight for 16 or more row blocks, else four.
template <int C> constexpr int inv_waves() { return C / 16 >= 16 ? 8 : 4; }

// One workgroup per (chunk, head, batch). T's blocks are kept in LDS as
// K = 32 operands whose rows are T's columns: slot (m, j) holds blocks (2m, j) and
// (2m + 1, j), lane (n, G) the elements [4G + r][n] of both. Slots exist for j <= 2m + 1;
// upper blocks stay zero. Row block i of T is computed from M's row block i (read from the
// workspace) against the slots of the rows above it; wavefront w takes the column blocks
// j = w (mod NW). A row's T blocks overwrite its M blocks in the workspace only after every
// wavefront has finished reading that row (one row later, past a barrier).
template <int D, int C>
__global__ __launch_bounds__(64 * inv_waves<C>()) void wy_inverse_kernel(const float *__restrict__ e,
                                                         unsigned char *__restrict__ ws, int T,
                                                         int H, int nchunks) {
    using SL = Slot<bf16_t, D, C>;
    using LY = InvLds<C>;
    using F = Frag<bf16_t>;
    using f4 = F::f4;
    using f8 = F::f8;
    constexpr int NB = C / 16, NP = NB / 2, TDS = LY::TDS, NW = inv_waves<C>();
    constexpr int NT = 64 * NW, NJ = (NB + NW - 1) / NW;

    extern __shared__ __align__(16) unsigned char smem[];
    float *sh_e = reinterpret_cast<float *>(smem + LY::E_OFF);
    float *sh_md = reinterpret_cast<float *>(smem + LY::MD_OFF);
    float *sh_td = reinterpret_cast<float *>(smem + LY::TD_OFF);
    f4 *sh_ta = reinterpret_cast<f4 *>(smem + LY::TA_OFF);
    f8 *sh_tb = reinterpret_cast<f8 *>(smem + LY::TB_OFF);
    auto tb = [&](int m, int j) { return sh_tb + (m * (m + 1) + j) * 64; };

    const int ci = blockIdx.x, hh = blockIdx.y, b = blockIdx.z;
    // The wavefront index is uniform: in a scalar register, offsets derived from it are too.
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, x = lane & 15, G = lane >> 4;
    unsigned char *slot = ws + ((size_t(b) * H + hh) * nchunks + ci) * SL::BYTES;
    bf16_t *gT = reinterpret_cast<bf16_t *>(slot + SL::M_OFF);
    const float *gMD = reinterpret_cast<const float *>(slot + SL::MD_OFF);
    const int t0 = ci * C, nreal = min(C, T - t0);

    // Erase strengths (0 past the sequence end: those rows of M are zero, T's are the
    // identity's), M's fp32 diagonal blocks, zeroed operand slots.
    for (int t = tid; t < C; t += NT) sh_e[t] = t < nreal ? e[(size_t(b) * T + t0 + t) * H + hh] : 0.f;
    for (int n = tid; n < NB * 64; n += NT) {
        const int i = n >> 6, q4 = n & 63;
        *reinterpret_cast<f32x4_t *>(sh_md + i * TDS + 4 * q4) =
            *reinterpret_cast<const f32x4_t *>(gMD + i * 256 + 4 * q4);
    }
    {
        const f8 z = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int n = tid; n < NP * (NP + 1) * 64; n += NT) sh_tb[n] = z;
    }
    lds_barrier();

    // T_ii, column c: x_t = [t == c] - e_t sum_{s<t} M_ii[t][s] x_s.
    for (int n = tid; n < NB * 16; n += NT) {
        const int i = n >> 4, c = n & 15;
        const float *md = sh_md + i * TDS;
        const float *ee = sh_e + 16 * i;
        float xv[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float acc = 0.f;
#pragma unroll
            for (int s = 0; s < t; ++s) acc += md[t * 16 + s] * xv[s];
            xv[t] = (t == c ? 1.f : 0.f) - ee[t] * acc;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) sh_td[i * TDS + t * 16 + c] = xv[t];
    }
    lds_barrier();

    // T_ii in bf16: rows (lane (x, G): T_ii[x][4G..4G+3]) as the A operand, columns
    // (lane (x, G): T_ii[4G..4G+3][x]) into its operand slot.
    for (int i = wave; i < NB; i += NW) {
        const float *td = sh_td + i * TDS;
        f32x4_t rowv, colv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            rowv[r] = td[x * 16 + 4 * G + r];
            colv[r] = td[(4 * G + r) * 16 + x];
        }
        sh_ta[i * 64 + lane] = F::pack(rowv);
        reinterpret_cast<f4 *>(tb(i >> 1, i) + lane)[i & 1] = F::pack(colv);
    }
    lds_barrier();

    f4 pend[NJ];  // this wavefront's blocks of the previous row, as rows (x, 4G..4G+3)
    auto flush = [&](int row) {
#pragma unroll
        for (int n = 0; n < NJ; ++n) {
            const int j = wave + NW * n;
            if (j < row) *reinterpret_cast<f4 *>(gT + SL::blk(row, j, 16 * x + 4 * G)) = pend[n];
        }
    };
    // M's pairs of row i that this wavefront uses (m >= wave / 2, 2m < i), loaded one row
    // ahead.
    const unsigned lo_pair = unsigned((4 * x + G) * 8);
    f8 mcur[NP], mnext[NP];
    auto load_row = [&](int i, f8 (&dst)[NP]) {
        const bf16_t *mrow = gT + size_t(SL::prow(i)) * 512 + lo_pair;
#pragma unroll
        for (int m = 0; m < NP; ++m)
            if (m >= (wave >> 1) && 2 * m < i) dst[m] = F::load8(mrow + size_t(m) * 512);
    };
    if (NB > 1) load_row(1, mnext);
    for (int i = 1; i < NB; ++i) {
        if (i > 1) flush(i - 1);
#pragma unroll
        for (int m = 0; m < NP; ++m) mcur[m] = mnext[m];
        if (i + 1 < NB) load_row(i + 1, mnext);
        const f4 ta = sh_ta[i * 64 + lane];
        const f32x4_t ev = *reinterpret_cast<const f32x4_t *>(sh_e + 16 * i + 4 * G);
#pragma unroll
        for (int n = 0; n < NJ; ++n) {
            const int j = wave + NW * n;
            if (j < i) {
                // X = sum over the pairs m holding blocks j .. i - 1 of M(i, pair m) T(pair m, j).
                // For odd i the last pair's second block is M_ii, stored as zero.
                f32x4_t X = zero4();
#pragma unroll
                for (int m = 0; m < NP; ++m)
                    if (m >= (j >> 1) && 2 * m < i) X = F::mma8(mcur[m], tb(m, j)[lane], X);
                const f4 xb = F::pack(X * ev);
                const f32x4_t y = F::mma16_fresh(ta, xb);   // lane (x, G): (T_ii X)[4G + r][x]
                const f32x4_t yt = F::mma16_fresh(xb, ta);  // lane (x, G): (T_ii X)[x][4G + r]
                reinterpret_cast<f4 *>(tb(i >> 1, j) + lane)[i & 1] = F::pack(-y);
                pend[n] = F::pack(-yt);
            }
        }
        lds_barrier();
    }
    if (NB > 1) flush(NB - 1);
    // Diagonal blocks last: for odd i the slot of T_ii is read above as M_ii (zero).
    for (int i = wave; i < NB; i += NW) {
        *reinterpret_cast<f4 *>(gT + SL::blk(i, i, 16 * x + 4 * G)) = sh_ta[i * 64 + lane];
        if ((i & 1) == 0) {
            const f4 z = {0, 0, 0, 0};
            *reinterpret_cast<f4 *>(gT + SL::blk(i, i + 1, 16 * x + 4 * G)) = z;
        }
    }
}

__device__ __forceinline__ float buf_load_bf16(rsrc_t r, unsigned voff, unsigned soff) {
    return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, int(voff), int(soff), 0));
}
__device__ __forceinline__ float buf_load_f(rsrc_t r, unsigned voff, unsigned soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, int(voff), int(soff), 0));
}
__device__ __forceinline__ void buf_store_bf16(rsrc_t r, unsigned voff, unsigned soff, float x) {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(x), r, int(voff), int(soff), 0);
}

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

// Token blocks (16 tokens) a wavefront of an NW-wavefront workgroup takes in the chunk-parallel
// kernels: blocks w and 2 NW - 1 - w when there are 2 NW of them (equal work under the
// triangular pair loops), else block w.
template <int NB, int NW> struct BlockDeal {
    static constexpr int NPW = NB >= 2 * NW ? NB / NW : 1;
    static __device__ __forceinline__ int block(int w, int k) {
        return NB >= 2 * NW ? 2 * NW * (k >> 1) + ((k & 1) ? 2 * NW - 1 - w : w) : w;
    }
    static __device__ __forceinline__ bool active(int w) { return w < NB; }
};

// LDS of the chunk-parallel precompute (bytes): two [C/32][D/16][64] operand-pair arrays, the
// pair decays and the erase strengths.
template <int D, int C> struct PreLds {
    static constexpr size_t B1_OFF = 0;
    static constexpr size_t B2_OFF = B1_OFF + size_t(C / 32) * (D / 16) * 64 * 16;
    static constexpr size_t PP_OFF = B2_OFF + size_t(C / 32) * (D / 16) * 64 * 16;
    static constexpr size_t E_OFF = PP_OFF + size_t(C / 32) * D * 4;
    static constexpr size_t BYTES = E_OFF + size_t(C) * 4;
};

// The chunk-parallel precompute, one workgroup of eight wavefronts per (chunk, head, batch),
// after the inverse. Three steps, separated by barriers:
//  1. the B operands of the two solves, e*(K*gamma) and w*v, in accumulator layout (rows =
//     tokens, 16 channels or value columns per tile): Kg and the row-layout w*v pass through a
//     K = 16 product against the identity; the pair decays and e go to LDS, gamma_C out;
//  2. W = T e*(K*gamma) and U~ = T (w*v) per token block, rounded to bf16 into LDS in place of
//     their operands (same layout: rows = tokens, so they are the next B operands);
//  3. A~^T and (K*beta)^T U~ by Horner over the leaf pairs (rows scaled by each pair's decay,
//     as in the channel-wise state carry), (P W)^T against Qh*gamma, and P U~.
template <int D, int C>
__global__ __launch_bounds__(512) void wy_precompute_kernel(
    const bf16_t *__restrict__ v, const float *__restrict__ e, const float *__restrict__ w,
    unsigned char *__restrict__ ws, int T, int H, int nchunks, int nslots) {
    using SL = Slot<bf16_t, D, C>;
    using XS = XSlot<D, C>;
    using LY = PreLds<D, C>;
    using F = Frag<bf16_t>;
    using f4 = F::f4;
    using f8 = F::f8;
    constexpr int NW = 8, NB = C / 16, NP = NB / 2, NCT = D / 16, NKD = D / 32;
    using BD = BlockDeal<NB, NW>;

    extern __shared__ __align__(16) unsigned char smem[];
    f8 *sh_b1 = reinterpret_cast<f8 *>(smem + LY::B1_OFF);  // [NP][NCT][64]: e*Kg, then W
    f8 *sh_b2 = reinterpret_cast<f8 *>(smem + LY::B2_OFF);  // [NP][NCT][64]: w*v, then U~
    float *sh_pp = reinterpret_cast<float *>(smem + LY::PP_OFF);  // [NP][D]
    float *sh_e = reinterpret_cast<float *>(smem + LY::E_OFF);    // [C]
    auto b1 = [&](int m, int c) { return sh_b1 + (m * NCT + c) * 64; };
    auto b2 = [&](int m, int c) { return sh_b2 + (m * NCT + c) * 64; };

    const int ci = blockIdx.x, hh = blockIdx.y, b = blockIdx.z;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int tid = threadIdx.x, lane = tid & 63, x = lane & 15, G = lane >> 4;
    const size_t sidx = (size_t(b) * H + hh) * nchunks + ci;
    const unsigned char *slot = ws + sidx * SL::BYTES;
    unsigned char *xslot = ws + size_t(nslots) * SL::BYTES + sidx * XS::BYTES;
    const bf16_t *gT = reinterpret_cast<const bf16_t *>(slot + SL::M_OFF);
    const bf16_t *gP = reinterpret_cast<const bf16_t *>(slot + SL::P_OFF);
    const bf16_t *gKg = reinterpret_cast<const bf16_t *>(slot + SL::KG_OFF);
    const bf16_t *gQg = reinterpret_cast<const bf16_t *>(slot + SL::QG_OFF);
    const bf16_t *gKbT = reinterpret_cast<const bf16_t *>(slot + SL::KBT_OFF);
    const float *gPP = reinterpret_cast<const float *>(slot + SL::PP_OFF);
    const int t0 = ci * C, nreal = min(C, T - t0);
    const size_t HD = size_t(H) * D;
    const unsigned lo_pair = unsigned((4 * x + G) * 8);
    const unsigned lo_frag = unsigned(lane * 8);
    auto pair = [&](const bf16_t *base, int bt, int m) {
        return F::load8(base + size_t(SL::prow(bt) + m) * 512 + lo_pair);
    };

    // ---- 1: operands in accumulator layout; pair decays, e and gamma_C ----
    for (int t = tid; t < C; t += 64 * NW) sh_e[t] = t < nreal ? e[(size_t(b) * T + t0 + t) * H + hh] : 0.f;
    for (int n = tid; n < NP * D; n += 64 * NW) sh_pp[n] = gPP[n];
    if (tid < D) {
        float gc = 1.f;
        for (int p = 0; p < NP; ++p) gc *= gPP[p * D + tid];
        reinterpret_cast<float *>(xslot + XS::GC_OFF)[tid] = gc;
    }
    {
        // w*v of token 16L + x, value columns 16c + 4G .. + 3 (row layout), tokens past the
        // end zero; then its transpose.
        const rsrc_t rv = make_rsrc(v + (size_t(b) * T + t0) * HD + size_t(hh) * D,
                                    unsigned((size_t(nreal - 1) * HD + D) * 2));
        const rsrc_t rw = make_rsrc(w + (size_t(b) * T + t0) * HD + size_t(hh) * D,
                                    unsigned((size_t(nreal - 1) * HD + D) * 4));
        const f4 unit = F::unit(x, G);
        for (int u = wave; u < NB * NCT; u += NW) {
            const int L = u / NCT, c = u % NCT;
            const unsigned off = unsigned(16 * L + x) * unsigned(HD) + unsigned(16 * c + 4 * G);
            const u16x4_t vv = Row4<bf16_t>::load(rv, off * 2u, 0u);
            const f32x4_t wv = buf_load_f4(rw, off * 4u, 0u);
            f32x4_t p;
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = wv[r] * bf16_to_f32(vv[r]);
            reinterpret_cast<f4 *>(b2(L >> 1, c) + lane)[L & 1] = F::pack(F::mma16_fresh(F::pack(p), unit));
        }
        // e * (K*gamma): one fragment gives both 16-channel halves of a channel group.
        for (int u = wave; u < NB * NKD; u += NW) {
            const int L = u / NKD, kk = u % NKD;
            const f8 kg = F::load8(gKg + frag_idx(16 * L, 32 * kk, D) + lo_frag);
            const f32x4_t ev = *reinterpret_cast<const f32x4_t *>(sh_e + 16 * L + 4 * G);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const f32x4_t t = F::mma16_fresh(hf ? F::hi(kg) : F::lo(kg), unit);
                reinterpret_cast<f4 *>(b1(L >> 1, 2 * kk + hf) + lane)[L & 1] = F::pack(t * ev);
            }
        }
    }
    lds_barrier();

    // ---- 2: W = T e*Kg and U~ = T w*v per token block ----
    {
        f32x4_t aw[BD::NPW][NCT], au[BD::NPW][NCT];
#pragma unroll
        for (int k = 0; k < BD::NPW; ++k)
#pragma unroll
            for (int c = 0; c < NCT; ++c) aw[k][c] = au[k][c] = zero4();
        if (BD::active(wave)) {
#pragma unroll
            for (int k = 0; k < BD::NPW; ++k) {
                const int i = BD::block(wave, k);
                for (int m = 0; m <= i / 2; ++m) {
                    const f8 tp = pair(gT, i, m);
#pragma unroll
                    for (int c = 0; c < NCT; ++c) {
                        aw[k][c] = F::mma8(tp, b1(m, c)[lane], aw[k][c]);
                        au[k][c] = F::mma8(tp, b2(m, c)[lane], au[k][c]);
                    }
                }
            }
        }
        lds_barrier();
        if (BD::active(wave)) {
#pragma unroll
            for (int k = 0; k < BD::NPW; ++k) {
                const int i = BD::block(wave, k);
#pragma unroll
                for (int c = 0; c < NCT; ++c) {
                    reinterpret_cast<f4 *>(b1(i >> 1, c) + lane)[i & 1] = F::pack(aw[k][c]);
                    reinterpret_cast<f4 *>(b2(i >> 1, c) + lane)[i & 1] = F::pack(au[k][c]);
                }
            }
        }
    }
    lds_barrier();

    // ---- 3a: A~ and (K*beta)^T U~, wavefront w for channel tile c = w ----
    if (wave < NCT) {
        const int c = wave;
        f32x4_t at[NCT], bc[NCT];
#pragma unroll
        for (int j = 0; j < NCT; ++j) at[j] = bc[j] = zero4();
        for (int p = 0; p < NP; ++p) {
            const f8 kb = F::load8(gKbT + frag_idx(16 * c, 32 * p, C) + lo_frag);
            const float pcol = sh_pp[p * D + 16 * c + x];  // A~^T: column = channel 16c + x
            const f32x4_t prow = *reinterpret_cast<const f32x4_t *>(sh_pp + p * D + 16 * c + 4 * G);
#pragma unroll
            for (int j = 0; j < NCT; ++j) {
                at[j] = F::mma8(b1(p, j)[lane], kb, at[j] * pcol);  // rows j (W), columns i
                bc[j] = F::mma8(kb, b2(p, j)[lane], bc[j] * prow);  // rows i, columns value j
            }
        }
        bf16_t *gAT = reinterpret_cast<bf16_t *>(xslot + XS::AT_OFF);
        float *gBC = reinterpret_cast<float *>(xslot + XS::BC_OFF);
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk)
            *reinterpret_cast<f8 *>(gAT + ((c * NKD + kk) * 64 + lane) * 8) =
                F::cat(F::pack(at[2 * kk]), F::pack(at[2 * kk + 1]));
#pragma unroll
        for (int j = 0; j < NCT; ++j) *reinterpret_cast<f32x4_t *>(gBC + ((c * NCT + j) * 64 + lane) * 4) = bc[j];
    }

    // ---- 3b: Q~ = Qh*gamma - P W and O~ = P U~ per token block ----
    if (BD::active(wave)) {
        bf16_t *gQT = reinterpret_cast<bf16_t *>(xslot + XS::QT_OFF);
        bf16_t *gOT = reinterpret_cast<bf16_t *>(xslot + XS::OT_OFF);
#pragma unroll
        for (int k = 0; k < BD::NPW; ++k) {
            const int i = BD::block(wave, k);
            f32x4_t pw[NCT], ou[NCT];
#pragma unroll
            for (int j = 0; j < NCT; ++j) pw[j] = ou[j] = zero4();
            for (int m = 0; m <= i / 2; ++m) {
                const f8 pp = pair(gP, i, m);
#pragma unroll
                for (int j = 0; j < NCT; ++j) {
                    pw[j] = F::mma8(b1(m, j)[lane], pp, pw[j]);  // (P W)^T: lane (t, G) row t
                    ou[j] = F::mma8(pp, b2(m, j)[lane], ou[j]);  // P U~: accumulator layout
                }
            }
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) {
                const size_t fo = frag_idx(16 * i, 32 * kk, D) + lo_frag;
                const f8 qg = F::load8(gQg + fo);
                f32x4_t lo, hi;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    lo[r] = bf16_to_f32(qg[r]) - pw[2 * kk][r];
                    hi[r] = bf16_to_f32(qg[4 + r]) - pw[2 * kk + 1][r];
                }
                *reinterpret_cast<f8 *>(gQT + fo) = F::cat(F::pack(lo), F::pack(hi));
            }
#pragma unroll
            for (int j = 0; j < NCT; ++j) *reinterpret_cast<f4 *>(gOT + ((i * NCT + j) * 64 + lane) * 4) = F::pack(ou[j]);
        }
    }
}

// The state scan: one workgroup of D/32 wavefronts per (batch x head, 16 value columns),
// sequential over chunks: S <- Diag(gamma_C) S - A~ S + BC, leaving each chunk's start state
// (as the readout's B operand) in the workspace. Wavefront w owns channels 32w .. 32w + 31
// (two 16-channel tiles); the state's bf16 copy for the product goes through LDS. Each
// chunk's operands (A~ rows, BC, gamma_C) are loaded four chunks ahead.
template <int D, int C>
__global__ __launch_bounds__(2 * D) void wy_state_kernel(const float *__restrict__ s0,
                                                         float *__restrict__ s_out,
                                                         unsigned char *__restrict__ ws, int H,
                                                         int BH, int nchunks, int nslots) {
    using XS = XSlot<D, C>;
    using F = Frag<bf16_t>;
    using f8 = F::f8;
    constexpr int NCT = D / 16, NKD = D / 32;
    constexpr unsigned OB = 2;
    __shared__ f8 sh_S[NKD][64];

    const int id = blockIdx.x;
    const int bh = (id >> 3) / NCT * 8 + (id & 7);
    const int vt = (id >> 3) % NCT;
    if (bh >= BH) return;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63, x = lane & 15, G = lane >> 4;
    const int j0 = 16 * vt;

    f32x4_t S[2];
    const float *s0h = s0 ? s0 + size_t(bh) * D * D + j0 : nullptr;
    float *south = s_out ? s_out + size_t(bh) * D * D + j0 : nullptr;
    auto sidx = [&](int hs, int r) { return size_t(32 * wave + 16 * hs + 4 * G + r) * D + x; };
#pragma unroll
    for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[hs][r] = s0h ? s0h[sidx(hs, r)] : 0.f;

    unsigned char *xbase = ws + size_t(nslots) * Slot<bf16_t, D, C>::BYTES + size_t(bh) * nchunks * XS::BYTES;
    const rsrc_t rx = make_rsrc(xbase, unsigned(size_t(nchunks) * XS::BYTES));
    auto xoff = [&](int ci, size_t off) { return unsigned(size_t(min(ci, nchunks - 1)) * XS::BYTES + off); };
    struct Ops {
        f8 at[2][NKD];
        f32x4_t bc[2], gc[2];
    };
    auto load = [&](int ci, Ops &op) {
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            const int c = 2 * wave + hs;
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk)
                op.at[hs][kk] = F::bload8(rx, unsigned(lane * 8) * OB, xoff(ci, XS::AT_OFF + size_t((c * NKD + kk) * 64) * 8 * OB));
            op.bc[hs] = buf_load_f4(rx, unsigned(lane * 16), xoff(ci, XS::BC_OFF + size_t((c * NCT + vt) * 64) * 16));
            op.gc[hs] = buf_load_f4(rx, unsigned(16 * c + 4 * G) * 4u, xoff(ci, XS::GC_OFF));
        }
    };
    auto step = [&](int ci, Ops &op) {
        const f8 mine = F::cat(F::pack(S[0]), F::pack(S[1]));
        sh_S[wave][lane] = mine;
        // The chunk's start state for the readout: [value tile][channel group][64][8].
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, mine), rx, int(lane * 16),
                                               int(xoff(ci, XS::SC_OFF + size_t((vt * NKD + wave) * 64) * 16)), 0);
        lds_barrier();
        f8 sb[NKD];
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk) sb[kk] = sh_S[kk][lane];
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            f32x4_t acc = zero4();
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) acc = F::mma8(op.at[hs][kk], sb[kk], acc);
            S[hs] = S[hs] * op.gc[hs] - acc + op.bc[hs];
        }
        load(ci + 4, op);  // this buffer's next chunk
        lds_barrier();
    };
    // Four operand buffers, for the chunks of each residue mod 4 (four chunks per iteration
    // keep every register index static).
    Ops op0, op1, op2, op3;
    if (nchunks > 0) {
        load(0, op0);
        load(1, op1);
        load(2, op2);
        load(3, op3);
    }
    for (int ci = 0; ci < nchunks; ci += 4) {
        step(ci, op0);
        if (ci + 1 < nchunks) step(ci + 1, op1);
        if (ci + 2 < nchunks) step(ci + 2, op2);
        if (ci + 3 < nchunks) step(ci + 3, op3);
    }
#pragma unroll
    for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (south) south[sidx(hs, r)] = S[hs][r];
}

// The readout, chunk-parallel: O = Q~ S + O~ per token block and value tile, one workgroup
// of eight wavefronts per (chunk, head, batch).
template <int D, int C>
__global__ __launch_bounds__(512) void wy_output_kernel(bf16_t *__restrict__ o,
                                                        const unsigned char *__restrict__ ws,
                                                        int T, int H, int nchunks, int nslots) {
    using XS = XSlot<D, C>;
    using F = Frag<bf16_t>;
    using f4 = F::f4;
    using f8 = F::f8;
    constexpr int NW = 8, NB = C / 16, NCT = D / 16, NKD = D / 32;
    using BD = BlockDeal<NB, NW>;

    const int ci = blockIdx.x, hh = blockIdx.y, b = blockIdx.z;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63, x = lane & 15, G = lane >> 4;
    if (!BD::active(wave)) return;
    const size_t sidx = (size_t(b) * H + hh) * nchunks + ci;
    const unsigned char *xslot = ws + size_t(nslots) * Slot<bf16_t, D, C>::BYTES + sidx * XS::BYTES;
    const bf16_t *gQT = reinterpret_cast<const bf16_t *>(xslot + XS::QT_OFF);
    const bf16_t *gOT = reinterpret_cast<const bf16_t *>(xslot + XS::OT_OFF);
    const bf16_t *gSC = reinterpret_cast<const bf16_t *>(xslot + XS::SC_OFF);
    const size_t HD = size_t(H) * D;
    const int t0 = ci * C;
    // o of this head from token t0; tokens at or past T fall outside and are dropped.
    const rsrc_t ro = make_rsrc(o + (size_t(b) * T + t0) * HD + size_t(hh) * D,
                                unsigned((size_t(T - t0 - 1) * HD + D) * 2));

    f8 qt[BD::NPW][NKD];
#pragma unroll
    for (int k = 0; k < BD::NPW; ++k)
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk)
            qt[k][kk] = F::load8(gQT + frag_idx(16 * BD::block(wave, k), 32 * kk, D) + lane * 8);
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
        f8 sc[NKD];
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk) sc[kk] = F::load8(gSC + ((j * NKD + kk) * 64 + lane) * 8);
#pragma unroll
        for (int k = 0; k < BD::NPW; ++k) {
            const int i = BD::block(wave, k);
            const f4 ot = F::load4(gOT + ((i * NCT + j) * 64 + lane) * 4);
            f32x4_t acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = bf16_to_f32(ot[r]);
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) acc = F::mma8(qt[k][kk], sc[kk], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                buf_store_bf16(ro, (unsigned(16 * i + 4 * G + r) * unsigned(HD) + unsigned(16 * j + x)) * 2u, 0u, acc[r]);
        }
    }
}

template <int D, int C>
size_t wy_bytes() { return Slot<bf16_t, D, C>::BYTES + XSlot<D, C>::BYTES; }

template <int D, int C>
hipError_t solve_typed(const void *v, const float *e, const float *w, int B, int T, int H,
                       void *workspace, hipStream_t stream) {
    const int nchunks = (T + C - 1) / C;
    if (nchunks == 0) return hipSuccess;
    {
        using LY = InvLds<C>;
        auto kern = wy_inverse_kernel<D, C>;
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(LY::BYTES));
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(kern, dim3(nchunks, H, B), dim3(64 * inv_waves<C>()), LY::BYTES, stream, e,
                           static_cast<unsigned char *>(workspace), T, H, nchunks);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    using LY = PreLds<D, C>;
    auto kern = wy_precompute_kernel<D, C>;
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(LY::BYTES));
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(nchunks, H, B), dim3(512), LY::BYTES, stream,
                       static_cast<const bf16_t *>(v), e, w, static_cast<unsigned char *>(workspace),
                       T, H, nchunks, B * H * nchunks);
    return hipGetLastError();
}

template <int D, int C>
hipError_t wy_scan_typed(const float *s0, void *o, float *s_out, int B, int T, int H,
                         void *workspace, hipStream_t stream) {
    const int nchunks = (T + C - 1) / C;
    const int BH = B * H;
    const int groups = (BH + 7) / 8;
    hipLaunchKernelGGL((wy_state_kernel<D, C>), dim3(groups * 8 * (D / 16)), dim3(2 * D), 0, stream,
                       s0, s_out, static_cast<unsigned char *>(workspace), H, BH, nchunks, BH * nchunks);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || nchunks == 0) return err;
    hipLaunchKernelGGL((wy_output_kernel<D, C>), dim3(nchunks, H, B), dim3(512), 0, stream,
                       static_cast<bf16_t *>(o), static_cast<const unsigned char *>(workspace), T, H,
                       nchunks, BH * nchunks);
    return hipGetLastError();
}

}  // namespace

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

hipError_t launch_wy_solve(const void *v, const float *e, const float *w, int B, int T, int H,
                           int d, int chunk, void *workspace, hipStream_t stream) {
#define MUIR_WY(D, C) \
    if (d == D && chunk == C) return solve_typed<D, C>(v, e, w, B, T, H, workspace, stream);
    MUIR_WY(64, 64) MUIR_WY(64, 128) MUIR_WY(64, 256)
    MUIR_WY(128, 64) MUIR_WY(128, 128) MUIR_WY(128, 256)
#undef MUIR_WY
    return hipErrorInvalidValue;
}

hipError_t launch_wy_scan(const float *s0, void *o, float *s_out, int B, int T, int H, int d,
                          int chunk, void *workspace, hipStream_t stream) {
#define MUIR_WY(D, C) \
    if (d == D && chunk == C) return wy_scan_typed<D, C>(s0, o, s_out, B, T, H, workspace, stream);
    MUIR_WY(64, 64) MUIR_WY(64, 128) MUIR_WY(64, 256)
    MUIR_WY(128, 64) MUIR_WY(128, 128) MUIR_WY(128, 256)
#undef MUIR_WY
    return hipErrorInvalidValue;
}

}  // namespace muir
