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

// One workgroup of four wavefronts per (chunk, head, batch). T's blocks are kept in LDS as
// K = 32 operands whose rows are T's columns: slot (m, j) holds blocks (2m, j) and
// (2m + 1, j), lane (n, G) the elements [4G + r][n] of both. Slots exist for j <= 2m + 1;
// upper blocks stay zero. Row block i of T is computed from M's row block i (read from the
// workspace) against the slots of the rows above it; wavefront w takes the column blocks
// j = w (mod 4). A row's T blocks overwrite its M blocks in the workspace only after every
// wavefront has finished reading that row (one row later, past a barrier).
template <int D, int C>
__global__ __launch_bounds__(256) void wy_inverse_kernel(const float *__restrict__ e,
                                                         unsigned char *__restrict__ ws, int T,
                                                         int H, int nchunks) {
    using SL = Slot<bf16_t, D, C>;
    using LY = InvLds<C>;
    using F = Frag<bf16_t>;
    using f4 = F::f4;
    using f8 = F::f8;
    constexpr int NB = C / 16, NP = NB / 2, TDS = LY::TDS, NJ = NB / 4;

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
    for (int t = tid; t < C; t += 256) sh_e[t] = t < nreal ? e[(size_t(b) * T + t0 + t) * H + hh] : 0.f;
    for (int n = tid; n < NB * 64; n += 256) {
        const int i = n >> 6, q4 = n & 63;
        *reinterpret_cast<f32x4_t *>(sh_md + i * TDS + 4 * q4) =
            *reinterpret_cast<const f32x4_t *>(gMD + i * 256 + 4 * q4);
    }
    {
        const f8 z = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int n = tid; n < NP * (NP + 1) * 64; n += 256) sh_tb[n] = z;
    }
    lds_barrier();

    // T_ii, column c: x_t = [t == c] - e_t sum_{s<t} M_ii[t][s] x_s.
    for (int n = tid; n < NB * 16; n += 256) {
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
    for (int i = wave; i < NB; i += 4) {
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
            const int j = wave + 4 * n;
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
            const int j = wave + 4 * n;
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
    for (int i = wave; i < NB; i += 4) {
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

// Wavefronts of the scan workgroup and the leaves each one takes: leaf k of wavefront w is
// 2 NW (k / 2) + w for even k and 2 NW (k / 2) + 2 NW - 1 - w for odd k, so that every
// wavefront needs the same number of pair products.
template <int C> struct ScanWaves {
    static constexpr int NB = C / 16;
    static constexpr int NW = NB >= 16 ? 8 : 4;
    static constexpr int NL = NB / NW;  // leaves per wavefront
    static __device__ __forceinline__ int leaf(int w, int k) {
        return 2 * NW * (k >> 1) + ((k & 1) ? 2 * NW - 1 - w : w);
    }
    // Pair slots that leaf k of any wavefront can have.
    static constexpr int npairs(int k) { return (2 * NW * (k >> 1) + ((k & 1) ? 2 * NW - 1 : NW - 1)) / 2 + 1; }
};

// The scan: one workgroup per (batch x head, 16 value columns), sequential over chunks.
// Every product has the tokens or the state's channels as rows and the 16 value columns
// as columns, so R, U and the state stay in accumulator layout (lane (x, G): rows
// 4G..4G+3 of column x) and are directly the B operands of the next products: no
// transposes. Per chunk, three phases separated by barriers:
//   1. for its leaves L: H = (K*gamma)_L S0 and (Qh*gamma)_L S0; R_L = w*v - e*H -> LDS
//   2. U_L = sum_{m <= L/2} T(L, pair m) R(pair m) -> LDS
//   3. O_L = (Qh*gamma)_L S0 + sum_m P(L, pair m) U(pair m) -> o; the state's owner
//      wavefronts carry it through the leaf pairs and leave its bf16 copy in LDS.
// The operands of each phase are loaded into registers one phase ahead (those of phase 1
// during the previous chunk's phase 3), so a chunk waits on memory about once rather
// than at every product.
template <int D, int C>
__global__ __launch_bounds__(64 * ScanWaves<C>::NW) void wy_scan_kernel(
    const bf16_t *__restrict__ v, const float *__restrict__ e, const float *__restrict__ w,
    const float *__restrict__ s0, bf16_t *__restrict__ o, float *__restrict__ s_out,
    const unsigned char *__restrict__ ws, int T, int H, int BH, int nchunks) {
    using SL = Slot<bf16_t, D, C>;
    using SW = ScanWaves<C>;
    using F = Frag<bf16_t>;
    using f4 = F::f4;
    using f8 = F::f8;
    constexpr int NB = C / 16, NP = NB / 2, NCT = D / 16, NKD = D / 32;
    constexpr int NW = SW::NW, NL = SW::NL;
    constexpr int TPW = NCT >= NW ? NCT / NW : 1;  // state tiles per owner wavefront
    constexpr int MPX = NP;                        // pair slots per leaf (upper bound)
    constexpr unsigned OB = 2;

    __shared__ f8 sh_S[NKD][64];  // state as B operand: channels 32kk + {4G.., 16 + 4G..}
    __shared__ f8 sh_R[NP][64];   // right-hand sides, leaves 2m and 2m + 1 of a lane
    __shared__ f8 sh_U[NP][64];   // solutions, likewise
    __shared__ f32x4_t sh_pp[NP * D / 4];  // pair decays of the chunk, [NP][D]

    // Value tiles of one head get ids equal mod 8: the same XCD and L2.
    const int id = blockIdx.x;
    const int bh = (id >> 3) / NCT * 8 + (id & 7);
    const int ct = (id >> 3) % NCT;
    if (bh >= BH) return;
    const int b = bh / H, h = bh % H, j0 = 16 * ct;
    // The wavefront index is uniform: in a scalar register, the buffer offsets derived from
    // it (leaf and pair slots) are scalar too.
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63, x = lane & 15, G = lane >> 4;
    const bool owner = wave * TPW < NCT;
    const size_t HD = size_t(H) * D;

    // State tile c = wave * TPW + tt: element (channel 16c + 4G + r, column j0 + x).
    f32x4_t S[TPW];
    const float *s0h = s0 ? s0 + size_t(bh) * D * D + j0 : nullptr;
    float *south = s_out ? s_out + size_t(bh) * D * D + j0 : nullptr;
    auto sidx = [&](int tt, int r) { return size_t(16 * (wave * TPW + tt) + 4 * G + r) * D + x; };
    auto put_state = [&]() {
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int c = wave * TPW + tt;
            reinterpret_cast<f4 *>(&sh_S[c >> 1][lane])[c & 1] = F::pack(S[tt]);
        }
    };
    if (owner) {
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) S[tt][r] = s0h ? s0h[sidx(tt, r)] : 0.f;
        put_state();
    }
    lds_barrier();

    // Workspace and token descriptors as in the channel-wise scan: tokens at or past T
    // read zero and their stores are dropped.
    const rsrc_t rws = make_rsrc(ws + size_t(bh) * nchunks * SL::BYTES, unsigned(size_t(nchunks) * SL::BYTES));
    auto wsoff = [&](int ci, size_t off) { return unsigned(size_t(ci) * SL::BYTES + off); };
    const size_t tok0 = size_t(b) * T * HD + size_t(h) * D + j0;
    const unsigned tok_elems = unsigned(size_t(T) * HD - size_t(h) * D - j0);
    const rsrc_t rv = make_rsrc(v + tok0, tok_elems * 2u);
    const rsrc_t rw = make_rsrc(w + tok0, tok_elems * 4u);
    const rsrc_t ro = make_rsrc(o + tok0, tok_elems * 2u);
    const rsrc_t re = make_rsrc(e + size_t(b) * T * H + h, unsigned((size_t(T) * H - h) * 4));
    // Per-lane element offset of token t, column j0 + x (the token depends on the lane, so
    // it goes into the vector offset; t is clamped to T, which lies outside the range).
    auto tok = [&](int t) { return unsigned(min(t, T)) * unsigned(HD) + unsigned(x); };
    const unsigned lo_pair = unsigned((4 * x + G) * 8) * OB;
    const unsigned lo_frag = unsigned(lane * 8) * OB;
    int Ls[NL];
#pragma unroll
    for (int k = 0; k < NL; ++k) Ls[k] = SW::leaf(wave, k);
    // Pair slots a leaf k can have (the loops below run to this bound, guarded by m <= L/2).
    auto npk = [](int k) { return SW::npairs(k); };

    struct Ops1 {
        f8 kg[NL][NKD], qg[NL][NKD];
        float vv[NL][4], wv[NL][4], ev[NL][4];
    };
    struct Ops2 {
        f8 tp[NL][MPX];
    };
    struct Ops3 {
        f32x4_t pd;  // this thread's share of the pair decays, staged through LDS
        f8 pp[NL][MPX];
        f8 kb[TPW][NP];
    };
    constexpr int PP4 = NP * D / 4;
    static_assert(PP4 <= 64 * NW, "one pair-decay vector per thread");
    auto load1 = [&](int ci, Ops1 &op) {
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int L = Ls[k];
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) {
                const size_t fo = frag_idx(16 * L, 32 * kk, D) * OB;
                op.kg[k][kk] = F::bload8(rws, lo_frag, wsoff(ci, SL::KG_OFF + fo));
                op.qg[k][kk] = F::bload8(rws, lo_frag, wsoff(ci, SL::QG_OFF + fo));
            }
            const int tb = ci * C + 16 * L + 4 * G;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                op.vv[k][r] = buf_load_bf16(rv, tok(tb + r) * 2u, 0u);
                op.wv[k][r] = buf_load_f(rw, tok(tb + r) * 4u, 0u);
                op.ev[k][r] = buf_load_f(re, unsigned(min(tb + r, T)) * unsigned(H) * 4u, 0u);
            }
        }
    };
    auto load2 = [&](int ci, Ops2 &op) {
#pragma unroll
        for (int k = 0; k < NL; ++k)
#pragma unroll
            for (int m = 0; m < npk(k); ++m)
                if (m <= Ls[k] / 2)
                    op.tp[k][m] = F::bload8(rws, lo_pair, wsoff(ci, SL::M_OFF + size_t(SL::prow(Ls[k]) + m) * 512 * OB));
    };
    auto load3 = [&](int ci, Ops3 &op) {
        if (int(threadIdx.x) < PP4) op.pd = buf_load_f4(rws, threadIdx.x * 16u, wsoff(ci, SL::PP_OFF));
#pragma unroll
        for (int k = 0; k < NL; ++k)
#pragma unroll
            for (int m = 0; m < npk(k); ++m)
                if (m <= Ls[k] / 2)
                    op.pp[k][m] = F::bload8(rws, lo_pair, wsoff(ci, SL::P_OFF + size_t(SL::prow(Ls[k]) + m) * 512 * OB));
        if (owner) {
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                const int c = wave * TPW + tt;
#pragma unroll
                for (int p = 0; p < NP; ++p)
                    op.kb[tt][p] = F::bload8(rws, lo_frag, wsoff(ci, SL::KBT_OFF + frag_idx(16 * c, 32 * p, C) * OB));
            }
        }
    };

    Ops1 o1;
    Ops2 o2;
    Ops3 o3;
    load1(0, o1);
    for (int ci = 0; ci < nchunks; ++ci) {
        // ---- phase 1: H and the S0 part of the readout; right-hand sides ----
        load2(ci, o2);
        f32x4_t QS[NL];
        {
            f8 sb[NKD];
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) sb[kk] = sh_S[kk][lane];
#pragma unroll
            for (int k = 0; k < NL; ++k) {
                f32x4_t Hc = zero4(), Qc = zero4();
#pragma unroll
                for (int kk = 0; kk < NKD; ++kk) {
                    Hc = F::mma8(o1.kg[k][kk], sb[kk], Hc);
                    Qc = F::mma8(o1.qg[k][kk], sb[kk], Qc);
                }
                QS[k] = Qc;
                f32x4_t R;
#pragma unroll
                for (int r = 0; r < 4; ++r) R[r] = o1.wv[k][r] * o1.vv[k][r] - o1.ev[k][r] * Hc[r];
                const int L = Ls[k];
                reinterpret_cast<f4 *>(&sh_R[L >> 1][lane])[L & 1] = F::pack(R);
            }
        }
        lds_barrier();

        // ---- phase 2: U = T R ----
        load3(ci, o3);
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int L = Ls[k];
            f32x4_t Uc = zero4();
#pragma unroll
            for (int m = 0; m < npk(k); ++m)
                if (m <= L / 2) Uc = F::mma8(o2.tp[k][m], sh_R[m][lane], Uc);
            reinterpret_cast<f4 *>(&sh_U[L >> 1][lane])[L & 1] = F::pack(Uc);
        }
        if (int(threadIdx.x) < PP4) sh_pp[threadIdx.x] = o3.pd;
        lds_barrier();

        // ---- phase 3: readout; state carry ----
        load1(min(ci + 1, nchunks - 1), o1);
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int L = Ls[k];
            f32x4_t Oc = QS[k];
#pragma unroll
            for (int m = 0; m < npk(k); ++m)
                if (m <= L / 2) Oc = F::mma8(o3.pp[k][m], sh_U[m][lane], Oc);
            const int tb = ci * C + 16 * L + 4 * G;
#pragma unroll
            for (int r = 0; r < 4; ++r) buf_store_bf16(ro, tok(tb + r) * 2u, 0u, Oc[r]);
        }
        if (owner) {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const f8 ub = sh_U[p][lane];
#pragma unroll
                for (int tt = 0; tt < TPW; ++tt) {
                    const f32x4_t pi = sh_pp[(p * D + 16 * (wave * TPW + tt) + 4 * G) / 4];
                    S[tt] = F::mma8(o3.kb[tt][p], ub, S[tt] * pi);
                }
            }
            put_state();
        }
        lds_barrier();
    }

    if (owner && south) {
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) south[sidx(tt, r)] = S[tt][r];
    }
}

template <int D, int C>
hipError_t solve_typed(const float *e, int B, int T, int H, void *workspace, hipStream_t stream) {
    const int nchunks = (T + C - 1) / C;
    if (nchunks == 0) return hipSuccess;
    using LY = InvLds<C>;
    auto kern = wy_inverse_kernel<D, C>;
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(LY::BYTES));
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(nchunks, H, B), dim3(256), LY::BYTES, stream, e,
                       static_cast<unsigned char *>(workspace), T, H, nchunks);
    return hipGetLastError();
}

template <int D, int C>
hipError_t wy_scan_typed(const void *v, const float *e, const float *w, const float *s0, void *o,
                         float *s_out, int B, int T, int H, const void *workspace,
                         hipStream_t stream) {
    const int nchunks = (T + C - 1) / C;
    const int BH = B * H;
    const int groups = (BH + 7) / 8;
    hipLaunchKernelGGL((wy_scan_kernel<D, C>), dim3(groups * 8 * (D / 16)), dim3(64 * ScanWaves<C>::NW),
                       0, stream,
                       static_cast<const bf16_t *>(v), e, w, s0, static_cast<bf16_t *>(o), s_out,
                       static_cast<const unsigned char *>(workspace), T, H, BH, nchunks);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_wy_solve(const float *e, int B, int T, int H, int d, int chunk, void *workspace,
                           hipStream_t stream) {
#define MUIR_WY(D, C) \
    if (d == D && chunk == C) return solve_typed<D, C>(e, B, T, H, workspace, stream);
    MUIR_WY(64, 64) MUIR_WY(64, 128) MUIR_WY(64, 256)
    MUIR_WY(128, 64) MUIR_WY(128, 128) MUIR_WY(128, 256)
#undef MUIR_WY
    return hipErrorInvalidValue;
}

hipError_t launch_wy_scan(const void *v, const float *e, const float *w, const float *s0, void *o,
                          float *s_out, int B, int T, int H, int d, int chunk,
                          const void *workspace, hipStream_t stream) {
#define MUIR_WY(D, C) \
    if (d == D && chunk == C) return wy_scan_typed<D, C>(v, e, w, s0, o, s_out, B, T, H, workspace, stream);
    MUIR_WY(64, 64) MUIR_WY(64, 128) MUIR_WY(64, 256)
    MUIR_WY(128, 64) MUIR_WY(128, 128) MUIR_WY(128, 256)
#undef MUIR_WY
    return hipErrorInvalidValue;
}

}  // namespace muir
