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
// that scheme's recursive block-Neumann form: 16x16 leaves T_ii = (I + Diag(e_i) M_ii)^-1 by
// forward substitution in fp32, then log2(C / 16) levels that combine pairs of diagonal blocks,
//   T21 = -T22 Diag(e2) M21 T11,
// on the matrix cores; it replaces M in the workspace.
#include "chunk_layout.hpp"
#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace muir {

namespace {

// LDS of the inverse kernel (bytes). Every lower 16x16 tile (i, j), i >= j, of T is kept once,
// as a row fragment in bf16 (lane (x, G): T[16i + x][16j + 4G .. + 3], 8 bytes): the diagonal
// tiles first (slot i), then the others (slot NB + i (i - 1) / 2 + j), which hold M's tiles
// until T's replace them. Then the strictly lower triangles of M's fp32 diagonal blocks
// (element (s, c), c < s, of block i at 120 i + s (s - 1) / 2 + c) and the erase strengths.
// About 76.5 KB at C = 256: two workgroups share a CU.
template <int C> struct InvLds {
    static constexpr int NB = C / 16, NTILE = NB * (NB + 1) / 2;
    static constexpr size_t TILE_OFF = 0;                        // [NTILE][64] x 8 B
    static constexpr size_t MD_OFF = size_t(NTILE) * 512;        // [NB][120] fp32
    static constexpr size_t E_OFF = MD_OFF + size_t(NB) * 480;   // [C] fp32
    static constexpr size_t BYTES = E_OFF + size_t(C) * 4;
};

// Wavefronts of the inverse kernel: eight for 16 or more row blocks, else four.
template <int C> constexpr int inv_waves() { return C / 16 >= 16 ? 8 : 4; }

// One workgroup per (chunk, head, batch): T = (I + Diag(e) M)^-1 by the recursive
// block-Neumann form (openai-hub news page, section on rewriting the long-sequence parallel
// algorithm for TPU: the unit lower-triangular inverse by recursive block products). For a
// diagonal block split into halves,
//   [L11 0; L21 L22]^-1 = [T11 0; -T22 L21 T11  T22],   L21 = Diag(e2) M21,
// so the 16x16 leaves T_ii = (I + Diag(e_i) M_ii)^-1 are solved first (in fp32, by the first
// half of the wavefronts while the second half brings M's tiles into LDS), then log2(C / 16)
// levels each combine pairs of diagonal blocks on the matrix cores: step 1
// Q = Diag(e2) M21 T11, a barrier, step 2 T21 = -T22 Q over M21's slots, a barrier. A level's
// work items are (pair, column tile of T11); an item's column strip of Q stays in registers.
// T goes out once, at the end, over M in the workspace: the kernel streams the M region in
// and out and the fp32 diagonal blocks in, and touches nothing else in HBM.
template <int D, int C>
__global__ __launch_bounds__(64 * inv_waves<C>()) __attribute__((amdgpu_waves_per_eu(4)))
void wy_inverse_kernel(const float *__restrict__ e, unsigned char *__restrict__ ws, int T, int H,
                       int nchunks) {
    using SL = Slot<bf16_t, D, C>;
    using LY = InvLds<C>;
    using F = Frag<bf16_t>;
    using f4 = F::f4;
    using f8 = F::f8;
    constexpr int NB = C / 16, NW = inv_waves<C>(), NT = 64 * NW, NPAIR = SL::NPAIR;
    constexpr int NW2 = NW / 2, NT2 = NT / 2;     // wavefronts and threads per half
    constexpr int NPW = (NPAIR + NW - 1) / NW;    // pair slots per wavefront in the write-out
    constexpr int NPL = (NPAIR + NW2 - 1) / NW2;  // pair slots per wavefront of the M half
    constexpr int NMD = NB * 64 / NT2;  // 16-byte loads of the fp32 diagonal blocks per thread
    static_assert(NB / 2 <= NW && NB * 16 <= NT2 && C <= NT2 && (NB * 64) % NT2 == 0,
                  "work split");

    extern __shared__ __align__(16) unsigned char smem[];
    f4 *sh_t = reinterpret_cast<f4 *>(smem + LY::TILE_OFF);
    float *sh_md = reinterpret_cast<float *>(smem + LY::MD_OFF);
    float *sh_e = reinterpret_cast<float *>(smem + LY::E_OFF);
    auto slot_of = [](int i, int j) { return i == j ? i : NB + i * (i - 1) / 2 + j; };

    const int ci = blockIdx.x, hh = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, x = lane & 15, G = lane >> 4;
    unsigned char *slot = ws + ((size_t(b) * H + hh) * nchunks + ci) * SL::BYTES;
    bf16_t *gT = reinterpret_cast<bf16_t *>(slot + SL::M_OFF);
    const float *gMD = reinterpret_cast<const float *>(slot + SL::MD_OFF);
    const int t0 = ci * C, nreal = min(C, T - t0);
    const unsigned lo_pair = unsigned((4 * x + G) * 8);  // lane's 8 elements of a pair slot
    const f4 z4 = {0, 0, 0, 0};

    // Block row and pair index of pair slot ps (wave-uniform): the row is the number of rows
    // after the first whose first slot is at or below ps, a sum of compile-time comparisons
    // (a search loop here cost more scalar instructions than the kernel's vector ones).
    auto pair_rc = [](int ps, int &row, int &m) {
        int t = 0;
#pragma unroll
        for (int k = 1; k < NB; ++k) t += SL::prow(k) <= ps ? 1 : 0;
        row = t;
        m = ps - SL::prow(t);
    };

    // Inputs. The two halves of the workgroup take different parts, so that each half's
    // waits cover only its own loads and no wavefront holds M's tiles in registers through the
    // leaves' substitution:
    //   leaf half (wavefronts 0 .. NW/2 - 1): e (0 past the sequence end) and the strict lower
    //     triangles of the fp32 diagonal blocks into LDS, a barrier, then the leaves;
    //   M half: its share of M's pair slots, in flight over that barrier, then into the
    //     off-diagonal tile slots. The pair slots holding an off-diagonal tile are all but the
    //     diagonal pair (t, t + 1) of an even row t (an odd row's last pair holds (t, t - 1) and
    //     the diagonal tile).
    // Every load is unconditional; an index past the end is clamped and reads valid, unused data.
    if (wave < NW2) {
        const float e_t = e[(size_t(b) * T + t0 + min(tid, nreal - 1)) * H + hh];
        f32x4_t mdv[NMD];
#pragma unroll
        for (int k = 0; k < NMD; ++k) mdv[k] = reinterpret_cast<const f32x4_t *>(gMD)[tid + k * NT2];
        if (tid < C) sh_e[tid] = tid < nreal ? e_t : 0.f;
#pragma unroll
        for (int k = 0; k < NMD; ++k) {
            const int n = tid + k * NT2, i = n >> 6, s2 = (n >> 2) & 15, c0 = 4 * (n & 3);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (c0 + q < s2) sh_md[i * 120 + s2 * (s2 - 1) / 2 + c0 + q] = mdv[k][q];
        }
        lds_barrier();
        // Leaves: thread (i, r) solves row r of T_ii from T L = I, right to left:
        // y_c = [c == r] - sum_{s > c} y_s e_s M_ii[s][c] (y_s = 0 for s > r), in fp32; each
        // group of four finished values goes to its row fragment at once.
        if (tid < NB * 16) {
            const int i = tid >> 4, r = tid & 15;
            const float *md = sh_md + i * 120;
            const float *ee = sh_e + 16 * i;
            float z[16];
            f32x4_t y4;
#pragma unroll
            for (int c = 15; c >= 0; --c) {
                float acc = 0.f;
#pragma unroll
                for (int s2 = c + 1; s2 < 16; ++s2) acc += z[s2] * md[s2 * (s2 - 1) / 2 + c];
                const float yc = (c == r ? 1.f : 0.f) - acc;
                z[c] = yc * ee[c];
                y4[c & 3] = yc;
                if ((c & 3) == 0) sh_t[slot_of(i, i) * 64 + r + 16 * (c >> 2)] = F::pack(y4);
            }
        }
    } else {
        const int mw = wave - NW2;
        f8 mreg[NPL];
#pragma unroll
        for (int n = 0; n < NPL; ++n)
            mreg[n] = F::load8(gT + size_t(min(mw + NW2 * n, NPAIR - 1)) * 512 + lo_pair);
        lds_barrier();
#pragma unroll
        for (int n = 0; n < NPL; ++n) {
            const int ps = mw + NW2 * n;
            int t, m;
            if (ps < NPAIR) {
                pair_rc(ps, t, m);
                if (2 * m < t) {
                    sh_t[slot_of(t, 2 * m) * 64 + lane] = F::lo(mreg[n]);
                    if (2 * m + 1 < t) sh_t[slot_of(t, 2 * m + 1) * 64 + lane] = F::hi(mreg[n]);
                }
            }
        }
    }
    lds_barrier();

    auto row = [&](int i, int j) { return sh_t[slot_of(i, j) * 64 + lane]; };
    // Column fragment of tile (i, j) (lane (x, G): T[4G + q][x]) from its row fragment, where
    // element (row, col) sits in lane row + 16 (col / 4), value col % 4.
    auto col = [&](int i, int j) {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(sh_t + slot_of(i, j) * 64);
        f4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = p[(4 * G + q + 16 * (x >> 2)) * 4 + (x & 3)];
        return v;
    };
    static_for<31 - __builtin_clz(NB)>([&](auto Lc) {
        constexpr int HB = 1 << decltype(Lc)::value;  // tiles per half of a combined block
        constexpr int NKQ = (HB + 1) / 2;             // K = 32 pairs over a half
        const int item = wave;                         // NB / 2 items, at most NW
        const bool active = item < NB / 2;
        const int p = item / HB;
        const int base1 = 2 * p * HB, base2 = base1 + HB;  // T11 and T22 tile ranges
        const int s0 = base1 + item % HB;                  // this item's column tile
        // Step 1: Q(t, s0) = Diag(e) sum_k M(t, k) T11(k, s0), k over T11's tiles k >= s0; for
        // HB = 1 the pair's second tile lies outside T11 and is zero.
        f4 Q[HB];
        if (active) {
            f32x4_t acc[HB];
#pragma unroll
            for (int tt = 0; tt < HB; ++tt) acc[tt] = zero4();
#pragma unroll
            for (int kq = 0; kq < NKQ; ++kq) {
                const int k0 = base1 + 2 * kq;
                if (k0 + 1 < s0) continue;  // both tiles above T11's diagonal
                const f8 bt = F::cat(k0 >= s0 ? col(k0, s0) : z4, HB > 1 ? col(k0 + 1, s0) : z4);
#pragma unroll
                for (int tt = 0; tt < HB; ++tt) {
                    const int t = base2 + tt;
                    const f8 mt = F::cat(row(t, k0), HB > 1 ? row(t, k0 + 1) : z4);
                    acc[tt] = F::mma8(mt, bt, acc[tt]);
                }
            }
#pragma unroll
            for (int tt = 0; tt < HB; ++tt) {
                const f32x4_t ev = *reinterpret_cast<const f32x4_t *>(sh_e + 16 * (base2 + tt) + 4 * G);
                Q[tt] = F::pack(acc[tt] * ev);
            }
        }
        lds_barrier();  // every read of M21 is done
        // Step 2: T21(t1, s0) = -sum_t T22(t1, t) Q(t, s0), t over T22's tiles t <= t1; for
        // HB = 1 the pair is (t1 - 1, t1) and only its second tile is T22's.
        if (active) {
#pragma unroll
            for (int tp = 0; tp < HB; ++tp) {
                const int t1 = base2 + tp;
                f32x4_t acc = zero4();
#pragma unroll
                for (int rq = 0; rq < NKQ; ++rq) {
                    if (2 * rq > tp) continue;  // tiles above T22's diagonal
                    const int r0 = HB == 1 ? t1 - 1 : base2 + 2 * rq;
                    const f4 lo = HB == 1 ? z4 : row(t1, r0);
                    const f4 hi = r0 + 1 <= t1 ? row(t1, r0 + 1) : z4;
                    const f8 q = HB == 1 ? F::cat(z4, Q[0])
                                         : F::cat(Q[2 * rq], Q[2 * rq + 1 < HB ? 2 * rq + 1 : 0]);
                    acc = F::mma8(q, F::cat(lo, hi), acc);  // lane (x, G): T21[x][4G + q]
                }
                sh_t[slot_of(t1, s0) * 64 + lane] = F::pack(-acc);
            }
        }
        lds_barrier();
    });

    // T over M in the workspace, one 16-byte store per lane and pair slot; the second tile of
    // an even row's diagonal pair is zero.
#pragma unroll
    for (int n = 0; n < NPW; ++n) {
        const int ps = wave + NW * n;
        int t, m;
        if (ps < NPAIR) {
            pair_rc(ps, t, m);
            const f4 hi = 2 * m + 1 <= t ? row(t, 2 * m + 1) : z4;
            *reinterpret_cast<f8 *>(gT + size_t(ps) * 512 + lo_pair) = F::cat(row(t, 2 * m), hi);
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

    // Every phase issues its global loads ahead of the work that waits for them (a wavefront's
    // loads complete in order, so a load used at once makes every later one wait): phase 1's at
    // the start, phase 2's T pairs when phase 1's work begins, phase 3's (K*beta)^T fragments and
    // P pairs when phase 2's products are done. All are unconditional: a pair index past a block
    // row's last is clamped to it and its product skipped.
    constexpr int NU1 = NB * NCT / NW;  // w*v tiles per wavefront
    constexpr int NU2 = NB * NKD / NW;  // e*(K*gamma) fragments per wavefront
    static_assert(NU1 * NW == NB * NCT && NU2 * NW == NB * NKD, "work split");
    // Pair slots of the k-th block a wavefront takes: at most this many.
    constexpr auto maxm = [](int k) {
        return (NB >= 2 * NW ? 2 * NW * (k >> 1) + ((k & 1) ? 2 * NW - 1 : NW - 1) : NB - 1) / 2 + 1;
    };

    // ---- 1: operands in accumulator layout; pair decays, e and gamma_C ----
    const float e_t = e[(size_t(b) * T + t0 + min(tid, nreal - 1)) * H + hh];
    constexpr int NPPL = (NP * D + 64 * NW - 1) / (64 * NW);
    float ppl[NPPL], gcl[NP];
#pragma unroll
    for (int n = 0; n < NPPL; ++n) ppl[n] = gPP[min(tid + n * 64 * NW, NP * D - 1)];
#pragma unroll
    for (int q = 0; q < NP; ++q) gcl[q] = gPP[q * D + (tid & (D - 1))];
    // w*v of token 16L + x, value columns 16c + 4G .. + 3 (row layout), tokens past the end zero;
    // e*(K*gamma): one fragment gives both 16-channel halves of a channel group.
    const rsrc_t rv = make_rsrc(v + (size_t(b) * T + t0) * HD + size_t(hh) * D,
                                unsigned((size_t(nreal - 1) * HD + D) * 2));
    const rsrc_t rw = make_rsrc(w + (size_t(b) * T + t0) * HD + size_t(hh) * D,
                                unsigned((size_t(nreal - 1) * HD + D) * 4));
    u16x4_t vv[NU1];
    f32x4_t wv[NU1];
    f8 kg[NU2];
#pragma unroll
    for (int k = 0; k < NU1; ++k) {
        const int u = wave + NW * k, L = u / NCT, c = u % NCT;
        const unsigned off = unsigned(16 * L + x) * unsigned(HD) + unsigned(16 * c + 4 * G);
        vv[k] = Row4<bf16_t>::load(rv, off * 2u, 0u);
        wv[k] = buf_load_f4(rw, off * 4u, 0u);
    }
#pragma unroll
    for (int k = 0; k < NU2; ++k) {
        const int u = wave + NW * k, L = u / NKD, kk = u % NKD;
        kg[k] = F::load8(gKg + frag_idx(16 * L, 32 * kk, D) + lo_frag);
    }
    if (tid < C) sh_e[tid] = tid < nreal ? e_t : 0.f;
#pragma unroll
    for (int n = 0; n < NPPL; ++n)
        if (tid + n * 64 * NW < NP * D) sh_pp[tid + n * 64 * NW] = ppl[n];
    if (tid < D) {
        float gc = 1.f;
#pragma unroll
        for (int q = 0; q < NP; ++q) gc *= gcl[q];
        reinterpret_cast<float *>(xslot + XS::GC_OFF)[tid] = gc;
    }
    lds_barrier();  // e is in LDS for every wavefront's e * (K*gamma) below

    // Phase 2's T pairs, in flight during phase 1's work.
    f8 tpr[BD::NPW][maxm(BD::NPW - 1)];
    static_for<BD::NPW>([&](auto Kc) {
        constexpr int k = decltype(Kc)::value;
        const int i = BD::block(wave, k);
#pragma unroll
        for (int m = 0; m < maxm(k); ++m) tpr[k][m] = pair(gT, i, min(m, i / 2));
    });
    {
        const f4 unit = F::unit(x, G);
#pragma unroll
        for (int k = 0; k < NU1; ++k) {
            const int u = wave + NW * k, L = u / NCT, c = u % NCT;
            f32x4_t p;
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = wv[k][r] * bf16_to_f32(vv[k][r]);
            reinterpret_cast<f4 *>(b2(L >> 1, c) + lane)[L & 1] = F::pack(F::mma16_fresh(F::pack(p), unit));
        }
#pragma unroll
        for (int k = 0; k < NU2; ++k) {
            const int u = wave + NW * k, L = u / NKD, kk = u % NKD;
            const f32x4_t ev = *reinterpret_cast<const f32x4_t *>(sh_e + 16 * L + 4 * G);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const f32x4_t t = F::mma16_fresh(hf ? F::hi(kg[k]) : F::lo(kg[k]), unit);
                reinterpret_cast<f4 *>(b1(L >> 1, 2 * kk + hf) + lane)[L & 1] = F::pack(t * ev);
            }
        }
    }
    lds_barrier();

    // ---- 2: W = T e*Kg and U~ = T w*v per token block ----
    f8 kbt[NP];
    f8 ppr[BD::NPW][maxm(BD::NPW - 1)];
    {
        f32x4_t aw[BD::NPW][NCT], au[BD::NPW][NCT];
#pragma unroll
        for (int k = 0; k < BD::NPW; ++k)
#pragma unroll
            for (int c = 0; c < NCT; ++c) aw[k][c] = au[k][c] = zero4();
        if (BD::active(wave)) {
            static_for<BD::NPW>([&](auto Kc) {
                constexpr int k = decltype(Kc)::value;
                const int i = BD::block(wave, k);
#pragma unroll
                for (int m = 0; m < maxm(k); ++m) {
                    if (m > i / 2) continue;
#pragma unroll
                    for (int c = 0; c < NCT; ++c) {
                        aw[k][c] = F::mma8(tpr[k][m], b1(m, c)[lane], aw[k][c]);
                        au[k][c] = F::mma8(tpr[k][m], b2(m, c)[lane], au[k][c]);
                    }
                }
            });
        }
        // Phase 3's operands, in flight over the barriers below.
        {
            const int c = wave < NCT ? wave : 0;
#pragma unroll
            for (int q = 0; q < NP; ++q) kbt[q] = F::load8(gKbT + frag_idx(16 * c, 32 * q, C) + lo_frag);
        }
        static_for<BD::NPW>([&](auto Kc) {
            constexpr int k = decltype(Kc)::value;
            const int i = BD::block(wave, k);
#pragma unroll
            for (int m = 0; m < maxm(k); ++m) ppr[k][m] = pair(gP, i, min(m, i / 2));
        });
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
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const float pcol = sh_pp[q * D + 16 * c + x];  // A~^T: column = channel 16c + x
            const f32x4_t prow = *reinterpret_cast<const f32x4_t *>(sh_pp + q * D + 16 * c + 4 * G);
#pragma unroll
            for (int j = 0; j < NCT; ++j) {
                at[j] = F::mma8(b1(q, j)[lane], kbt[q], at[j] * pcol);  // rows j (W), columns i
                bc[j] = F::mma8(kbt[q], b2(q, j)[lane], bc[j] * prow);  // rows i, columns value j
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
        static_for<BD::NPW>([&](auto Kc) {
            constexpr int k = decltype(Kc)::value;
            const int i = BD::block(wave, k);
            f8 qg[NKD];
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) qg[kk] = F::load8(gQg + frag_idx(16 * i, 32 * kk, D) + lo_frag);
            f32x4_t pw[NCT], ou[NCT];
#pragma unroll
            for (int j = 0; j < NCT; ++j) pw[j] = ou[j] = zero4();
#pragma unroll
            for (int m = 0; m < maxm(k); ++m) {
                if (m > i / 2) continue;
#pragma unroll
                for (int j = 0; j < NCT; ++j) {
                    pw[j] = F::mma8(b1(m, j)[lane], ppr[k][m], pw[j]);  // (P W)^T: lane (t, G) row t
                    ou[j] = F::mma8(ppr[k][m], b2(m, j)[lane], ou[j]);  // P U~: accumulator layout
                }
            }
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) {
                const size_t fo = frag_idx(16 * i, 32 * kk, D) + lo_frag;
                f32x4_t lo, hi;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    lo[r] = bf16_to_f32(qg[kk][r]) - pw[2 * kk][r];
                    hi[r] = bf16_to_f32(qg[kk][4 + r]) - pw[2 * kk + 1][r];
                }
                *reinterpret_cast<f8 *>(gQT + fo) = F::cat(F::pack(lo), F::pack(hi));
            }
#pragma unroll
            for (int j = 0; j < NCT; ++j) *reinterpret_cast<f4 *>(gOT + ((i * NCT + j) * 64 + lane) * 4) = F::pack(ou[j]);
        });
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
