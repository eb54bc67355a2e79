// The sequential phase of the chunk forward with its work split over four wavefronts, one
// per SIMD, that meet at one LDS barrier per 16-token leaf.
//
// The serial dependency of the scan runs through every leaf of every chunk: leaf L's
// right-hand side needs U of leaf L - 1, so one wavefront must take each leaf's
// forward substitution in turn (openai-hub news page, section on rewriting the
// long-sequence parallel algorithm for TPU: the recursive block-Neumann solve; here its
// off-diagonal products between leaves run on the matrix cores and its 16-token leaves by
// substitution). Everything else a leaf needs can be made while the previous leaves are
// being solved. A wavefront issues its instructions in order, so a chain that also issues
// those other products and their loads is slowed by them even when they are independent
// of it; here they go to wavefronts of their own:
//
//   chain (wave 0)   per leaf L: acc = acc_pre + M_{L,serial pair} U, the right-hand side
//                    w*v - e*acc, the forward substitution, the transpose of u into the U
//                    operand, which it leaves in LDS. During leaf L it also forms acc_pre
//                    of leaf L + 1 from what the helper left in LDS.
//   helper (wave 1)  during leaf L, the part of leaf L + 2's right-hand side that does not
//                    need the last leaves' U: (K*gamma)_{L+2} S0 + sum M_{L+2,l} U_l over the
//                    leaf pairs l that are solved by then (the first term from wave 3).
//   state (wave 2)   the state carry in Horner form, one leaf pair at a time as soon as its
//                    U is in LDS: S <- Diag(pair decay) S + (K*beta')^T U, and at each chunk
//                    start the state's bf16 operand copy for the helper (and, through the
//                    readout region of the workspace, for the readout kernel below).
//   hand-over (wave 3) H_L = (K*gamma)_L S0 of leaves L >= 2 a phase before the helper
//                    needs it; U of the chunk before, one leaf pair per phase, into the
//                    readout region; the staging of the next chunk's pair decays and
//                    diagonal blocks into LDS and its L2 warm-up.
//
// The readout O = (Qh*gamma) S0 + P U needs nothing from the next chunk, and inside the scan
// its operand loads (Qh*gamma and P, the same for all of a head's workgroups) compete with the
// chain's for the compute unit's load path; as a kernel of its own it runs over all chunks at
// once, at the rate of its memory traffic.
//
// Which leaf pairs go where: the chain multiplies the pair that holds leaf L - 1 (for odd L
// that is leaf L - 1 and the zero diagonal block), and for odd L also the pair before, into
// acc_pre during leaf L - 1; the helper takes all earlier pairs. The helper then needs U
// only up to leaf L - 3, so it can work two leaves ahead. Every sum is accumulated in the
// same order as in the two-wavefront scan (H first, then the pairs in order, the serial
// pair last), so both kernels give the same bits.
//
// Per chunk there are NB leaf phases and two more: in the first the state wavefront applies
// the chunk before's last leaf pair and publishes the new chunk's start state; in the
// second the helper makes the first two leaves' right-hand sides from it (and the hand-over
// wavefront H_2). One extra iteration after the last chunk lets the state and hand-over
// wavefronts finish. Every wavefront passes the same barriers in the same order.
#include <type_traits>
#include <utility>

#include "chunk_layout.hpp"
#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"
#include "scan_leaf.hpp"

namespace muir {

namespace {

// Leaf pairs j < help_pairs(L) of leaf L's right-hand side are the helper's: the chain takes
// the pair holding leaf L - 1, and for odd L the pair before it as well.
constexpr int help_pairs(int L) { return L < 2 ? 0 : (L - 2 - (L & 1)) / 2; }
// The pair of row L >= 1 holding leaf L - 1 (for odd L, leaf L - 1 and the zero diagonal).
constexpr int ser_pair(int L) { return (L - 1) / 2; }

// PK: e and w tile-packed, [B*H][D/8][T][8] fp32, so that a leaf's rows of this workgroup's eight
// columns are one contiguous 512-byte run each (with the [B, T, H, D] layout they are sixteen
// 32-byte pieces of sixteen cache lines).
// SAVE (the backward pass's rerun of the forward): no readout; the chain keeps u = w*v - e*p of
// every token in fp32 ([B, T, H, D], u_save) and the state wavefront the state at every 64-token
// block start and at the end ([B*H][ceil(T/64) + 1][D][D] fp32, st_save), as the two-wavefront
// scan's saving instance does, bit for bit.
template <int D, int C, int VC, bool PK, bool SAVE = false>
__global__ __launch_bounds__(256) void chunk_scan_split_kernel(
    const bf16_t *__restrict__ v, const float *__restrict__ e, const float *__restrict__ w,
    const float *__restrict__ s0, float *__restrict__ s_out, const unsigned char *__restrict__ ws,
    unsigned char *__restrict__ rd, int T, int H, int BH, int nchunks,
    float *__restrict__ u_save = nullptr, float *__restrict__ st_save = nullptr) {
    using SL = Slot<bf16_t, D, C>;
    using F = Frag<bf16_t>;
    using f4 = F::f4;
    using f8 = F::f8;
    constexpr int NB = C / 16;    // leaves per chunk
    constexpr int NCT = D / 16;   // 16-channel tiles of the state
    constexpr int NKD = D / 32;   // K = 32 steps over the channels
    constexpr int HALF = NCT / 2; // state tiles carried per phase
    constexpr int NP = NB / 2;    // leaf pairs per chunk
    constexpr unsigned OB = 2;    // operand bytes
    static_assert(!PK || VC == 2, "packed e and w come in 8-column tiles");
    static_assert(!SAVE || C % 64 == 0, "saved states are 64 tokens apart");

    // S0 of a chunk as bf16 operands, by chunk parity (state -> helper, readout).
    __shared__ f4 sh_fS[2][NCT][64];
    // U of every leaf, by chunk parity, leaves 2j and 2j + 1 of a lane as one K = 32 operand.
    __shared__ f8 sh_U[2][NP][64];
    // Pair decays per channel and the fp32 diagonal blocks of M, by chunk parity (staged by
    // the hand-over wavefront one chunk ahead).
    __shared__ __align__(16) float sh_pp[2][NP][D];
    __shared__ __align__(16) f32x4_t sh_md[2][NB][64];
    // acc_pre parts from the helper, a ring over leaves (written two leaves ahead).
    __shared__ __align__(16) f32x4_t sh_acc[4][64];
    // H_L = (K*gamma)_L S0 of leaves L >= 2 from the hand-over wavefront, a ring over leaves
    // (written three leaves ahead, one phase before the helper adds the leaf pairs to it).
    __shared__ __align__(16) f32x4_t sh_h[4][64];

    // Workgroups go to the eight XCDs round-robin; a head's value tiles share one XCD.
    constexpr int NVT = D / (4 * VC);
    const int id = blockIdx.x;
    const int bh = (id >> 3) / NVT * 8 + (id & 7);
    const int ct = (id >> 3) % NVT;
    if (bh >= BH) return;  // the whole workgroup: no barrier is left waiting
    const int b = bh / H, h = bh % H;
    const int j0 = 4 * VC * ct;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, x = lane & 15, g = lane >> 4;
    const size_t HD = size_t(H) * D;
    const bool col_ok = (x & 3) < VC;
    const unsigned lo_st = unsigned(4 * g * D + VC * (x >> 2) + (x & 3));  // state [4g][column]
    const float *s0h = s0 ? s0 + size_t(bh) * D * D + j0 : nullptr;
    float *south = s_out ? s_out + size_t(bh) * D * D + j0 : nullptr;

    // SAVE: this head's saved states, from this tile's first column.
    const int n64 = (T + 63) / 64;
    float *svst = SAVE ? st_save + size_t(bh) * (n64 + 1) * D * D + j0 : nullptr;
    if (nchunks == 0) {
        if (wave == 0 && col_ok) {
#pragma unroll
            for (int c = 0; c < NCT; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x0 = s0h ? s0h[size_t(16 * c + i) * D + lo_st] : 0.f;
                    if (south) south[size_t(16 * c + i) * D + lo_st] = x0;
                    if constexpr (SAVE) svst[size_t(16 * c + i) * D + lo_st] = x0;
                }
        }
        return;
    }

    const unsigned lo_pair = unsigned((4 * x + g) * 8) * OB;  // block pair: row x, cols 4g..
    const unsigned lo_frag = unsigned(lane * 8) * OB;         // lane's share of a fragment
    const unsigned lo_f = unsigned(x * HD + VC * g) * 4u;     // e, w, og: token x, group g
    const unsigned lo_q = unsigned(x * HD + VC * g) * 2u;     // v, o
    // Descriptors: this head's chunk slots (a chunk index past the end is clamped, so
    // prefetches read valid, unused data) and one [B, T, H, *] column tile per token tensor
    // (rows at or past T read zero, stores there are dropped).
    const rsrc_t rws = make_rsrc(ws + size_t(bh) * nchunks * SL::BYTES, unsigned(size_t(nchunks) * SL::BYTES));
    auto wsoff = [&](int ci, size_t off) { return unsigned(size_t(min(ci, nchunks - 1)) * SL::BYTES + off); };
    const size_t tok0 = size_t(b) * T * HD + size_t(h) * D + j0;
    const unsigned tok_elems = unsigned(size_t(T) * HD - size_t(h) * D - j0);
    auto trow = [&](int t, unsigned es) { return unsigned(min(t, T)) * unsigned(HD) * es; };
    auto load_kg = [&](int ci, int L, size_t OFF, f8 (&dst)[NKD]) {
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk)
            dst[kk] = F::bload8(rws, lo_frag, wsoff(ci, OFF + frag_idx(16 * L, 32 * kk, D) * OB));
    };
    // Blocks (bt, 2j) and (bt, 2j + 1) of M or P as one K = 32 operand.
    auto load_pair = [&](int ci, size_t OFF, int bt, int j) {
        return F::bload8(rws, lo_pair, wsoff(ci, OFF + size_t(SL::prow(bt) + j) * 512 * OB));
    };
    auto u_put = [&](int buf, int L, f4 u) {
        reinterpret_cast<f4 *>(&sh_U[buf][L >> 1][lane])[L & 1] = u;
    };
    // The readout region of this head's 16-column tile ct / 2: fragment row x + 2 (ct % 2)
    // holds what lane row x holds here (lanes with x % 4 >= 2 hold padding and store nothing).
    constexpr size_t TB = readout_tile_bytes(D, C), RCB = readout_chunk_bytes(D, C);
    const rsrc_t rrd = make_rsrc(rd + size_t(bh) * nchunks * RCB + size_t(ct >> 1) * TB,
                                 unsigned(size_t(nchunks) * RCB - size_t(ct >> 1) * TB));
    const unsigned lo_rd = unsigned(16 * (16 * g + x + 2 * (ct & 1)));
    auto rd_put = [&](int ci, int frag, f8 val) {
        if constexpr (SAVE) return;  // no readout: nothing to hand over
        if (col_ok)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, val), rrd, int(lo_rd),
                                                   int(size_t(ci) * RCB + size_t(frag) * 1024), 0);
    };

    // ------------------------------------------------------------------------------------
    if (wave == 3) {
        // Hands U of the chunk before to the readout region, one leaf pair per phase (the
        // chain fills the other parity's buffer meanwhile), and stages the next chunk's pair
        // decays and diagonal blocks into LDS.
        constexpr int PP4 = NP * D / 4;
        constexpr int PPN = (PP4 + 63) / 64;
        f32x4_t ppt[PPN], mdt[NB];
        auto load_stage = [&](int ci) {
#pragma unroll
            for (int n = 0; n < PPN; ++n)
                if (n * 64 + lane < PP4)
                    ppt[n] = buf_load_f4(rws, unsigned(16 * (n * 64 + lane)), wsoff(ci, SL::PP_OFF));
#pragma unroll
            for (int L = 0; L < NB; ++L) mdt[L] = buf_load_f4(rws, unsigned(16 * lane), wsoff(ci, SL::MD_OFF + L * 1024));
        };
        auto put_stage = [&](int ci) {
            f32x4_t *dst = reinterpret_cast<f32x4_t *>(&sh_pp[ci & 1][0][0]);
#pragma unroll
            for (int n = 0; n < PPN; ++n)
                if (n * 64 + lane < PP4) dst[n * 64 + lane] = ppt[n];
#pragma unroll
            for (int L = 0; L < NB; ++L) sh_md[ci & 1][L][lane] = mdt[L];
        };
        // Every workgroup of a head reads the same chunk slots in step, so each touches its
        // share of the next chunk's slot a chunk ahead (one word per 128-byte line), and the
        // head's other workgroups then find those lines in the L2 they share.
        // Only the slot's parts the scan reads: M and the pair decays, K*gamma, and (K*beta')^T
        // with the diagonal blocks (Qh*gamma and P are the readout kernel's; touching them cost
        // the scan 2-3%).
        constexpr int LA = int(SL::P_OFF / 128), LB = int((SL::QG_OFF - SL::KG_OFF) / 128),
                      LC = int((SL::BYTES - SL::KBT_OFF) / 128);
        constexpr int LINES = LA + LB + LC;
        constexpr int LINES_WG = (LINES + NVT - 1) / NVT;
        constexpr int NTOUCH = (LINES_WG + 63) / 64;
        unsigned touched = 0;
        auto touch = [&](int ci, int n) {
            const int v = min(ct * LINES_WG + n * 64 + lane, LINES - 1);
            const int line = v < LA ? v
                           : v < LA + LB ? int(SL::KG_OFF / 128) + (v - LA)
                                         : int(SL::KBT_OFF / 128) + (v - LA - LB);
            const unsigned off = unsigned(line) * 128u;
            touched += __builtin_amdgcn_raw_buffer_load_b32(rws, int(off), int(wsoff(ci, 0)), 0);
        };
        // The next chunk's staging goes to the buffers of the other parity: nobody reads them
        // during this chunk (the state wavefront's carry of the chunk before's last pair comes
        // before phase 2). A clamped chunk index past the end reads valid, unused data.
        auto stage_phase = [&](int cn, auto Lc) {
            constexpr int L = decltype(Lc)::value;
            if constexpr (L == 0) load_stage(cn);
            if constexpr (L == 2) put_stage(cn);
            if constexpr (L < NTOUCH) touch(cn, L);
        };
        // H_L = (K*gamma)_L S0 of leaves 2 .. NB - 1: H_2 in phase Z2, H_{L+3} in leaf phase L,
        // each from K*gamma rows loaded two phases ahead (leaves 2 .. 4 of the next chunk in
        // the last phases of a chunk), in a ring over leaves.
        constexpr int RK = 4;
        f8 kgr[RK][NKD];
        f4 fS[NCT];
        auto h_make = [&](auto Lc) {
            constexpr int L = decltype(Lc)::value;
            f32x4_t a = zero4();
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) a = F::mma8(F::cat(fS[2 * kk], fS[2 * kk + 1]), kgr[L % RK][kk], a);
            sh_h[L & 3][lane] = a;
        };
        auto load_next = [&](int cn, auto Lc) {
            constexpr int L = decltype(Lc)::value;
            if constexpr (L == (NB > 3 ? NB - 3 : 0)) {
                if constexpr (2 < NB) load_kg(cn, 2, SL::KG_OFF, kgr[2 % RK]);
                if constexpr (3 < NB) load_kg(cn, 3, SL::KG_OFF, kgr[3 % RK]);
            }
            if constexpr (L == (NB > 3 ? NB - 2 : 0) && 4 < NB) load_kg(cn, 4, SL::KG_OFF, kgr[4 % RK]);
        };
        // Iteration k: H of chunk k (WH), U of chunk k - 1 (WU), staging of chunk k + 1.
        auto iter = [&](int k, auto wh, auto wu) {
            constexpr bool WH = decltype(wh)::value, WU = decltype(wu)::value;
            lds_barrier();  // phase Z1: the state wavefront publishes S0
            if constexpr (WH) {
#pragma unroll
                for (int t = 0; t < NCT; ++t) fS[t] = sh_fS[k & 1][t][lane];
                if constexpr (2 < NB) h_make(std::integral_constant<int, 2>{});
            }
            lds_barrier();  // phase Z2
            static_for<NB>([&](auto Lc) {
                constexpr int L = decltype(Lc)::value;
                stage_phase(k + 1, Lc);
                if constexpr (WU && L < NP) rd_put(k - 1, NKD + L, sh_U[(k - 1) & 1][L][lane]);
                if constexpr (WH) {
                    if constexpr (L + 5 < NB) load_kg(k, L + 5, SL::KG_OFF, kgr[(L + 5) % RK]);
                    if constexpr (L + 3 < NB) h_make(std::integral_constant<int, L + 3>{});
                    load_next(k + 1, Lc);
                }
                lds_barrier();  // end of leaf phase L
            });
        };
        load_stage(0);
        put_stage(0);
        load_next(0, std::integral_constant<int, (NB > 3 ? NB - 3 : 0)>{});
        load_next(0, std::integral_constant<int, (NB > 3 ? NB - 2 : 0)>{});
        lds_barrier();
        iter(0, std::true_type{}, std::false_type{});
        for (int k = 1; k < nchunks; ++k) iter(k, std::true_type{}, std::true_type{});
        iter(nchunks, std::false_type{}, std::true_type{});
        // The touched words are not needed; this keeps their loads.
        asm volatile("" ::"v"(touched));
        return;
    }

    // ------------------------------------------------------------------------------------
    if (wave == 2) {
        // The state: S[t][i] = state[16t + 4g + i][j0 + x], fp32 accumulators, carried in
        // Horner form over leaf pairs.
        f32x4_t S[NCT];
#pragma unroll
        for (int t = 0; t < NCT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[t][i] = s0h && col_ok ? s0h[size_t(16 * t + i) * D + lo_st] : 0.f;
        auto load_kbt = [&](int ci, int pair, int t) {
            return F::bload8(rws, lo_frag, wsoff(ci, SL::KBT_OFF + frag_idx(16 * t, 32 * pair, C) * OB));
        };
        auto lds_pp = [&](int ci, int pair, int t) {
            return *reinterpret_cast<const f32x4_t *>(&sh_pp[ci & 1][pair][16 * t + 4 * g]);
        };
        // Tiles of phase L >= 2: pair (L - 2) / 2, tiles (L & 1) * HALF + [0, HALF); loaded RS - 1
        // phases ahead, those of phases 2 .. RS in phase Z1.
        constexpr int RS = 4;
        f8 kbt[RS][HALF], kbtLast[NCT];
        auto load_half = [&](int ci, int L, f8 (&dst)[HALF]) {
#pragma unroll
            for (int t = 0; t < HALF; ++t) dst[t] = load_kbt(ci, (L - 2) / 2, t + (L & 1) * HALF);
        };
        auto save_state = [&](int slot) {
            if (col_ok) {
                float *dst = svst + size_t(slot) * D * D;
#pragma unroll
                for (int t = 0; t < NCT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) dst[size_t(16 * t + i) * D + lo_st] = S[t][i];
            }
        };
        // The chunk before's last leaf pair (all tiles), into the state.
        auto carry_last = [&](int cp) {
            const f8 u2 = sh_U[cp & 1][NP - 1][lane];
#pragma unroll
            for (int t = 0; t < NCT; ++t) S[t] = F::mma8(kbtLast[t], u2, S[t] * lds_pp(cp, NP - 1, t));
        };
        lds_barrier();
        for (int c = 0; c < nchunks; ++c) {
            static_for<RS - 1>([&](auto Ic) {
                constexpr int L = 2 + decltype(Ic)::value;
                if constexpr (L < NB) load_half(c, L, kbt[L % RS]);
            });
            if (c >= 1) carry_last(c - 1);
            if constexpr (SAVE) save_state(c * (C / 64));
            f4 pk[NCT];
#pragma unroll
            for (int t = 0; t < NCT; ++t) {
                pk[t] = F::pack(S[t]);
                sh_fS[c & 1][t][lane] = pk[t];
            }
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) rd_put(c, kk, F::cat(pk[2 * kk], pk[2 * kk + 1]));
            lds_barrier();  // phase Z1
            lds_barrier();  // phase Z2
            static_for<NB>([&](auto Lc) {
                constexpr int L = decltype(Lc)::value;
                if constexpr (L >= 2 && L + RS - 1 < NB) load_half(c, L + RS - 1, kbt[(L + RS - 1) % RS]);
                if constexpr (L == (NB > 4 ? NB - 4 : 1)) {
#pragma unroll
                    for (int t = 0; t < NCT; ++t) kbtLast[t] = load_kbt(c, NP - 1, t);
                }
                if constexpr (L >= 2) {
                    constexpr int p = (L - 2) / 2, off = (L & 1) * HALF;
                    const f8 u2 = sh_U[c & 1][p][lane];
#pragma unroll
                    for (int t = 0; t < HALF; ++t)
                        S[t + off] = F::mma8(kbt[L % RS][t], u2, S[t + off] * lds_pp(c, p, t + off));
                }
                // SAVE inside a chunk: after phase 4q + 1 every tile has taken the leaf pairs of
                // tokens 0 .. 64q - 1 and no later one, so S is the state at the chunk's 64q-th
                // token. A boundary past the sequence goes to the final state's slot, which the
                // final state overwrites.
                if constexpr (SAVE && L % 4 == 1 && L >= 5) {
                    constexpr int q = (L - 1) / 4;
                    save_state(c * C + 64 * q < T ? c * (C / 64) + q : n64);
                }
                lds_barrier();
            });
        }
        // The iteration after the last chunk: its last pair, then the hand-over wavefront's phases.
        carry_last(nchunks - 1);
        lds_barrier();  // phase Z1
        lds_barrier();  // phase Z2
        for (int L = 0; L < NB; ++L) lds_barrier();
        if (south && col_ok) {
#pragma unroll
            for (int t = 0; t < NCT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) south[size_t(16 * t + i) * D + lo_st] = S[t][i];
        }
        if constexpr (SAVE) save_state(n64);
        return;
    }

    // ------------------------------------------------------------------------------------
    if (wave == 1) {
        // Helper: during leaf phase L, leaf L + 2's right-hand side part: H_{L+2} from the
        // hand-over wavefront plus the leaf pairs below help_pairs(L + 2); at phase Z2, H of
        // leaves 0 and 1 (S0 only).
        auto load_mp = [&](int ci, auto ltc, f8 (&dst)[NP]) {
            constexpr int Lt = decltype(ltc)::value;
#pragma unroll
            for (int j = 0; j < help_pairs(Lt); ++j) dst[j] = load_pair(ci, SL::M_OFF, Lt, j);
        };
        // Leaf Lt's pairs load RH - 1 phases ahead, those of leaves 2 .. RH in phase Z1;
        // kg0, kg1 (leaves 0 and 1 of the next chunk) a few phases before the chunk ends.
        constexpr int RH = 3;
        f8 kg0[NKD], kg1[NKD];
        f8 mp[RH][NP];
        f4 fS[NCT];
        load_kg(0, 0, SL::KG_OFF, kg0);
        load_kg(0, 1, SL::KG_OFF, kg1);
        lds_barrier();
        for (int c = 0; c < nchunks; ++c) {
            static_for<RH - 1>([&](auto Ic) {
                constexpr int Lt = 2 + decltype(Ic)::value;
                if constexpr (Lt < NB) load_mp(c, std::integral_constant<int, Lt>{}, mp[Lt % RH]);
            });
            lds_barrier();  // phase Z1: the state wavefront publishes S0
#pragma unroll
            for (int t = 0; t < NCT; ++t) fS[t] = sh_fS[c & 1][t][lane];
            {
                f32x4_t a0 = zero4(), a1 = zero4();
#pragma unroll
                for (int kk = 0; kk < NKD; ++kk) {
                    a0 = F::mma8(F::cat(fS[2 * kk], fS[2 * kk + 1]), kg0[kk], a0);
                    a1 = F::mma8(F::cat(fS[2 * kk], fS[2 * kk + 1]), kg1[kk], a1);
                }
                sh_acc[0][lane] = a0;
                sh_acc[1][lane] = a1;
            }
            lds_barrier();  // phase Z2
            static_for<NB>([&](auto Lc) {
                constexpr int L = decltype(Lc)::value;
                constexpr int Lt = L + 2;
                if constexpr (Lt + RH - 1 < NB)
                    load_mp(c, std::integral_constant<int, Lt + RH - 1>{}, mp[(Lt + RH - 1) % RH]);
                if constexpr (L == (NB > 4 ? NB - 5 : 0)) load_kg(c + 1, 0, SL::KG_OFF, kg0);
                if constexpr (L == (NB > 4 ? NB - 4 : 1)) load_kg(c + 1, 1, SL::KG_OFF, kg1);
                if constexpr (Lt < NB) {
                    f32x4_t a = sh_h[Lt & 3][lane];
#pragma unroll
                    for (int j = 0; j < help_pairs(Lt); ++j) a = F::mma8(sh_U[c & 1][j][lane], mp[Lt % RH][j], a);
                    sh_acc[Lt & 3][lane] = a;
                }
                lds_barrier();
            });
        }
        for (int k = 0; k < NB + 2; ++k) lds_barrier();  // the iteration after the last chunk
        return;
    }

    // ------------------------------------------------------------------------------------
    // Chain. Where several workgroups share a SIMD it wins instruction arbitration.
    __builtin_amdgcn_s_setprio(1);
    const f4 unit = F::unit(x, g);
    // Packed e and w: this tile's T rows of 8 values; rows at or past T read zero as well.
    const size_t pk0 = (size_t(bh) * (D / 8) + size_t(ct)) * size_t(T) * 8;
    const rsrc_t re = PK ? make_rsrc(e + pk0, unsigned(T) * 32u) : make_rsrc(e + tok0, tok_elems * 4u);
    const rsrc_t rwt = PK ? make_rsrc(w + pk0, unsigned(T) * 32u) : make_rsrc(w + tok0, tok_elems * 4u);
    const rsrc_t rv = make_rsrc(v + tok0, tok_elems * 2u);
    const rsrc_t rus = make_rsrc(SAVE ? u_save + tok0 : nullptr, SAVE ? tok_elems * 4u : 0u);
    const unsigned lo_pk = unsigned(8 * x + VC * g) * 4u;  // packed e, w: token x, group g
    auto load_leaf = [&](int ci, int L, LeafIn<bf16_t, VC> &in) {
        if constexpr (PK) {
            const unsigned so = unsigned(min(ci * C + 16 * L, T)) * 32u;
            in.ev = buf_load_fn<VC>(re, lo_pk, so);
            in.wv = buf_load_fn<VC>(rwt, lo_pk, so);
        } else {
            const unsigned so = trow(ci * C + 16 * L, 4u);
            in.ev = buf_load_fn<VC>(re, lo_f, so);
            in.wv = buf_load_fn<VC>(rwt, lo_f, so);
        }
        in.vv = RowV<bf16_t, VC>::load(rv, lo_q, trow(ci * C + 16 * L, 2u));
    };
    // Rings over leaves: the leaf inputs (slot = leaf mod RT, which divides the leaves per
    // chunk, so slots carry across chunks), loaded RT - 1 leaves ahead; the serial pair of
    // leaf L and, for odd L >= 3, the pair before it (used in phase L - 1), RC - 1 ahead.
    constexpr int RC = 4;                  // M pairs
    constexpr int RT = NB < 8 ? NB : 8;    // leaf inputs (divides NB)
    static_assert(NB % RT == 0, "ring");
    LeafIn<bf16_t, VC> in[RT];
    static_for<RT - 1>([&](auto Ic) {
        constexpr int L = decltype(Ic)::value;
        load_leaf(L / NB, L % NB, in[L]);
    });
    f8 mser[RC], mpre[RC];
    f32x4_t mdn[4];   // diagonal block rows of the next leaf
    f32x4_t accpre;   // right-hand side of the next leaf, without its serial pair
    f4 U1 = unit, U2 = unit;  // U of leaves L - 1 and L - 2
    lds_barrier();
    for (int c = 0; c < nchunks; ++c) {
        const int buf = c & 1;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) mdn[q4] = sh_md[buf][0][4 * x + q4];
        mser[1] = load_pair(c, SL::M_OFF, 1, ser_pair(1));
        mser[2] = load_pair(c, SL::M_OFF, 2, ser_pair(2));
        mpre[3] = load_pair(c, SL::M_OFF, 3, ser_pair(3) - 1);
        lds_barrier();  // phase Z1
        lds_barrier();  // phase Z2: H of leaves 0 and 1 are in LDS
        accpre = sh_acc[0][lane];
        static_for<NB>([&](auto Lc) {
            constexpr int L = decltype(Lc)::value;
            LeafIn<bf16_t, VC> &cin = in[L % RT];
            f32x4_t md[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) md[q4] = mdn[q4];
            // Loads for the phases ahead.
            if constexpr (L + 1 < NB) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) mdn[q4] = sh_md[buf][L + 1][4 * x + q4];
            }
            if constexpr (L + 3 < NB) mser[(L + 3) % RC] = load_pair(c, SL::M_OFF, L + 3, ser_pair(L + 3));
            if constexpr (L + 4 < NB && ((L + 4) & 1))
                mpre[(L + 4) % RC] = load_pair(c, SL::M_OFF, L + 4, ser_pair(L + 4) - 1);

            // ---- serial path ----
            f32x4_t acc = accpre;
            if constexpr (L > 0) {
                const f8 mp = mser[L % RC];
                if constexpr (L % 2 == 0) acc = F::mma8(F::cat(U2, U1), mp, acc);
                else acc = F::mma8(F::cat(U1, U1), mp, acc);
            }
            // The next leaf's right-hand side part from the helper (and for odd L + 1 the pair
            // of leaves L - 2, L - 1, whose U this wavefront holds).
            if constexpr (L + 1 < NB) {
                accpre = sh_acc[(L + 1) & 3][lane];
                if constexpr (((L + 1) & 1) && L + 1 >= 3) accpre = F::mma8(F::cat(U2, U1), mpre[(L + 1) % RC], accpre);
            }
            float ne[4] = {0.f, 0.f, 0.f, 0.f};
            float x0, x1, x2, x3;
            {
                float r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < VC; ++i) {
                    ne[i] = -cin.ev[i];
                    r[i] = fmaf(ne[i], acc[i], cin.wv[i] * RowV<bf16_t, VC>::get(cin.vv, i));
                }
                x0 = r[0]; x1 = r[1]; x2 = r[2]; x3 = r[3];
            }
            auto step = [&](auto Sc) {
                constexpr int St = decltype(Sc)::value;
                const float m = md[St / 4][St % 4];
                float n[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < VC; ++i) n[i] = ne[i] * m;
                subst_step<St, VC>(x0, x1, x2, x3, n[0], n[1], n[2], n[3]);
            };
            // Step 15 would update no token (M is strictly lower triangular): left out.
            static_for<15>([&](auto Sc) { step(std::integral_constant<int, decltype(Sc)::value>{}); });
            if constexpr (SAVE)
                RowV<float, VC>::store(rus, lo_f, trow(c * C + 16 * L, 4u), f32x4_t{x0, x1, x2, x3});
            const f4 U = F::pack(F::mma16_fresh(F::pack(f32x4_t{x0, x1, x2, x3}), unit));
            u_put(buf, L, U);
            U2 = U1;
            U1 = U;
            // Leaf L + RT - 1 into the slot of leaf L - 1.
            load_leaf(c + (L + RT - 1) / NB, (L + RT - 1) % NB, in[(L + RT - 1) % RT]);
            lds_barrier();
        });
    }
    for (int k = 0; k < NB + 2; ++k) lds_barrier();  // the iteration after the last chunk
}

// The readout of the split scan, O = (Qh*gamma) S0 + P U and the output gate, for every chunk
// at once. One workgroup per (batch*head, chunk, half of the value columns) stages the S0 and
// U fragments of its value tiles from the readout region into LDS; each of its four
// wavefronts then takes a quarter of the chunk's leaves (mirrored, so that every wavefront
// has about the same number of P blocks), loads each leaf's Qh*gamma and P operands once and
// applies them to every tile. Each output element takes the same products in the same order
// as the in-scan readout of the other scan (S0 first, then the leaf pairs in order), so the
// two give the same bits.
template <int D, int C, bool GATED>
__global__ __launch_bounds__(256) void chunk_readout_kernel(
    const float *__restrict__ og, bf16_t *__restrict__ o, const unsigned char *__restrict__ ws,
    const unsigned char *__restrict__ rd, int T, int H, int BH, int nchunks) {
    using SL = Slot<bf16_t, D, C>;
    using F = Frag<bf16_t>;
    using f8 = F::f8;
    constexpr int NB = C / 16, NKD = D / 32, NP = NB / 2;
    constexpr int NF = NKD + NP;   // fragments per 16-column tile
    constexpr int NQ = D / 32;     // tiles per workgroup (half of the head's D / 16)
    constexpr int NLW = NB / 4;    // leaves per wavefront
    constexpr unsigned OB = 2;
    constexpr size_t TB = readout_tile_bytes(D, C), RCB = readout_chunk_bytes(D, C);
    static_assert(TB == size_t(NF) * 1024 && (NQ * NF) % 4 == 0, "readout layout");
    __shared__ f8 sh[NQ * NF][64];

    // Workgroups go to the eight XCDs round-robin: ids 16n + x and 16n + 8 + x, the two halves
    // of one (batch*head, chunk), share XCD x and so the L2 that serves both their Qh*gamma and
    // P loads.
    const int id = blockIdx.x;
    const int hf = (id >> 3) & 1;
    const int unit = (id >> 4) * 8 + (id & 7);
    if (unit >= BH * nchunks) return;  // the whole workgroup, before any barrier
    const int bh = unit / nchunks, c = unit % nchunks;
    const int b = bh / H, h = bh % H;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, x = lane & 15, g = lane >> 4;
    const size_t HD = size_t(H) * D;
    const size_t ci = size_t(bh) * nchunks + c;
    const rsrc_t rws = make_rsrc(ws + ci * SL::BYTES, unsigned(SL::BYTES));
    const rsrc_t rrd = make_rsrc(rd + ci * RCB + size_t(hf) * NQ * TB, unsigned(NQ * TB));
#pragma unroll
    for (int n = 0; n < NQ * NF / 4; ++n) {
        const int f = n * 4 + wave;
        sh[f][lane] = F::bload8(rrd, unsigned(lane * 16), unsigned(f * 1024));
    }
    __syncthreads();

    // This head's tokens, from column 0; rows at or past T read zero, stores there are dropped.
    // Output lane (token x, group g) of tile p holds its rows 4g + i: columns 16p + 2g + i
    // (i < 2) and 16p + 8 + 2g + (i - 2) (i >= 2).
    const size_t tok0 = size_t(b) * T * HD + size_t(h) * D;
    const unsigned tok_elems = unsigned(size_t(T) * HD - size_t(h) * D);
    const rsrc_t ro_ = make_rsrc(o + tok0, tok_elems * 2u);
    const rsrc_t rog = make_rsrc(GATED ? og + tok0 : nullptr, GATED ? tok_elems * 4u : 0u);
    const unsigned lo_x = unsigned(x * HD + 2 * g);
    auto trow = [&](int t, unsigned es) { return unsigned(min(t, T)) * unsigned(HD) * es; };
    const unsigned lo_frag = unsigned(lane * 8) * OB;
    const unsigned lo_pair = unsigned((4 * x + g) * 8) * OB;

    struct Win {
        f8 qg[NKD];
        f8 pq[NP];
        f32x2_t oa[NQ], ob[NQ];  // output gate (GATED)
    };
    // Wavefront W takes leaves 4m + W (m even) and 4m + 3 - W (m odd). Its code is made for
    // its own leaves, so that no loop bound or load is a runtime branch (at a join the
    // wait-count pass would wait for every load in flight, the prefetches included).
    auto body = [&](auto Wc) {
        constexpr int W = decltype(Wc)::value;
        auto load_win = [&](auto Lc, Win &wn) {
            constexpr int L = decltype(Lc)::value;
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk)
                wn.qg[kk] = F::bload8(rws, lo_frag, unsigned(SL::QG_OFF + frag_idx(16 * L, 32 * kk, D) * OB));
#pragma unroll
            for (int j = 0; j <= L / 2; ++j)
                wn.pq[j] = F::bload8(rws, lo_pair, unsigned(SL::P_OFF + size_t(SL::prow(L) + j) * 512 * OB));
            if constexpr (GATED) {
                const unsigned row = trow(c * C + 16 * L, 4u);
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const unsigned col = unsigned(16 * (hf * NQ + q));
                    wn.oa[q] = __builtin_bit_cast(f32x2_t, buf_load8(rog, (lo_x + col) * 4u, row));
                    wn.ob[q] = __builtin_bit_cast(f32x2_t, buf_load8(rog, (lo_x + col + 8u) * 4u, row));
                }
            }
        };
        constexpr auto leaf = [](int m) { return (m & 1) ? 4 * m + 3 - W : 4 * m + W; };
        Win win[2];
        load_win(std::integral_constant<int, leaf(0)>{}, win[0]);
        static_for<NLW>([&](auto Mc) {
            constexpr int m = decltype(Mc)::value;
            constexpr int L = leaf(m);
            if constexpr (m + 1 < NLW) load_win(std::integral_constant<int, leaf(m + 1)>{}, win[(m + 1) & 1]);
            const Win &cw = win[m & 1];
            const unsigned row = trow(c * C + 16 * L, 1u);
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const unsigned col = unsigned(16 * (hf * NQ + q));
                f32x4_t ro = zero4();
#pragma unroll
                for (int kk = 0; kk < NKD; ++kk) ro = F::mma8(sh[q * NF + kk][lane], cw.qg[kk], ro);
#pragma unroll
                for (int j = 0; j <= L / 2; ++j) ro = F::mma8(sh[q * NF + NKD + j][lane], cw.pq[j], ro);
                f32x4_t va = {ro[0], ro[1], 0.f, 0.f}, vb = {ro[2], ro[3], 0.f, 0.f};
                if constexpr (GATED) {
                    va *= f32x4_t{cw.oa[q][0], cw.oa[q][1], 0.f, 0.f};
                    vb *= f32x4_t{cw.ob[q][0], cw.ob[q][1], 0.f, 0.f};
                }
                RowV<bf16_t, 2>::store(ro_, (lo_x + col) * 2u, row * 2u, va);
                RowV<bf16_t, 2>::store(ro_, (lo_x + col + 8u) * 2u, row * 2u, vb);
                // One tile's LDS operands in registers at a time: without this the scheduler
                // hoists every tile's reads and runs out of registers.
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    };
    switch (wave) {
        case 0: body(std::integral_constant<int, 0>{}); break;
        case 1: body(std::integral_constant<int, 1>{}); break;
        case 2: body(std::integral_constant<int, 2>{}); break;
        default: body(std::integral_constant<int, 3>{}); break;
    }
}

}  // namespace

hipError_t launch_chunk_scan_split_save(const void *v, const float *e, const float *w,
                                        const float *s0, float *s_out, float *u_out, float *states,
                                        int B, int T, int H, int d, int chunk, const void *workspace,
                                        hipStream_t stream) {
    const int nchunks = (T + chunk - 1) / chunk;
    const int BH = B * H;
    const int groups = (BH + 7) / 8;
    constexpr int VC = 2;
    unsigned char *ws = static_cast<unsigned char *>(const_cast<void *>(workspace));
    auto run = [&](auto dc, auto cc) {
        constexpr int D = decltype(dc)::value, C = decltype(cc)::value;
        hipLaunchKernelGGL((chunk_scan_split_kernel<D, C, VC, false, true>),
                           dim3(groups * 8 * (D / (4 * VC))), dim3(256), 0, stream,
                           static_cast<const bf16_t *>(v), e, w, s0, s_out, ws, nullptr, T, H, BH,
                           nchunks, u_out, states);
        return hipGetLastError();
    };
#define MUIR_SPLIT(D, C) \
    if (d == D && chunk == C) return run(std::integral_constant<int, D>{}, std::integral_constant<int, C>{});
    MUIR_SPLIT(64, 64) MUIR_SPLIT(64, 128) MUIR_SPLIT(64, 256)
    MUIR_SPLIT(128, 64) MUIR_SPLIT(128, 128) MUIR_SPLIT(128, 256)
#undef MUIR_SPLIT
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_scan_split(const void *v, const float *e, const float *w, const float *og,
                                   const float *s0, void *o, float *s_out, int B, int T, int H,
                                   int d, int chunk, void *workspace, hipStream_t stream,
                                   bool packed_ew) {
    const int nchunks = (T + chunk - 1) / chunk;
    const int BH = B * H;
    const int groups = (BH + 7) / 8;
    // Eight value columns per workgroup: sixteen (four per lane group) measured slower, the
    // chain's substitution then having twice the steps' instructions.
    constexpr int VC = 2;
    const dim3 block(256);
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    unsigned char *rd = ws + chunk_slots_bytes(B, T, H, d, chunk, true);
    auto run = [&](auto dc, auto cc) {
        constexpr int D = decltype(dc)::value, C = decltype(cc)::value;
        const dim3 grid(groups * 8 * (D / (4 * VC)));
        if (packed_ew)
            hipLaunchKernelGGL((chunk_scan_split_kernel<D, C, VC, true>), grid, block, 0, stream,
                               static_cast<const bf16_t *>(v), e, w, s0, s_out, ws, rd, T, H, BH,
                               nchunks);
        else
            hipLaunchKernelGGL((chunk_scan_split_kernel<D, C, VC, false>), grid, block, 0, stream,
                               static_cast<const bf16_t *>(v), e, w, s0, s_out, ws, rd, T, H, BH,
                               nchunks);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess || nchunks == 0) return err;
        const dim3 rgrid(unsigned((size_t(BH) * nchunks + 7) / 8 * 16));
        if (og)
            hipLaunchKernelGGL((chunk_readout_kernel<D, C, true>), rgrid, block, 0, stream, og,
                               static_cast<bf16_t *>(o), ws, rd, T, H, BH, nchunks);
        else
            hipLaunchKernelGGL((chunk_readout_kernel<D, C, false>), rgrid, block, 0, stream, og,
                               static_cast<bf16_t *>(o), ws, rd, T, H, BH, nchunks);
        return hipGetLastError();
    };
#define MUIR_SPLIT(D, C) \
    if (d == D && chunk == C) return run(std::integral_constant<int, D>{}, std::integral_constant<int, C>{});
    MUIR_SPLIT(64, 64) MUIR_SPLIT(64, 128) MUIR_SPLIT(64, 256)
    MUIR_SPLIT(128, 64) MUIR_SPLIT(128, 128) MUIR_SPLIT(128, 256)
#undef MUIR_SPLIT
    return hipErrorInvalidValue;
}

}  // namespace muir
