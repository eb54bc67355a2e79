// Chunkwise-parallel forward of the gated delta rule with matched-filter readout.
//
// The pages' stable large-chunk scheme (liuch.name summary of arXiv 2611.08376, third
// bullet; openai-hub news page, section on rewriting the long-sequence parallel
// algorithm for TPU): every decay that crosses a block boundary is split into two
// running products pivoted at that boundary, both in [0, 1], so nothing is ever
// divided by a cumulative decay; the intra-chunk unit lower-triangular system is solved
// by block-Neumann recursion whose off-diagonal products run on the matrix cores;
// chunks are chained by carrying the fp32 state.
//
// Per chunk of C tokens with start state S0 (all products run from the chunk start):
//   gamma_t = prod_{tau<=t} a_tau, beta_s = prod_{s<tau<=C} a_tau, Gamma_ts = prod_{s<tau<=t} a_tau
//   M_ts = sum_i k_ti Gamma_tsi k_si  (s < t)        P_ts = sum_i qh_ti Gamma_tsi k_si  (s <= t)
//   H = (K*gamma) S0;  (I + Diag(E_j) M) U_j = (W*V)_j - E_j * H_j   for each value column j
//   O = (Qh*gamma) S0 + P U;   S_C = Diag(gamma_C) S0 + (K*beta)^T U
// where qh = r * g * q. This follows from unrolling the token recurrence (decay, erase
// the decayed state's prediction for k_t under the value-channel gate e_t, write
// w_t * v_t, read with r * g_t * q_t). The state carry is evaluated in Horner form over
// 32-token leaf pairs: S <- Diag(pi_p) S + (K*beta')_p^T U_p per pair p, from S0, where
// pi_p is the pair's whole decay and beta'_s the decay from s to the end of its pair;
// this ends at the S_C above, with every factor in [0, 1].
//
// Two kernels:
//  * the parallel phase, one workgroup per (chunk, head, batch): decay products, the
//    operands K*gamma, Qh*gamma, (K*beta')^T, the pair decays, and the lower-triangular
//    M and P in 16x16 blocks. Off-diagonal block (bt, bs) is one MFMA product
//    (K_bs * sigma_bs * D)(K_bt * pi_bt)^T pivoted at the start of block bt: pi is the
//    running product inside bt from its start, sigma the running product inside bs after
//    s, D the product of the whole blocks in between. The 16x16 diagonal blocks recurse
//    further (pivots every 8, 4, 2, 1 tokens), each level one masked MFMA tile, so the
//    Gram work is all on the matrix cores. chunk_prepare_bf16_kernel streams the chunk
//    once for bf16 operands; chunk_prepare_kernel serves fp32 operands.
//  * chunk_scan_kernel, one workgroup per (batch x head, 16 or 8 value columns),
//    sequential over chunks (value columns are exactly independent). Its chain wavefront carries
//    the serial path: for leaf L (16 tokens) it subtracts E_L * (M_{L,<L} U_{<L}) from
//    the leaf's right-hand side on MFMA -- the off-diagonal products of the block-Neumann
//    recursion, grouped by the leaf they update -- then solves the 16x16 unit
//    lower-triangular leaf of every column by forward substitution, and carries the
//    state. Its readout wavefront computes O = (Qh*gamma) S0 + P U one chunk behind.
#include <type_traits>
#include <utility>

#include "chunk_layout.hpp"
#include "scan_leaf.hpp"
#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace muir {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr size_t kLdsBudget = 160 * 1024 - 1024;

// LDS of the prepare kernel: block totals, K*sigma (padded rows), per-wave tables.
template <typename OpT, int D, int C> struct PrepLds {
    static constexpr int DP = D + 4;                               // fp32 table row pitch
    static constexpr int DB = D + 16 / int(sizeof(OpT));           // operand row pitch
    static constexpr size_t PI = size_t(C / 16) * D * 4;
    static constexpr size_t BB = size_t(C) * DB * sizeof(OpT);
    static constexpr size_t SCR = size_t(16) * DP * 4;
    static constexpr int NW_FIT = int((kLdsBudget - PI - BB) / SCR);
    static constexpr int NW = NW_FIT < kWaves ? NW_FIT : kWaves;  // waves in the Gram phase
    static constexpr size_t BYTES = PI + BB + size_t(NW) * SCR;
    static_assert(NW >= 1, "LDS budget");
};

// ---------------------------------------------------------------------------------
// Phase P: decay products, pivoted operands and the intra-chunk Gram blocks.
// ---------------------------------------------------------------------------------
template <typename QT, typename OpT, int D, int C>
__global__ __launch_bounds__(kThreads) void chunk_prepare_kernel(
    const QT *__restrict__ q, const QT *__restrict__ k, const float *__restrict__ a,
    const float *__restrict__ g, const float *__restrict__ r, unsigned char *__restrict__ ws,
    int T, int H, int nchunks) {
    using SL = Slot<OpT, D, C>;
    using LY = PrepLds<OpT, D, C>;
    using MM = Mma<OpT>;
    constexpr int NB = C / 16;
    constexpr int NK = D / MM::KSTEP;  // k-steps over the channels
    constexpr int VALS = MM::VALS;
    constexpr int DP = LY::DP, DB = LY::DB;

    extern __shared__ __align__(16) unsigned char smem[];
    float *__restrict__ sh_pi = reinterpret_cast<float *>(smem);                   // [NB][D]
    OpT *__restrict__ sh_bb = reinterpret_cast<OpT *>(smem + LY::PI);             // [C][DB]
    float *__restrict__ sh_scr = reinterpret_cast<float *>(smem + LY::PI + LY::BB); // [NW][16][DP]

    const int ci = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    unsigned char *slot = ws + ((size_t(b) * H + h) * nchunks + ci) * SL::BYTES;
    OpT *__restrict__ gM = reinterpret_cast<OpT *>(slot + SL::M_OFF);
    OpT *__restrict__ gP = reinterpret_cast<OpT *>(slot + SL::P_OFF);
    OpT *__restrict__ gKg = reinterpret_cast<OpT *>(slot + SL::KG_OFF);
    OpT *__restrict__ gQg = reinterpret_cast<OpT *>(slot + SL::QG_OFF);
    OpT *__restrict__ gKbT = reinterpret_cast<OpT *>(slot + SL::KBT_OFF);
    float *__restrict__ gPP = reinterpret_cast<float *>(slot + SL::PP_OFF);
    float *__restrict__ gMD = reinterpret_cast<float *>(slot + SL::MD_OFF);

    const int t0 = ci * C;
    const int nreal = min(C, T - t0);
    const size_t HD = size_t(H) * D;
    const size_t base = (size_t(b) * T + t0) * HD + size_t(h) * D;  // token t0, channel 0
    const QT *__restrict__ qb = q + base;
    const QT *__restrict__ kb = k + base;
    const float *__restrict__ ab = a + base;
    const float *__restrict__ gb = g + base;
    const float *__restrict__ rh = r + size_t(h) * D;
    const int tid = threadIdx.x;

    // Padded tokens (t >= nreal) behave as a = 1, k = q = 0: they add nothing and
    // leave every decay product of the real tokens unchanged.

    // a1: whole-block decay products Pi_b = prod of the 16 decays of block b, per row.
    for (int idx = tid; idx < NB * D; idx += kThreads) {
        const int bb = idx / D, ch = idx % D;
        float av[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int tt = 16 * bb + t;
            av[t] = ab[min(tt, nreal - 1) * HD + ch];
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) av[t] = 16 * bb + t < nreal ? av[t] : 1.f;
        float p = 1.f;
#pragma unroll
        for (int t = 0; t < 16; ++t) p *= av[t];
        sh_pi[idx] = p;
    }
    lds_barrier();

    // a1/a2: per (block, row): pi (running product from the block start, inclusive) and
    // sigma (running product after s to the block end). gamma_t = G_b * pi_t with G_b the
    // product of the earlier blocks; beta_s = sigma_s * Gs_b with Gs_b the product of the
    // later blocks. All factors lie in [0, 1]; nothing is divided.
    for (int idx = tid; idx < NB * D; idx += kThreads) {
        const int bb = idx / D, ch = idx % D;
        float av[16], kv[16], qv[16];
        const float rc = rh[ch];
        float gv[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const size_t off = size_t(min(16 * bb + t, nreal - 1)) * HD + ch;
            av[t] = ab[off];
            kv[t] = elem<QT>::load(kb, off);
            qv[t] = elem<QT>::load(qb, off);
            gv[t] = gb[off];
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const bool in = 16 * bb + t < nreal;
            av[t] = in ? av[t] : 1.f;
            kv[t] = in ? kv[t] : 0.f;
            qv[t] = in ? rc * gv[t] * qv[t] : 0.f;
        }
        float G = 1.f;
        for (int x = 0; x < bb; ++x) G *= sh_pi[x * D + ch];
        // (K*beta)^T is pivoted at the end of the block pair: the second block's product
        // scales the first block's keys. The pair's whole product is stored for the scan.
        const float Gp = (bb & 1) ? 1.f : sh_pi[(bb + 1) * D + ch];
        if (bb & 1) gPP[(bb >> 1) * D + ch] = sh_pi[(bb - 1) * D + ch] * sh_pi[bb * D + ch];
        float pi = 1.f;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int tt = 16 * bb + t;
            pi *= av[t];
            const float gam = G * pi;
            gKg[frag_idx(tt, pair_perm(ch), D)] = MM::from_f32(kv[t] * gam);
            gQg[frag_idx(tt, pair_perm(ch), D)] = MM::from_f32(qv[t] * gam);
        }
        float kbt[16];
        float sig = 1.f;
#pragma unroll
        for (int t = 15; t >= 0; --t) {
            kbt[t] = kv[t] * (sig * Gp);
            sh_bb[(16 * bb + t) * DB + ch] = MM::from_f32(kv[t] * sig);
            sig *= av[t];
        }
#pragma unroll
        for (int t = 0; t < 16; t += 4)
            store4(gKbT + frag_idx(ch, pair_perm(16 * bb + t), C),
                   f32x4_t{kbt[t], kbt[t + 1], kbt[t + 2], kbt[t + 3]});
    }
    lds_barrier();

    // a3: Gram blocks. Wave w handles row blocks bt = w, w + NW, ... Tiles are computed
    // transposed (rows = earlier token s, columns = later token t) so that each lane
    // holds 4 consecutive s of one t and stores them as one vector.
    const int wave = tid >> 6, lane = tid & 63;
    if (wave >= LY::NW) return;
    float *__restrict__ scr = sh_scr + size_t(wave) * 16 * DP;
    const int tl = lane & 15;          // fragment row (token within the block)
    const int og = (lane >> 4) * 4;    // accumulator rows og..og+3 (token s)
    constexpr int CPL = D / 64;        // channels per lane for the running products

    for (int bt = wave; bt < NB; bt += LY::NW) {
        float av[CPL][16];
#pragma unroll
        for (int m = 0; m < CPL; ++m)
#pragma unroll
            for (int t = 0; t < 16; ++t)
                av[m][t] = ab[size_t(min(16 * bt + t, nreal - 1)) * HD + lane + 64 * m];
        float kf[NK][VALS], qf[NK][VALS];
        {
            const int tt = 16 * bt + tl;
            const size_t row = size_t(min(tt, nreal - 1)) * HD;
            float gv[NK][VALS], rv[NK][VALS];
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                const int c0 = kk * MM::KSTEP + MM::kidx(lane, 0);
                load_vec<VALS>(kb + row + c0, kf[kk]);
                load_vec<VALS>(qb + row + c0, qf[kk]);
                load_vec<VALS>(gb + row + c0, gv[kk]);
                load_vec<VALS>(rh + c0, rv[kk]);
            }
            const bool in = tt < nreal;
#pragma unroll
            for (int kk = 0; kk < NK; ++kk)
#pragma unroll
                for (int j = 0; j < VALS; ++j) {
                    kf[kk][j] = in ? kf[kk][j] : 0.f;
                    qf[kk][j] = in ? qf[kk][j] * gv[kk][j] * rv[kk][j] : 0.f;
                }
        }
#pragma unroll
        for (int m = 0; m < CPL; ++m)
#pragma unroll
            for (int t = 0; t < 16; ++t) av[m][t] = 16 * bt + t < nreal ? av[m][t] : 1.f;

        // Diagonal block: recursive pivots inside the block (node sizes 16, 8, 4, 2).
        f32x4_t leafM = zero4(), leafP = zero4();
#pragma unroll
        for (int half = 8; half >= 1; half >>= 1) {
            // Table: right half of each node -> prod from the pivot m up to t (inclusive);
            // left half -> prod after s up to m (exclusive of m).
#pragma unroll
            for (int m = 0; m < CPL; ++m) {
                const int ch = lane + 64 * m;
#pragma unroll
                for (int n0 = 0; n0 < 16; n0 += 2 * half) {
                    float run = 1.f;
#pragma unroll
                    for (int t = n0 + half; t < n0 + 2 * half; ++t) {
                        run *= av[m][t];
                        scr[t * DP + ch] = run;
                    }
                    run = 1.f;
#pragma unroll
                    for (int s = n0 + half - 1; s >= n0; --s) {
                        scr[s * DP + ch] = run;
                        run *= av[m][s];
                    }
                }
            }
            wave_lds_sync();
            f32x4_t accM = zero4(), accP = zero4();
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                float f[VALS], xk[VALS], xq[VALS];
                load_vec<VALS>(scr + tl * DP + kk * MM::KSTEP + MM::kidx(lane, 0), f);
#pragma unroll
                for (int j = 0; j < VALS; ++j) {
                    xk[j] = kf[kk][j] * f[j];
                    xq[j] = qf[kk][j] * f[j];
                }
                const auto fk = MM::pack(xk);
                const auto fq = MM::pack(xq);
                accM = MM::mma(fk, fk, accM);
                accP = MM::mma(fk, fq, accP);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = og + i, t = tl;
                const bool valid = ((t ^ s) < 2 * half) && (t & half) && !(s & half);
                leafM[i] += valid ? accM[i] : 0.f;
                leafP[i] += valid ? accP[i] : 0.f;
            }
            wave_lds_sync();
        }
        {   // diagonal of P: qh_t . k_t
            f32x4_t accD = zero4();
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) accD = MM::mma(MM::pack(kf[kk]), MM::pack(qf[kk]), accD);
#pragma unroll
            for (int i = 0; i < 4; ++i) leafP[i] += (og + i == tl) ? accD[i] : 0.f;
        }
        store4(gMD + size_t(bt) * 256 + tl * 16 + og, leafM);
        store4(gP + SL::blk(bt, bt, tl * 16 + og), leafP);
        store4(gM + SL::blk(bt, bt, tl * 16 + og), zero4());
        if ((bt & 1) == 0) store4(gP + SL::blk(bt, bt + 1, tl * 16 + og), zero4());
        if (bt == 0) continue;

        // Off-diagonal blocks (bt, bs), bs < bt, pivot at the start of block bt:
        // columns t: K_bt * pi_bt (and Qh_bt * pi_bt); rows s: K_bs * sigma_bs * D(bs, bt).
#pragma unroll
        for (int m = 0; m < CPL; ++m) {
            float run = 1.f;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                run *= av[m][t];
                scr[t * DP + lane + 64 * m] = run;
            }
        }
        wave_lds_sync();
        typename MM::frag fAk[NK], fAq[NK];
        float dm[NK][VALS];
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            float f[VALS], xk[VALS], xq[VALS];
            load_vec<VALS>(scr + tl * DP + kk * MM::KSTEP + MM::kidx(lane, 0), f);
#pragma unroll
            for (int j = 0; j < VALS; ++j) {
                xk[j] = kf[kk][j] * f[j];
                xq[j] = qf[kk][j] * f[j];
                dm[kk][j] = 1.f;
            }
            fAk[kk] = MM::pack(xk);
            fAq[kk] = MM::pack(xq);
        }
        wave_lds_sync();
        for (int bs = bt - 1; bs >= 0; --bs) {
            f32x4_t accM = zero4(), accP = zero4();
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                const int c0 = kk * MM::KSTEP + MM::kidx(lane, 0);
                float xb[VALS], pv[VALS];
                load_vec<VALS>(sh_bb + (16 * bs + tl) * DB + c0, xb);
                load_vec<VALS>(sh_pi + bs * D + c0, pv);
#pragma unroll
                for (int j = 0; j < VALS; ++j) {
                    xb[j] *= dm[kk][j];
                    dm[kk][j] *= pv[j];
                }
                const auto fb = MM::pack(xb);
                accM = MM::mma(fb, fAk[kk], accM);
                accP = MM::mma(fb, fAq[kk], accP);
            }
            store4(gM + SL::blk(bt, bs, tl * 16 + og), accM);
            store4(gP + SL::blk(bt, bs, tl * 16 + og), accP);
        }
    }
}

// ---------------------------------------------------------------------------------
// Phase S: sequential chunk scan.
// ---------------------------------------------------------------------------------

// ---------------------------------------------------------------------------------
// Phase P for bf16 operands: the same outputs in one streaming pass over the chunk.
// ---------------------------------------------------------------------------------
// Row scans over the 16 tokens of a block run on the 16-lane DPP rows. dpp_mv<CTRL>
// moves x across lanes with DPP control CTRL; lanes whose source lies outside their row
// read 0, and every use below replaces those lanes' value by a select.
template <int CTRL> __device__ __forceinline__ float dpp_mv(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL,
                                                              0xf, 0xf, true));
}
constexpr int kRowShl1 = 0x101, kRowShl4 = 0x104, kRowShr1 = 0x111, kRowShr4 = 0x114;
constexpr int quad_perm(int a, int b, int c, int d) { return a | (b << 2) | (c << 4) | (d << 6); }
constexpr int row_bcast(int n) { return 0x150 + n; }  // lane n of each row to the whole row

// LDS of the bf16 prepare kernel (bytes).
template <int D, int C> struct Prep2Lds {
    static constexpr int NB = C / 16, NG = D / 32;
    static constexpr size_t BB_OFF = 0;                                  // [C][D] K*sigma
    static constexpr size_t A_OFF = BB_OFF + size_t(C) * D * 2;          // [2][2][16][D] K*pi, Qh*pi
    static constexpr size_t KT_OFF = A_OFF + size_t(2) * 2 * 16 * D * 2; // [D][32] (K*beta')^T
    static constexpr size_t PI_OFF = KT_OFF + size_t(D) * 32 * 2;        // [NB][D] block decays
    static constexpr size_t FT_OFF = PI_OFF + size_t(NB) * D * 4;        // [NB][D] decay to the pair
    static constexpr size_t DG_OFF = FT_OFF + size_t(NB) * D * 4;        // [2][NG][2][64] partials
    static constexpr size_t BYTES = DG_OFF + size_t(2) * NG * 2 * 64 * 16;
};

// Operand rows in LDS ([row][D] bf16) are stored as D/8 chunks of 16 bytes, chunk c of
// row r at chunk position c ^ (r mod D/8): a 16-lane read of one chunk column over 16
// rows then touches 16 different bank groups.
template <int D> __device__ __forceinline__ int swz(int row, int chunk) {
    return row * D + 8 * (chunk ^ (row & (D / 8 - 1)));
}

// One workgroup of 4D threads (8 wavefronts at D = 128) per (chunk, head, batch), walking
// the chunk one leaf pair (two 16-token blocks) at a time with the next pair's inputs in
// flight. Wavefront w = h * NG + cg holds block h of the pair and channel group cg (32
// channels); lane 16 G + t holds token t of the block and channels 32cg + 4G + {0..3}
// and 32cg + 16 + 4G + {0..3} -- value j is channel 32cg + 4G + (j & 3) + 16 (j >> 2) --
// which are the operand positions 32cg + 8G .. + 7, so a thread's share of a Kg or Qg row
// is one 16-byte vector, and its eight values are its lane's share of a K = 32 matrix-core
// operand over the group's channels.
//
// Per pair p (blocks 2p, 2p + 1), for each channel:
//   pi_t   = prod of a from the block start to t (inclusive)     (row prefix scan)
//   sigma_s = prod of a after s to the block end                (row suffix scan)
//   Kg = k * G_b * pi, Qg = qh * G_b * pi with G_b the product of the earlier blocks;
//   (K*beta')^T = k * sigma * (decay of block 2p + 1 for block 2p), pivoted at the pair end;
//   the pair's decay; the diagonal blocks of M and P from the recursive pivots inside the
//   block (the scan's nested levels give every level's running products); the
//   off-diagonal blocks (bt, bs) against the K*sigma of all earlier blocks kept in LDS,
//   scaled by the decay of the whole blocks in between.
//
// LR: the decay a and the query gate g are not read but formed from the low-rank gate
// projection (the pages' fused rank-512 gate projection: openai-hub page, section on
// sensitivity-allocated gating, gate table): a = exp(-exp(z_decay . U_a + c_a)) and
// g = sigmoid(z_read . U_g + c_g), each a 16-channel x 16-token matrix-core tile per K = 32
// rank step, whose accumulator is exactly this thread's (token, 8 channels) share. The
// wavefront's up-projection rows stay in registers for the whole chunk; z rows (shared by
// every head) replace the fp32 a and g rows in the pair prefetch.
struct LowRankGates {
    const bf16_t *z;          // [B, T, 512]
    const bf16_t *Ua, *Ug;    // [H, D, 64], [H, D, 128]
    const float *ca, *cg;     // [H, D]
};
constexpr int kZRankAll = 512, kZOffDecay = 0, kZOffRead = 384;

// LDS of the LR variant, after the prepare's own: the head's U_g rows (and U_a's when they
// fit, else each wavefront keeps its four U_a fragments in registers), rows padded against
// bank conflicts, and the two offset vectors.
template <int D, int C> struct LrLds {
    static constexpr int UAP = 64 + 8, UGP = 128 + 8;  // row pitches, elements
    static constexpr size_t UG_OFF = Prep2Lds<D, C>::BYTES;
    static constexpr size_t CO_OFF = UG_OFF + size_t(D) * UGP * 2;  // [2][D] fp32: c_a, c_g
    static constexpr size_t UA_OFF = CO_OFF + size_t(2) * D * 4;
    static constexpr bool UA_IN_LDS = UA_OFF + size_t(D) * UAP * 2 <= 160 * 1024 - 1024;
    static constexpr size_t BYTES = UA_IN_LDS ? UA_OFF + size_t(D) * UAP * 2 : UA_OFF;
    static_assert(UA_OFF <= 160 * 1024 - 1024, "LDS budget");
};

// NORD: for a forward that keeps the state and does not read out (the backward pass's rerun):
// neither P nor Qh*gamma is formed, and q is not read.
template <int D, int C, bool LR, bool NORD = false>
__global__ __launch_bounds__(4 * D) void chunk_prepare_bf16_kernel(
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k, const float *__restrict__ a,
    const float *__restrict__ g, const float *__restrict__ r, LowRankGates lr,
    unsigned char *__restrict__ ws, int T, int H, int nchunks) {
    using SL = Slot<bf16_t, D, C>;
    using LY = Prep2Lds<D, C>;
    using F = Frag<bf16_t>;
    using f8 = F::f8;
    constexpr int NB = C / 16, NP = NB / 2, NG = D / 32, NW = 2 * NG, NT = 64 * NW;

    extern __shared__ __align__(16) unsigned char smem[];
    bf16_t *sh_bb = reinterpret_cast<bf16_t *>(smem + LY::BB_OFF);
    bf16_t *sh_A = reinterpret_cast<bf16_t *>(smem + LY::A_OFF);
    bf16_t *sh_kt = reinterpret_cast<bf16_t *>(smem + LY::KT_OFF);
    float *sh_pi = reinterpret_cast<float *>(smem + LY::PI_OFF);
    float *sh_ft = reinterpret_cast<float *>(smem + LY::FT_OFF);
    f32x4_t *sh_dg = reinterpret_cast<f32x4_t *>(smem + LY::DG_OFF);

    const int ci = blockIdx.x, hh = blockIdx.y, b = blockIdx.z;
    // The wavefront index is made visibly uniform: the row offsets of the buffer loads derive
    // from it and must be scalar (else every load becomes a loop over lanes' offsets).
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int hb = wave / NG, cg = wave % NG;  // block of the pair, channel group
    const int G = lane >> 4, t = lane & 15;
    const int pos0 = 32 * cg + 8 * G;          // operand positions of the thread
    const int chl = 32 * cg + 4 * G;           // channels chl + {0..3}, chl + 16 + {0..3}

    unsigned char *slot = ws + ((size_t(b) * H + hh) * nchunks + ci) * SL::BYTES;
    bf16_t *gM = reinterpret_cast<bf16_t *>(slot + SL::M_OFF);
    bf16_t *gP = reinterpret_cast<bf16_t *>(slot + SL::P_OFF);
    bf16_t *gKg = reinterpret_cast<bf16_t *>(slot + SL::KG_OFF);
    bf16_t *gQg = reinterpret_cast<bf16_t *>(slot + SL::QG_OFF);
    bf16_t *gKbT = reinterpret_cast<bf16_t *>(slot + SL::KBT_OFF);
    float *gPP = reinterpret_cast<float *>(slot + SL::PP_OFF);
    float *gMD = reinterpret_cast<float *>(slot + SL::MD_OFF);

    // Inputs through buffer resources covering tokens t0 .. t0 + nreal - 1 of this head:
    // padded tokens read zero (k = q = 0); their decay is set to 1 below.
    const int t0 = ci * C;
    const int nreal = min(C, T - t0);
    const size_t HD = size_t(H) * D;
    const size_t base = (size_t(b) * T + t0) * HD + size_t(hh) * D;
    const unsigned span = unsigned((size_t(nreal - 1) * HD + D));
    const rsrc_t rk = make_rsrc(k + base, span * 2u);
    const rsrc_t rq = make_rsrc(NORD ? nullptr : q + base, NORD ? 0u : span * 2u);
    const unsigned vo = unsigned(size_t(t) * HD + chl);
    // Gate rows: fp32 a and g, or (LR) the z rows of the decay and read slices, K = 32 rank
    // steps of 8 values per lane (lane (t, G): token t, ranks 32s + 8G .. + 7).
    struct GateIn {
        f32x4_t a0, a1, g0, g1;
    };
    struct GateInLR {
        f8 zd[2], zg[4];
    };
    struct In : std::conditional_t<LR, GateInLR, GateIn> {
        u16x4_t k0, k1, q0, q1;
    };
    const rsrc_t ra = make_rsrc(LR ? nullptr : a + base, LR ? 0u : span * 4u);
    const rsrc_t rg = make_rsrc(LR ? nullptr : g + base, LR ? 0u : span * 4u);
    const rsrc_t rz = make_rsrc(LR ? lr.z + (size_t(b) * T + t0) * kZRankAll : nullptr,
                                LR ? unsigned(nreal) * kZRankAll * 2u : 0u);
    auto load_in = [&](int p, In &in) {
        const unsigned row = unsigned(32 * p + 16 * hb) * unsigned(HD);
        if constexpr (LR) {
            const unsigned zrow = unsigned(32 * p + 16 * hb) * (kZRankAll * 2u);
            const unsigned zo = unsigned(t) * (kZRankAll * 2u) + unsigned(8 * G) * 2u;
#pragma unroll
            for (int s = 0; s < 2; ++s) in.zd[s] = F::bload8(rz, zo + unsigned(kZOffDecay + 32 * s) * 2u, zrow);
#pragma unroll
            for (int s = 0; s < 4; ++s) in.zg[s] = F::bload8(rz, zo + unsigned(kZOffRead + 32 * s) * 2u, zrow);
        } else {
            in.a0 = buf_load_f4(ra, vo * 4u, row * 4u);
            in.a1 = buf_load_f4(ra, vo * 4u + 64u, row * 4u);
            in.g0 = buf_load_f4(rg, vo * 4u, row * 4u);
            in.g1 = buf_load_f4(rg, vo * 4u + 64u, row * 4u);
        }
        in.k0 = Row4<bf16_t>::load(rk, vo * 2u, row * 2u);
        in.k1 = Row4<bf16_t>::load(rk, vo * 2u + 32u, row * 2u);
        if constexpr (!NORD) {
            in.q0 = Row4<bf16_t>::load(rq, vo * 2u, row * 2u);
            in.q1 = Row4<bf16_t>::load(rq, vo * 2u + 32u, row * 2u);
        } else {
            in.q0 = in.q1 = u16x4_t{0, 0, 0, 0};
        }
    };
    float rr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) rr[j] = r[size_t(hh) * D + chl + (j & 3) + 16 * (j >> 2)];
    // LR: the head's up-projection rows and offsets into LDS (U_a, when it does not fit,
    // is read per pair from the head's rows in memory, which stay in the L1 cache).
    using LL = LrLds<D, C>;
    if constexpr (LR) {
        bf16_t *sh_ug = reinterpret_cast<bf16_t *>(smem + LL::UG_OFF);
        float *sh_co = reinterpret_cast<float *>(smem + LL::CO_OFF);
        for (int n = tid; n < D * 16; n += NT) {  // U_g: D rows x 16 chunks of 8
            const int row = n >> 4, c8 = n & 15;
            *reinterpret_cast<f8 *>(sh_ug + row * LL::UGP + 8 * c8) =
                F::load8(lr.Ug + (size_t(hh) * D + row) * 128 + 8 * c8);
        }
        for (int n = tid; n < D; n += NT) {
            sh_co[n] = lr.ca[size_t(hh) * D + n];
            sh_co[D + n] = lr.cg[size_t(hh) * D + n];
        }
        if constexpr (LL::UA_IN_LDS) {
            bf16_t *sh_ua = reinterpret_cast<bf16_t *>(smem + LL::UA_OFF);
            for (int n = tid; n < D * 8; n += NT) {
                const int row = n >> 3, c8 = n & 7;
                *reinterpret_cast<f8 *>(sh_ua + row * LL::UAP + 8 * c8) =
                    F::load8(lr.Ua + (size_t(hh) * D + row) * 64 + 8 * c8);
            }
        }
        lds_barrier();
    }

    auto pack8 = [](const float (&x)[8]) {
        return F::cat(F::pack(f32x4_t{x[0], x[1], x[2], x[3]}), F::pack(f32x4_t{x[4], x[5], x[6], x[7]}));
    };
    auto ld8f = [](const float *p, float (&x)[8]) {
        const f32x4_t lo = *reinterpret_cast<const f32x4_t *>(p);
        const f32x4_t hi = *reinterpret_cast<const f32x4_t *>(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[i] = lo[i]; x[4 + i] = hi[i]; }
    };
    auto st8f = [](float *p, const float (&x)[8]) {
        *reinterpret_cast<f32x4_t *>(p) = f32x4_t{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<f32x4_t *>(p + 4) = f32x4_t{x[4], x[5], x[6], x[7]};
    };
    // Accumulator layout of the 16x16 products: lane (x = t, G) holds column t (the later
    // token) and rows s = 4G + i (the earlier token), stored row-major as [t][s].
    const unsigned blk_lo = unsigned(t * 16 + 4 * G);

    // (K*beta')^T of pair p from LDS to the workspace: thread -> (channel, 8 positions).
    auto kbt_out = [&](int p) {
        const int ch = tid >> 2, c4 = tid & 3;
        const f8 v = *reinterpret_cast<const f8 *>(sh_kt + ch * 32 + 8 * (c4 ^ ((ch >> 2) & 3)));
        *reinterpret_cast<f8 *>(gKbT + frag_idx(ch, 32 * p + 8 * c4, C)) = v;
    };
    // Decay between block bs and the start of pair p + 1, from the one to pair p.
    auto ft_update = [&](int p) {
        constexpr int Q = D / 4;
        for (int idx = tid; idx < (2 * p + 2) * Q; idx += NT) {
            const int bs = idx / Q, c4 = 4 * (idx % Q);
            const f32x4_t p0 = *reinterpret_cast<const f32x4_t *>(sh_pi + (2 * p) * D + c4);
            const f32x4_t p1 = *reinterpret_cast<const f32x4_t *>(sh_pi + (2 * p + 1) * D + c4);
            f32x4_t *dst = reinterpret_cast<f32x4_t *>(sh_ft + bs * D + c4);
            if (bs < 2 * p) *dst = *dst * (p0 * p1);
            else if (bs == 2 * p) *dst = p1;
            else *dst = f32x4_t{1.f, 1.f, 1.f, 1.f};
        }
    };

    In in;
    load_in(0, in);
    float Gp[8];  // product of the blocks before the current pair
#pragma unroll
    for (int j = 0; j < 8; ++j) Gp[j] = 1.f;

    for (int p = 0; p < NP; ++p) {
        const int bt = 2 * p + hb;
        // ------------------------------ phase 1 ------------------------------
        if (p > 0) {
            kbt_out(p - 1);
            ft_update(p - 1);
        }
        float av[8], kv[8], qh[8];
        {
            const bool real = 16 * bt + t < nreal;
            f32x4_t a0, a1, g0, g1;
            if constexpr (LR) {
                const bf16_t *sh_ug = reinterpret_cast<const bf16_t *>(smem + LL::UG_OFF);
                const float *sh_co = reinterpret_cast<const float *>(smem + LL::CO_OFF);
                f32x4_t y[4];
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    y[ct] = *reinterpret_cast<const f32x4_t *>(sh_co + chl + 16 * ct);
                    y[2 + ct] = *reinterpret_cast<const f32x4_t *>(sh_co + D + chl + 16 * ct);
                    const int row = 32 * cg + 16 * ct + t;
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        f8 ua;
                        if constexpr (LL::UA_IN_LDS)
                            ua = *reinterpret_cast<const f8 *>(reinterpret_cast<const bf16_t *>(smem + LL::UA_OFF) +
                                                               row * LL::UAP + 32 * s + 8 * G);
                        else
                            ua = F::load8(lr.Ua + (size_t(hh) * D + row) * 64 + 32 * s + 8 * G);
                        y[ct] = F::mma8(ua, in.zd[s], y[ct]);
                    }
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        y[2 + ct] = F::mma8(*reinterpret_cast<const f8 *>(sh_ug + row * LL::UGP + 32 * s + 8 * G),
                                            in.zg[s], y[2 + ct]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a0[i] = gate_decay(y[0][i]);
                    a1[i] = gate_decay(y[1][i]);
                    g0[i] = gate_sigmoid(y[2][i]);
                    g1[i] = gate_sigmoid(y[3][i]);
                }
            } else {
                a0 = in.a0; a1 = in.a1; g0 = in.g0; g1 = in.g1;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[i] = real ? a0[i] : 1.f;
                av[4 + i] = real ? a1[i] : 1.f;
                kv[i] = bf16_to_f32(in.k0[i]);
                kv[4 + i] = bf16_to_f32(in.k1[i]);
                qh[i] = rr[i] * g0[i] * bf16_to_f32(in.q0[i]);
                qh[4 + i] = rr[4 + i] * g1[i] * bf16_to_f32(in.q1[i]);
            }
        }
        if (p + 1 < NP) load_in(p + 1, in);

        // Prefix products inside aligned segments of 2, 4, 8 and 16 tokens (each level
        // multiplies the upper half of a segment by the last value of its lower half).
        // Every DPP move runs with all lanes active (a lane can only read a lane that
        // executes the move), and the lane's choice is a select afterwards.
        float R2[8], R4[8], R8[8], pi[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float x = av[j], y;
            y = dpp_mv<kRowShr1>(x);
            x *= (t & 1) ? y : 1.f;
            R2[j] = x;
            y = dpp_mv<quad_perm(0, 1, 1, 1)>(x);
            x *= (t & 2) ? y : 1.f;
            R4[j] = x;
            y = dpp_mv<kRowShr4>(dpp_mv<quad_perm(3, 3, 3, 3)>(x));
            x *= (t & 4) ? y : 1.f;
            R8[j] = x;
            y = dpp_mv<row_bcast(7)>(x);
            x *= (t & 8) ? y : 1.f;
            pi[j] = x;
        }
        // Suffix products likewise; the exclusive suffix inside a segment of size n is the
        // inclusive one of the next token (1 at the segment's last token). Level tables:
        // f_n(t) = prefix from the segment start (t in an upper half of a 2n-node) or
        // exclusive suffix to the segment end (t in a lower half).
        float f8t[8], f4t[8], f2t[8], f1t[8], sig[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float x = av[j], y, l;
            f1t[j] = (t & 1) ? x : 1.f;
            y = dpp_mv<kRowShl1>(x);
            x *= (t & 1) ? 1.f : y;  // S2
            l = dpp_mv<kRowShl1>(x);
            f2t[j] = (t & 2) ? R2[j] : ((t & 1) ? 1.f : l);
            y = dpp_mv<quad_perm(2, 2, 2, 2)>(x);
            x *= (t & 2) ? 1.f : y;  // S4
            l = dpp_mv<kRowShl1>(x);
            f4t[j] = (t & 4) ? R4[j] : (((t & 3) == 3) ? 1.f : l);
            y = dpp_mv<kRowShl4>(dpp_mv<quad_perm(0, 0, 0, 0)>(x));
            x *= (t & 4) ? 1.f : y;  // S8
            l = dpp_mv<kRowShl1>(x);
            f8t[j] = (t & 8) ? R8[j] : (((t & 7) == 7) ? 1.f : l);
            y = dpp_mv<row_bcast(8)>(x);
            x *= (t & 8) ? 1.f : y;  // S16
            y = dpp_mv<kRowShl1>(x);
            sig[j] = (t == 15) ? 1.f : y;
        }

        // LDS: K*sigma of the block (all later pairs), K*pi and Qh*pi (this pair's
        // off-diagonal blocks), the block's decay (lane t = 15 holds it in pi).
        {
            float x[8], y[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = kv[j] * sig[j];
            *reinterpret_cast<f8 *>(sh_bb + swz<D>(16 * bt + t, 4 * cg + G)) = pack8(x);
#pragma unroll
            for (int j = 0; j < 8; ++j) { x[j] = kv[j] * pi[j]; y[j] = qh[j] * pi[j]; }
            *reinterpret_cast<f8 *>(sh_A + (hb * 2 + 0) * 16 * D + swz<D>(t, 4 * cg + G)) = pack8(x);
            if constexpr (!NORD) *reinterpret_cast<f8 *>(sh_A + (hb * 2 + 1) * 16 * D + swz<D>(t, 4 * cg + G)) = pack8(y);
            if (t == 15) st8f(sh_pi + bt * D + pos0, pi);
        }
        // This wavefront's share (its 32 channels) of the diagonal blocks of M and P: one
        // masked product per recursion level, plus the diagonal of P.
        {
            f32x4_t lm = zero4(), lp = zero4();
            auto level = [&](const float (&f)[8], int half) {
                float x[8], y[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) { x[j] = kv[j] * f[j]; y[j] = qh[j] * f[j]; }
                const f8 fk = pack8(x), fq = pack8(y);
                const f32x4_t am = F::mma8(fk, fk, zero4());
                const f32x4_t ap = NORD ? zero4() : F::mma8(fk, fq, zero4());
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s = 4 * G + i;
                    const bool valid = ((t ^ s) < 2 * half) && (t & half) && !(s & half);
                    lm[i] += valid ? am[i] : 0.f;
                    lp[i] += valid ? ap[i] : 0.f;
                }
            };
            level(f8t, 8);
            level(f4t, 4);
            level(f2t, 2);
            level(f1t, 1);
            if constexpr (!NORD) {
                const f32x4_t ad = F::mma8(pack8(kv), pack8(qh), zero4());
#pragma unroll
                for (int i = 0; i < 4; ++i) lp[i] += (4 * G + i == t) ? ad[i] : 0.f;
            }
            sh_dg[((hb * NG + cg) * 2 + 0) * 64 + lane] = lm;
            sh_dg[((hb * NG + cg) * 2 + 1) * 64 + lane] = lp;
        }
        lds_barrier();

        // ------------------------------ phase 2 ------------------------------
        float P0[8], P1[8];  // decays of blocks 2p and 2p + 1 at the thread's positions
        ld8f(sh_pi + (2 * p) * D + pos0, P0);
        ld8f(sh_pi + (2 * p + 1) * D + pos0, P1);
        {
            float x[8], y[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float gam = Gp[j] * (hb ? P0[j] : 1.f) * pi[j];
                x[j] = kv[j] * gam;
                y[j] = qh[j] * gam;
            }
            const size_t row = frag_idx(16 * bt + t, pos0, D);
            *reinterpret_cast<f8 *>(gKg + row) = pack8(x);
            if constexpr (!NORD) *reinterpret_cast<f8 *>(gQg + row) = pack8(y);
            // (K*beta')^T into LDS: channel row, position 8 (t / 4) + 4 hb + t % 4 of the
            // pair (the 32-group order), 16-byte chunks rotated by (channel / 4) mod 4.
            const int pp = 8 * (t >> 2) + 4 * hb + (t & 3);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int ch = chl + (j & 3) + 16 * (j >> 2);
                const float kb = kv[j] * sig[j] * (hb ? 1.f : P1[j]);
                sh_kt[ch * 32 + 8 * ((pp >> 3) ^ ((ch >> 2) & 3)) + (pp & 7)] = bf16_t{f32_to_bf16(kb)};
            }
            if (hb == 1 && t == 15) {
                *reinterpret_cast<f32x4_t *>(gPP + p * D + chl) =
                    f32x4_t{P0[0] * P1[0], P0[1] * P1[1], P0[2] * P1[2], P0[3] * P1[3]};
                *reinterpret_cast<f32x4_t *>(gPP + p * D + chl + 16) =
                    f32x4_t{P0[4] * P1[4], P0[5] * P1[5], P0[6] * P1[6], P0[7] * P1[7]};
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) Gp[j] *= P0[j] * P1[j];
        }
        if (cg == 0) {
            // Diagonal blocks: sum of the channel groups' shares.
            f32x4_t lm = zero4(), lp = zero4();
#pragma unroll
            for (int c = 0; c < NG; ++c) {
                lm += sh_dg[((hb * NG + c) * 2 + 0) * 64 + lane];
                lp += sh_dg[((hb * NG + c) * 2 + 1) * 64 + lane];
            }
            *reinterpret_cast<f32x4_t *>(gMD + size_t(bt) * 256 + blk_lo) = lm;
            if constexpr (!NORD) store4(gP + SL::blk(bt, bt, blk_lo), lp);
            // The pair slots the scan reads whole: M's diagonal block (its products use
            // the fp32 copy above) and, for even bt, P's block (bt, bt + 1) above the
            // diagonal hold zeros.
            store4(gM + SL::blk(bt, bt, blk_lo), zero4());
            if (!NORD && (bt & 1) == 0) store4(gP + SL::blk(bt, bt + 1, blk_lo), zero4());
        }
        // Off-diagonal blocks of the pair: (2p, bs < 2p) and (2p + 1, bs <= 2p). Rows s:
        // K*sigma of block bs times the decay of the whole blocks between bs and bt;
        // columns t: K*pi (Qh*pi) of block bt. The two blocks of one bs < 2p are done
        // together by one wavefront, bs dealt to the wavefronts in turn.
        if (wave < 2 * p + 1) {
            f8 ak[2][NG], aq[2][NG];
            float pb0[NG][8];  // decay of block 2p at the operand positions of this lane
#pragma unroll
            for (int kk = 0; kk < NG; ++kk) {
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    ak[h2][kk] = *reinterpret_cast<const f8 *>(sh_A + (h2 * 2 + 0) * 16 * D + swz<D>(t, 4 * kk + G));
                    if constexpr (!NORD)
                        aq[h2][kk] = *reinterpret_cast<const f8 *>(sh_A + (h2 * 2 + 1) * 16 * D + swz<D>(t, 4 * kk + G));
                }
                ld8f(sh_pi + (2 * p) * D + 32 * kk + 8 * G, pb0[kk]);
            }
            // Both blocks (2p, bs) and (2p + 1, bs) from one read of block bs's K*sigma:
            // decay F[bs] for the even row, F[bs] times the decay of block 2p for the odd.
            auto block_pair = [&](int bs) {
                f32x4_t am0 = zero4(), ap0 = zero4(), am1 = zero4(), ap1 = zero4();
#pragma unroll
                for (int kk = 0; kk < NG; ++kk) {
                    const f8 xb = *reinterpret_cast<const f8 *>(sh_bb + swz<D>(16 * bs + t, 4 * kk + G));
                    float dm[8], x0[8], x1[8];
                    ld8f(sh_ft + bs * D + 32 * kk + 8 * G, dm);
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        x0[j] = bf16_to_f32(xb[j]) * dm[j];
                        x1[j] = x0[j] * pb0[kk][j];
                    }
                    const f8 fb0 = pack8(x0), fb1 = pack8(x1);
                    am0 = F::mma8(fb0, ak[0][kk], am0);
                    am1 = F::mma8(fb1, ak[1][kk], am1);
                    if constexpr (!NORD) {
                        ap0 = F::mma8(fb0, aq[0][kk], ap0);
                        ap1 = F::mma8(fb1, aq[1][kk], ap1);
                    }
                }
                store4(gM + SL::blk(2 * p, bs, blk_lo), am0);
                store4(gM + SL::blk(2 * p + 1, bs, blk_lo), am1);
                if constexpr (!NORD) {
                    store4(gP + SL::blk(2 * p, bs, blk_lo), ap0);
                    store4(gP + SL::blk(2 * p + 1, bs, blk_lo), ap1);
                }
            };
            // Block (2p + 1, 2p): no whole block in between.
            auto block_adjacent = [&]() {
                f32x4_t am = zero4(), ap = zero4();
#pragma unroll
                for (int kk = 0; kk < NG; ++kk) {
                    const f8 xb = *reinterpret_cast<const f8 *>(sh_bb + swz<D>(16 * (2 * p) + t, 4 * kk + G));
                    am = F::mma8(xb, ak[1][kk], am);
                    if constexpr (!NORD) ap = F::mma8(xb, aq[1][kk], ap);
                }
                store4(gM + SL::blk(2 * p + 1, 2 * p, blk_lo), am);
                if constexpr (!NORD) store4(gP + SL::blk(2 * p + 1, 2 * p, blk_lo), ap);
            };
            for (int n = wave; n < 2 * p; n += NW) block_pair(n);
            if (2 * p % NW == wave) block_adjacent();
        }
        lds_barrier();
    }
    kbt_out(NP - 1);
}

// The scan: one workgroup of two wavefronts per (batch, head, 4 VC value columns),
// sequential over chunks and over the 16-token leaves inside each chunk. Value columns
// are exactly independent, so nothing is shared between workgroups. For leaf L of a
// chunk with start state S0:
//   acc = (K*gamma)_L S0 + sum_{l<L} M_{L,l} U_l          (matrix cores)
//   (I + Diag(e) M_LL) u = w*v - e*acc                      (forward substitution)
//   S_C = Diag(gamma_C) S0 + sum_L (K*beta)_L^T U_L         (matrix cores)
//   O_L = (Qh*gamma)_L S0 + sum_{l<=L} P_{L,l} U_l          (matrix cores)
// The chain wavefront (wave 0) computes the first three; only M_{L,L-1} U_{L-1}, the
// substitution and one transpose lie on its serial path, the other products of each
// leaf are issued while the substitution runs. The readout wavefront (wave 1) computes
// O one chunk behind, from the chunk's S0 and U that the chain leaves in LDS; the two
// meet at one barrier per chunk. Splitting the operand streams between two wavefronts
// doubles the loads each chain keeps in flight (vector-memory loads return in order, so
// one wavefront's prefetch depth is bounded by what it can hold).
//
// Layouts: "row layout" (lane (t, g): token t, tile rows 4g..4g+3) is what the
// substitution works in, and is the accumulator layout of products whose B operand rows
// are tokens. U is kept as an operand with rows = tile rows and values = tokens 4g..4g+3
// of the leaf; an mma4 against the identity turns a row-layout u into it. The state is
// kept as accumulators with rows = channels, columns = tile rows.
//
// Value columns per workgroup: the matrix-core tiles are 16 rows wide, and tile row
// 4G + i holds value column j0 + VC G + i for i < VC (VC = 4 or 2). The other tile rows
// stay exactly zero (zero initial state, zero solution), so each lane's substitution
// handles only VC columns. Narrower tiles give more workgroups with shorter serial chains
// for the same products; they pay off when 16-column tiles leave compute units idle.
//
// GATED: the output-gate epilogue, o <- o * og elementwise with og [B, T, H, dv] fp32 (the
// output gate of the pages' gate table, applied as the readout is stored).
//
// LRS: e and w are not read but formed inside the kernel from the low-rank gate projection
// (the pages' fused rank-512 gate projection: openai-hub page, section on
// sensitivity-allocated gating, gate table): e = sigmoid(z_erase . U_e + c_e) and
// w = sigmoid(z_write . U_w + c_w). A third wavefront makes them one chunk ahead of the
// chain into LDS, one matrix-core tile per 16-token leaf and rank step (rows = the tile's
// value columns, columns = tokens, so its accumulator is the chain's row layout), in the
// same order of operations as the standalone gate kernel, so the values are the same bits.
// With GATED, the same wavefront also forms the output gate og = sigmoid(z_output . U_o +
// c_o) of the chain's current chunk into LDS, where the readout takes it a chunk later.
// Built for 16-column tiles only.
struct ScanGates {
    const bf16_t *z;          // [B, T, 512]
    const bf16_t *Ue, *Uw;    // [H, D, 64], [H, D, 128]
    const float *ce, *cw;     // [H, D]
    const bf16_t *Uo;         // [H, D, 128] (LRS with GATED)
    const float *co;          // [H, D]
};
constexpr int kZOffErase = 64, kZOffOutput = 128, kZOffWrite = 256;
// What the forward keeps for the backward pass (SAVE): u = b - e * p of every token in fp32,
// [B, T, H, D] like v, and the state at the start of every 64-token block and at the end,
// fp32 [B * H][ceil(T / 64) + 1][D][D], whatever the forward's own chunk size.
struct ScanSave {
    float *u;
    float *states;
};
template <typename QT, typename OpT, int D, int C, bool GATED, int VC, bool LRS, bool SAVE = false>
__global__ __launch_bounds__(LRS ? 192 : 128) void chunk_scan_kernel(
    const QT *__restrict__ v, const float *__restrict__ e, const float *__restrict__ w,
    const float *__restrict__ og, const float *__restrict__ s0, QT *__restrict__ o,
    float *__restrict__ s_out, const unsigned char *__restrict__ ws, ScanGates sg, int T, int H,
    int BH, int nchunks, ScanSave sv = {}) {
    using SL = Slot<OpT, D, C>;
    using F = Frag<OpT>;
    using f4 = typename F::f4;
    using f8 = typename F::f8;
    constexpr int NB = C / 16;    // leaves per chunk
    constexpr int NCT = D / 16;   // 16-channel tiles of the state
    constexpr int NKD = D / 32;   // K = 32 steps over the channels
    constexpr int HALF = NCT / 2; // state tiles updated per leaf

    // Chunk hand-over from the chain to the readout wavefront, double-buffered by chunk
    // parity: S0 as operands and every leaf's U, both in the lane order of the operands.
    __shared__ f4 sh_fS[2][NCT][64];
    // U of every leaf of the chunk, interleaved by leaf pairs: leaves 2j and 2j + 1 of a
    // lane are one 8-value K = 32 operand.
    __shared__ f8 sh_U[2][NB / 2][64];
    // Decay of every leaf pair of a chunk, per channel, double-buffered by chunk parity;
    // staged by the readout wavefront one chunk ahead of the chain.
    constexpr int NP = NB / 2;
    __shared__ __align__(16) float sh_pp[2][NP][D];
    // The chunk's fp32 diagonal blocks of M (row-major [t][s] per leaf), staged the same
    // way: whole 16-byte pieces, so each load of the stager uses full cache lines.
    __shared__ __align__(16) f32x4_t sh_md[2][NB][64];
    // LRS: e and w of every leaf of a chunk in the chain's row layout, double-buffered by
    // chunk parity.
    static_assert(!LRS || VC == 4, "the in-kernel gates run with 16-column tiles");
    __shared__ __align__(16) f32x4_t sh_ew[LRS ? 2 : 1][LRS ? NB : 1][2][64];
    // LRS with GATED: the output gate of every leaf of a chunk in the readout's row layout,
    // double-buffered by chunk parity.
    constexpr bool OGL = LRS && GATED;
    __shared__ __align__(16) f32x4_t sh_og[OGL ? 2 : 1][OGL ? NB : 1][64];

    // Workgroups are dealt to the eight XCDs round-robin; the value tiles of one head
    // get ids that are equal mod 8, so they share an XCD and its L2.
    constexpr int NVT = D / (4 * VC);  // value tiles per head
    const int id = blockIdx.x;
    const int bh = (id >> 3) / NVT * 8 + (id & 7);
    const int ct = (id >> 3) % NVT;
    if (bh >= BH) return;
    const int b = bh / H, h = bh % H;
    const int j0 = 4 * VC * ct;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63, x = lane & 15, g = lane >> 4;
    const size_t HD = size_t(H) * D;
    // Tile row x of the state holds value column j0 + VC (x / 4) + x % 4, if x % 4 < VC.
    const bool col_ok = (x & 3) < VC;
    const unsigned lo_st = unsigned(4 * g * D + VC * (x >> 2) + (x & 3));  // state [4g][column]
    auto u_put = [&](int buf, int L, f4 u) {
        reinterpret_cast<f4 *>(&sh_U[buf][L >> 1][lane])[L & 1] = u;
    };
    auto u_pair = [&](int buf, int j) { return sh_U[buf][j][lane]; };
    const float *s0h = s0 ? s0 + size_t(bh) * D * D + j0 : nullptr;
    float *south = s_out ? s_out + size_t(bh) * D * D + j0 : nullptr;

    // SAVE: the state at every 64-token block start and at the end, [BH][n64 + 1][D][D].
    static_assert(!SAVE || C % 64 == 0, "saved states are 64 tokens apart");
    const int n64 = (T + 63) / 64;
    float *svst = SAVE ? sv.states + size_t(bh) * (n64 + 1) * D * D + j0 : nullptr;
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

    // Per-lane byte offsets (each load adds one to a uniform base and offset).
    constexpr unsigned OB = sizeof(OpT);
    const unsigned lo_pair = unsigned((4 * x + g) * 8) * OB;  // block pair: row x, cols 4g..
    const unsigned lo_frag = unsigned(lane * 8) * OB;        // lane's share of an operand fragment
    const unsigned lo_f = unsigned(x * HD + VC * g) * 4u;            // e, w: token x, group g
    const unsigned lo_q = unsigned(x * HD + VC * g) * unsigned(sizeof(QT));  // v, o

    // Descriptors (loop-invariant). The workspace one covers this head's chunk slots;
    // a chunk index past the end is clamped to the last chunk (prefetches read valid,
    // unused data). The token ones cover rows 0..T-1 of this head and column tile of one
    // [B, T, H, *] tensor, from (b, 0, h, j0): the end of row T-1's tile lies inside, row
    // T starts outside, so tokens at or past T read zero and their stores are dropped.
    // The bounds check includes the scalar offset, which carries the token row.
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

    if constexpr (LRS) {
        if (wave == 2) {
            // ---------------- gate wavefront: e, w of chunk p + 1 in phase p ----------------
            using F8 = Frag<bf16_t>;
            using g8 = typename F8::f8;
            const rsrc_t rz = make_rsrc(sg.z + size_t(b) * T * kZRankAll, unsigned(size_t(T) * kZRankAll * 2));
            // Up-projection rows as A operands (lane (x, g): column j0 + x, ranks 32s + 8g ..
            // + 7), and the offsets as the accumulators' start (lane (t, g): columns
            // j0 + 4g .. + 3).
            g8 ue[2], uw[4];
#pragma unroll
            for (int s = 0; s < 2; ++s) ue[s] = F8::load8(sg.Ue + (size_t(h) * D + j0 + x) * 64 + 32 * s + 8 * g);
#pragma unroll
            for (int s = 0; s < 4; ++s) uw[s] = F8::load8(sg.Uw + (size_t(h) * D + j0 + x) * 128 + 32 * s + 8 * g);
            f32x4_t ce4, cw4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ce4[i] = sg.ce[size_t(h) * D + j0 + 4 * g + i];
                cw4[i] = sg.cw[size_t(h) * D + j0 + 4 * g + i];
            }
            // z rows of four leaves: erase slice (2 rank steps) and write slice (4).
            constexpr int NL = NB < 4 ? NB : 4;
            struct ZGroup {
                g8 ze[NL][2], zw[NL][4];
            };
            auto load_group = [&](int ci, int grp, ZGroup &zg) {
#pragma unroll
                for (int l = 0; l < NL; ++l) {
                    const int t = ci * C + 16 * (grp * NL + l) + x;
                    const unsigned zoff = unsigned(min(t, T)) * (kZRankAll * 2u) + 16u * unsigned(g);
#pragma unroll
                    for (int s = 0; s < 2; ++s) zg.ze[l][s] = F8::bload8(rz, zoff + unsigned(kZOffErase + 32 * s) * 2u, 0u);
#pragma unroll
                    for (int s = 0; s < 4; ++s) zg.zw[l][s] = F8::bload8(rz, zoff + unsigned(kZOffWrite + 32 * s) * 2u, 0u);
                }
            };
            auto make_group = [&](int ci, int grp, const ZGroup &zg) {
#pragma unroll
                for (int l = 0; l < NL; ++l) {
                    const int L = grp * NL + l;
                    const bool real = ci * C + 16 * L + x < T;  // tokens past T: e = w = 0
                    f32x4_t ye = ce4, yw = cw4;
#pragma unroll
                    for (int s = 0; s < 2; ++s) ye = F8::mma8(ue[s], zg.ze[l][s], ye);
#pragma unroll
                    for (int s = 0; s < 4; ++s) yw = F8::mma8(uw[s], zg.zw[l][s], yw);
                    f32x4_t ev, wv;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        ev[i] = real ? gate_sigmoid(ye[i]) : 0.f;
                        wv[i] = real ? gate_sigmoid(yw[i]) : 0.f;
                    }
                    sh_ew[ci & 1][L][0][lane] = ev;
                    sh_ew[ci & 1][L][1][lane] = wv;
                }
            };
            auto make_chunk = [&](int ci) {
                ZGroup zg[2];
                load_group(ci, 0, zg[0]);
                static_for<NB / NL>([&](auto Gc) {
                    constexpr int grp = decltype(Gc)::value;
                    if constexpr (grp + 1 < NB / NL) load_group(ci, grp + 1, zg[(grp + 1) & 1]);
                    make_group(ci, grp, zg[grp & 1]);
                });
            };
            // The output gate (GATED): rows of U_o and c_o as for the write gate, z's output
            // slice (4 rank steps) per leaf.
            g8 uo[OGL ? 4 : 1];
            f32x4_t co4 = zero4();
            if constexpr (OGL) {
#pragma unroll
                for (int s = 0; s < 4; ++s) uo[s] = F8::load8(sg.Uo + (size_t(h) * D + j0 + x) * 128 + 32 * s + 8 * g);
#pragma unroll
                for (int i = 0; i < 4; ++i) co4[i] = sg.co[size_t(h) * D + j0 + 4 * g + i];
            }
            struct OGroup {
                g8 zo[NL][4];
            };
            auto load_ogroup = [&](int ci, int grp, OGroup &zg) {
#pragma unroll
                for (int l = 0; l < NL; ++l) {
                    const int t = ci * C + 16 * (grp * NL + l) + x;
                    const unsigned zoff = unsigned(min(t, T)) * (kZRankAll * 2u) + 16u * unsigned(g);
#pragma unroll
                    for (int s = 0; s < 4; ++s) zg.zo[l][s] = F8::bload8(rz, zoff + unsigned(kZOffOutput + 32 * s) * 2u, 0u);
                }
            };
            auto make_og = [&](int ci) {
                OGroup zg[2];
                load_ogroup(ci, 0, zg[0]);
                static_for<NB / NL>([&](auto Gc) {
                    constexpr int grp = decltype(Gc)::value;
                    if constexpr (grp + 1 < NB / NL) load_ogroup(ci, grp + 1, zg[(grp + 1) & 1]);
#pragma unroll
                    for (int l = 0; l < NL; ++l) {
                        f32x4_t yo = co4;
#pragma unroll
                        for (int s = 0; s < 4; ++s) yo = F8::mma8(uo[s], zg[grp & 1].zo[l][s], yo);
                        f32x4_t ov;
#pragma unroll
                        for (int i = 0; i < 4; ++i) ov[i] = gate_sigmoid(yo[i]);
                        sh_og[ci & 1][grp * NL + l][lane] = ov;
                    }
                });
            };
            make_chunk(0);
            lds_barrier();
            for (int p = 0; p <= nchunks; ++p) {
                if (p + 1 < nchunks) make_chunk(p + 1);
                if constexpr (OGL) {
                    if (p < nchunks) make_og(p);  // read out in phase p + 1
                }
                lds_barrier();
            }
            return;
        }
    }

    if (wave == 1) {
        // ---------------- readout wavefront: O of chunk p - 1 in phase p ----------------
        const rsrc_t ro_ = make_rsrc(SAVE ? nullptr : o + tok0, SAVE ? 0u : tok_elems * unsigned(sizeof(QT)));
        const rsrc_t rog = make_rsrc(GATED && !OGL ? og + tok0 : nullptr, GATED && !OGL ? tok_elems * 4u : 0u);
        // Operands of leaf L's readout: (Qh*gamma)_L and P_{L,0..L} in block pairs (and the
        // output gate rows), loaded one leaf ahead.
        struct RWin {
            f8 qg[NKD];
            f8 pq[NB / 2];
            f32x4_t og;
        };
        auto load_rwin = [&](int ci, int L, RWin &wn) {
            load_kg(ci, L, SL::QG_OFF, wn.qg);
#pragma unroll
            for (int j = 0; j <= L / 2; ++j) wn.pq[j] = load_pair(ci, SL::P_OFF, L, j);
            if constexpr (GATED && !OGL) wn.og = buf_load_fn<VC>(rog, lo_f, trow(ci * C + 16 * L, 4u));
        };
        // SAVE (the backward's rerun) keeps u and the states and does not read out: the
        // wavefront only stages the chain's pair decays and diagonal blocks.
        RWin rw[2];
        if constexpr (!SAVE) load_rwin(0, 0, rw[0]);
        // Pair decays of chunk ci into sh_pp[ci & 1] (NP * D floats, four per lane and
        // step).
        constexpr int PP4 = NP * D / 4;
        constexpr int PPN = (PP4 + 63) / 64;
        auto load_ppt = [&](int ci, f32x4_t (&dst)[PPN]) {
#pragma unroll
            for (int n = 0; n < PPN; ++n)
                if (n * 64 + lane < PP4)
                    dst[n] = buf_load_f4(rws, unsigned(16 * (n * 64 + lane)), wsoff(ci, SL::PP_OFF));
        };
        auto put_ppt = [&](int ci, const f32x4_t (&src)[PPN]) {
            f32x4_t *dst = reinterpret_cast<f32x4_t *>(&sh_pp[ci & 1][0][0]);
#pragma unroll
            for (int n = 0; n < PPN; ++n)
                if (n * 64 + lane < PP4) dst[n * 64 + lane] = src[n];
        };
        f32x4_t ppt[PPN];
        load_ppt(0, ppt);
        put_ppt(0, ppt);
        // Diagonal blocks of chunk ci (NB KiB): lane l holds floats 4l .. 4l+3 of each leaf.
        f32x4_t mdt[NB];
        auto load_mdt = [&](int ci) {
#pragma unroll
            for (int L = 0; L < NB; ++L) mdt[L] = buf_load_f4(rws, unsigned(16 * lane), wsoff(ci, SL::MD_OFF + L * 1024));
        };
        auto put_mdt = [&](int ci) {
#pragma unroll
            for (int L = 0; L < NB; ++L) sh_md[ci & 1][L][lane] = mdt[L];
        };
        load_mdt(0);
        put_mdt(0);
        lds_barrier();
        for (int p = 0; p <= nchunks; ++p) {
            if (p + 1 < nchunks) {
                load_ppt(p + 1, ppt);
                load_mdt(p + 1);
            }
            if (!SAVE && p >= 1) {
                const int ci = p - 1;
                const int buf = ci & 1;
                f4 fS[NCT];
#pragma unroll
                for (int c = 0; c < NCT; ++c) fS[c] = sh_fS[buf][c][lane];

                static_for<NB>([&](auto Lc) {
                    constexpr int L = decltype(Lc)::value;
                    RWin &cw = rw[L & 1];
                    // The next leaf's operands (the next chunk's first leaf after the last).
                    load_rwin(L + 1 < NB ? ci : ci + 1, (L + 1) % NB, rw[(L + 1) & 1]);

                    f32x4_t ro = zero4();
#pragma unroll
                    for (int kk = 0; kk < NKD; ++kk)
                        ro = F::mma8(F::cat(fS[2 * kk], fS[2 * kk + 1]), cw.qg[kk], ro);
#pragma unroll
                    for (int l = 0; l <= L; l += 2) {
                        ro = F::mma8(u_pair(buf, l / 2), cw.pq[l / 2], ro);
                    }
                    if constexpr (OGL) ro *= sh_og[buf][L][lane];
                    else if constexpr (GATED) ro *= cw.og;
                    RowV<QT, VC>::store(ro_, lo_q, trow(ci * C + 16 * L, unsigned(sizeof(QT))), ro);
                });
            }
            if (p + 1 < nchunks) {
                put_ppt(p + 1, ppt);
                put_mdt(p + 1);
            }
            lds_barrier();
        }
        return;
    }

    // ---------------- chain wavefront ----------------
    // The chain is the critical path: where several workgroups share a SIMD, its wavefront
    // wins instruction arbitration over the others' readout and gate wavefronts.
    __builtin_amdgcn_s_setprio(1);
    // State: S[c][i] = state[16c + 4g + i][j0 + x].
    f32x4_t S[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[c][i] = s0h && col_ok ? s0h[size_t(16 * c + i) * D + lo_st] : 0.f;

    const f4 unit = F::unit(x, g);
    const rsrc_t re = make_rsrc(e + tok0, tok_elems * 4u);
    const rsrc_t rwt = make_rsrc(w + tok0, tok_elems * 4u);
    const rsrc_t rv = make_rsrc(v + tok0, tok_elems * unsigned(sizeof(QT)));
    const rsrc_t rus = make_rsrc(SAVE ? sv.u + tok0 : nullptr, SAVE ? tok_elems * 4u : 0u);
    auto save_state = [&](int ci) {
        if (col_ok) {
            float *dst = svst + size_t(ci) * D * D;
#pragma unroll
            for (int c = 0; c < NCT; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[size_t(16 * c + i) * D + lo_st] = S[c][i];
        }
    };

    auto load_leaf = [&](int ci, int L, LeafIn<QT, VC> &in) {
        const unsigned so = trow(ci * C + 16 * L, 4u);
        if constexpr (!LRS) {
            in.ev = buf_load_fn<VC>(re, lo_f, so);
            in.wv = buf_load_fn<VC>(rwt, lo_f, so);
        }
        in.vv = RowV<QT, VC>::load(rv, lo_q, trow(ci * C + 16 * L, unsigned(sizeof(QT))));
    };
    auto load_kbt = [&](int ci, int pair, int c) {
        return F::bload8(rws, lo_frag, wsoff(ci, SL::KBT_OFF + frag_idx(16 * c, 32 * pair, C) * OB));
    };
    // Decay over leaf pair `pair` of chunk ci of the rows of state tile c.
    auto lds_pp = [&](int ci, int pair, int c) {
        return *reinterpret_cast<const f32x4_t *>(&sh_pp[ci & 1][pair][16 * c + 4 * g]);
    };

    // Matrix-core operands of leaf L's window, loaded at the start of leaf L - 1:
    //   kg    (K*gamma) of leaf L + 1 (for its H), or of leaf 0 of the next chunk
    //   mp    M_{L+1,l} (l <= L) in block pairs: the right-hand side of leaf L + 1
    //   kbt   (K*beta)^T of leaf pair (L-2, L-1) for half of the state tiles, pivoted
    //         at the pair's end
    struct Win {
        f8 kg[NKD], kbt[HALF];
        f8 mp[NB / 2];
    };
    auto load_win = [&](int ci, int L, Win &wn) {
        if (L + 1 < NB) load_kg(ci, L + 1, SL::KG_OFF, wn.kg);
        else load_kg(ci + 1, 0, SL::KG_OFF, wn.kg);
        if (L + 1 < NB) {
#pragma unroll
            for (int j = 0; j <= L / 2; ++j) wn.mp[j] = load_pair(ci, SL::M_OFF, L + 1, j);
        }
        if (L >= 2) {
#pragma unroll
            for (int c = 0; c < HALF; ++c) wn.kbt[c] = load_kbt(ci, (L - 2) / 2, c + (L & 1) * HALF);
        }
    };

    // Leaf inputs: in[L & 1] holds leaf L and is refilled with leaf L + 2 once leaf L is
    // solved. Window operands: win[L & 1] (see Win).
    LeafIn<QT, VC> in[2];
    load_leaf(0, 0, in[0]);
    load_leaf(0, 1, in[1]);
    Win win[2];
    f8 kgH[NKD];  // (K*gamma) of leaf 0 of the current chunk
    load_kg(0, 0, SL::KG_OFF, kgH);
    load_win(0, 0, win[0]);
    f8 kbtLast[NCT];  // (K*beta)^T of the chunk's last leaf pair

    lds_barrier();  // the first chunk's pair decays are in LDS
    for (int p = 0; p <= nchunks; ++p) {
        if (p < nchunks) {
            const int ci = p;
            const int buf = ci & 1;
            // Chunk start: S holds S0. Its operand copy serves the whole chunk (and the
            // readout, through LDS); S itself becomes the accumulator of S_C, carried in
            // Horner form: per leaf pair, S <- Diag(pair decay) S + (K*beta')^T U, with
            // beta' pivoted at the pair's end, which ends at Diag(gamma_C) S0 +
            // (K*beta)^T U.
            f4 fS[NCT];
#pragma unroll
            for (int c = 0; c < NCT; ++c) {
                fS[c] = F::pack(S[c]);
                sh_fS[buf][c][lane] = fS[c];
            }
            if constexpr (SAVE) save_state(ci * (C / 64));
            f32x4_t acc = zero4();  // right-hand-side accumulator of the current leaf
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) acc = F::mma8(F::cat(fS[2 * kk], fS[2 * kk + 1]), kgH[kk], acc);

            f4 Ulast = F::unit(x, g);  // U of the previous leaf
            f4 Uprev = Ulast;          // and of the one before
            static_for<NB>([&](auto Lc) {
                constexpr int L = decltype(Lc)::value;
                constexpr bool more = L + 1 < NB;
                Win &cw = win[L & 1];
                Win &nw = win[(L + 1) & 1];
                LeafIn<QT, VC> &cin = in[L & 1];
                // Row t of the leaf's diagonal M block, from LDS (staged a chunk ahead).
                f32x4_t md[4];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) md[q4] = sh_md[buf][L][4 * x + q4];
                // The leaf's erase and write gates (LRS: from the gate wavefront, in LDS).
                f32x4_t evv = cin.ev, wvv = cin.wv;
                if constexpr (LRS) {
                    evv = sh_ew[buf][L][0][lane];
                    wvv = sh_ew[buf][L][1][lane];
                }
                const int ciN = more ? ci : ci + 1;  // chunk of leaf L + 1
                constexpr int LN = (L + 1) % NB;     // leaf L + 1 within it

                // ---- serial path: last M term and right-hand side ----
                if constexpr (L > 0) {
                    // The block pair of row L that holds M_{L,L-1}, from the window loaded for
                    // leaf L - 1, as one K = 32 product: for even L it also carries
                    // M_{L,L-2} U_{L-2} (left out of the precomputed part); for odd L its
                    // second block is the diagonal block, which is stored as zeros.
                    const f8 mpair = win[(L - 1) & 1].mp[(L - 1) / 2];
                    if constexpr (L % 2 == 0) acc = F::mma8(F::cat(Uprev, Ulast), mpair, acc);
                    else acc = F::mma8(F::cat(Ulast, Ulast), mpair, acc);
                }
                load_win(ciN, LN, nw);
                // Tokens past T read e = w = v = 0 (outside the resource): r = 0, u = 0. Tile
                // rows past VC in each group hold no column: their u is zero.
                float ne[4] = {0.f, 0.f, 0.f, 0.f};
                float x0, x1, x2, x3;
                {
                    float r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < VC; ++i) {
                        ne[i] = -evv[i];
                        r[i] = fmaf(ne[i], acc[i], wvv[i] * RowV<QT, VC>::get(cin.vv, i));
                    }
                    x0 = r[0]; x1 = r[1]; x2 = r[2]; x3 = r[3];
                }
                // Coefficients of step s: -e_c * M_LL[t][s], formed just before the step.
                auto step = [&](auto Sc) {
                    constexpr int St = decltype(Sc)::value;
                    const float m = md[St / 4][St % 4];
                    float n[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < VC; ++i) n[i] = ne[i] * m;
                    subst_step<St, VC>(x0, x1, x2, x3, n[0], n[1], n[2], n[3]);
                };

                static_for<4>([&](auto Sc) { step(std::integral_constant<int, decltype(Sc)::value>{}); });

                // ---- window, part 1: H of the next leaf ----
                f32x4_t accN = zero4();
                if constexpr (more) {
#pragma unroll
                    for (int kk = 0; kk < NKD; ++kk)
                        accN = F::mma8(F::cat(fS[2 * kk], fS[2 * kk + 1]), cw.kg[kk], accN);
                } else {
#pragma unroll
                    for (int kk = 0; kk < NKD; ++kk) kgH[kk] = cw.kg[kk];
                }

                static_for<4>([&](auto Sc) { step(std::integral_constant<int, 4 + decltype(Sc)::value>{}); });

                // ---- window, part 2: earlier leaves' terms, state carry of a leaf pair ----
                if constexpr (more) {
                    // Earlier leaves in whole pairs; the pair holding leaf L - 1 (or L alone)
                    // is the next leaf's serial product.
#pragma unroll
                    for (int j = 0; j < L / 2; ++j) accN = F::mma8(u_pair(buf, j), cw.mp[j], accN);
                }
                if constexpr (L >= 2) {
                    constexpr int p0 = (L - 2) & ~1;
                    const f8 u2 = u_pair(buf, p0 / 2);
#pragma unroll
                    for (int c = 0; c < HALF; ++c) {
                        constexpr int off = (L & 1) * HALF;
                        S[c + off] = F::mma8(cw.kbt[c], u2, S[c + off] * lds_pp(ci, p0 / 2, c + off));
                    }
                }
                // SAVE inside a chunk: after this update of leaf 4 q + 1 every tile has taken
                // the leaf pairs of tokens 0 .. 64 q - 1 and no later one (the lower tiles take
                // pair 2 q at leaf 4 q + 2), so S is the state at the chunk's 64 q-th token. A
                // boundary past the sequence goes to the final state's slot, which the final
                // state overwrites.
                if constexpr (SAVE && L % 4 == 1 && L >= 5) {
                    constexpr int q = (L - 1) / 4;
                    save_state(ci * C + 64 * q < T ? ci * (C / 64) + q : n64);
                }
                if constexpr (!more) {
#pragma unroll
                    for (int c = 0; c < NCT; ++c) kbtLast[c] = load_kbt(ci, NB / 2 - 1, c);
                }

                // Step 15 would update no token (M is strictly lower triangular): left out.
                static_for<7>([&](auto Sc) { step(std::integral_constant<int, 8 + decltype(Sc)::value>{}); });

                if constexpr (SAVE)
                    RowV<float, VC>::store(rus, lo_f, trow(ci * C + 16 * L, 4u), f32x4_t{x0, x1, x2, x3});
                // ---- u -> U operand (transpose on the matrix cores), hand-over ----
                Uprev = Ulast;
                Ulast = F::pack(F::mma16_fresh(F::pack(f32x4_t{x0, x1, x2, x3}), unit));
                u_put(buf, L, Ulast);
                if constexpr (more) acc = accN;
                load_leaf(L + 2 < NB ? ci : ci + 1, (L + 2) % NB, cin);  // leaf L + 2
            });
            // Chunk end: the last leaf pair's share of the state.
            {
                const f8 u2 = F::cat(Uprev, Ulast);
#pragma unroll
                for (int c = 0; c < NCT; ++c) S[c] = F::mma8(kbtLast[c], u2, S[c] * lds_pp(ci, NP - 1, c));
            }
        }
        lds_barrier();
    }

    if (south && col_ok) {
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) south[size_t(16 * c + i) * D + lo_st] = S[c][i];
    }
    if constexpr (SAVE) save_state(n64);
}

template <typename QT, typename OpT, int D, int C>
hipError_t prepare_typed(const void *q, const void *k, const float *a, const float *g,
                         const float *r, const LowRankGates &lr, int B, int T, int H,
                         void *workspace, hipStream_t stream) {
    const int nchunks = (T + C - 1) / C;
    if (nchunks == 0) return hipSuccess;
    if constexpr (std::is_same_v<OpT, bf16_t>) {
        const size_t lds = lr.z ? LrLds<D, C>::BYTES : Prep2Lds<D, C>::BYTES;
        auto kern = lr.z ? chunk_prepare_bf16_kernel<D, C, true> : chunk_prepare_bf16_kernel<D, C, false>;
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(lds));
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(kern, dim3(nchunks, H, B), dim3(4 * D), lds, stream,
                           static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(k), a, g,
                           r, lr, static_cast<unsigned char *>(workspace), T, H, nchunks);
        return hipGetLastError();
    } else {
        using LY = PrepLds<OpT, D, C>;
        auto kern = chunk_prepare_kernel<QT, OpT, D, C>;
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(LY::BYTES));
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(kern, dim3(nchunks, H, B), dim3(kThreads), LY::BYTES, stream,
                           static_cast<const QT *>(q), static_cast<const QT *>(k), a, g, r,
                           static_cast<unsigned char *>(workspace), T, H, nchunks);
        return hipGetLastError();
    }
}

template <typename QT, typename OpT, int D, int C, int VC, bool LRS = false>
hipError_t scan_vc(const void *v, const float *e, const float *w, const float *og,
                   const float *s0, void *o, float *s_out, int B, int T, int H,
                   const void *workspace, hipStream_t stream, ScanGates sg = {}) {
    const int nchunks = (T + C - 1) / C;
    const int BH = B * H;
    const int groups = (BH + 7) / 8;
    const dim3 grid(groups * 8 * (D / (4 * VC)));
    const dim3 block(LRS ? 192 : 128);
    // The output-gate epilogue: og read from memory, or (LRS) formed from z in the kernel.
    if (LRS ? sg.Uo != nullptr : og != nullptr) {
        hipLaunchKernelGGL((chunk_scan_kernel<QT, OpT, D, C, true, VC, LRS>), grid, block, 0,
                           stream, static_cast<const QT *>(v), e, w, og, s0, static_cast<QT *>(o),
                           s_out, static_cast<const unsigned char *>(workspace), sg, T, H, BH, nchunks);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((chunk_scan_kernel<QT, OpT, D, C, false, VC, LRS>), grid, block, 0, stream,
                       static_cast<const QT *>(v), e, w, og, s0, static_cast<QT *>(o), s_out,
                       static_cast<const unsigned char *>(workspace), sg, T, H, BH, nchunks);
    return hipGetLastError();
}

// Value columns per scan workgroup (4 VC): eight when that still gives at most one
// workgroup per compute unit, else sixteen (bf16 operands; the fp32 path always takes
// sixteen). A second chain on a compute unit costs more than the narrower tiles save.
// Both widths give the same results bit for bit: every value column goes through the same
// operations.
constexpr int kScanCUs = 256;
bool scan_narrow_tiles(int B, int H, int d) { return size_t(B) * H * (d / 8) <= size_t(kScanCUs); }

template <typename QT, typename OpT, int D, int C>
hipError_t scan_typed(const void *v, const float *e, const float *w, const float *og,
                      const float *s0, void *o, float *s_out, int B, int T, int H,
                      void *workspace, hipStream_t stream, bool packed_ew) {
    if constexpr (std::is_same_v<QT, bf16_t>) {
        if (split_scan_applies(B, H, D))
            return launch_chunk_scan_split(v, e, w, og, s0, o, s_out, B, T, H, D, C, workspace, stream,
                                           packed_ew);
    }
    if (packed_ew) return hipErrorInvalidValue;  // only the split scan reads packed gates
    if constexpr (std::is_same_v<QT, bf16_t>) {
        if (scan_narrow_tiles(B, H, D))
            return scan_vc<QT, OpT, D, C, 2>(v, e, w, og, s0, o, s_out, B, T, H, workspace, stream);
    }
    return scan_vc<QT, OpT, D, C, 4>(v, e, w, og, s0, o, s_out, B, T, H, workspace, stream);
}

}  // namespace

hipError_t launch_chunk_prepare(const void *q, const void *k, const float *a, const float *g,
                                const float *r, int B, int T, int H, int d, int chunk, bool bf16,
                                void *workspace, hipStream_t stream) {
    const LowRankGates none{nullptr, nullptr, nullptr, nullptr, nullptr};
#define MUIR_PREP(D, C)                                                                        \
    if (d == D && chunk == C)                                                                  \
        return bf16 ? prepare_typed<bf16_t, bf16_t, D, C>(q, k, a, g, r, none, B, T, H,         \
                                                          workspace, stream)                   \
                    : prepare_typed<float, float, D, C>(q, k, a, g, r, none, B, T, H,           \
                                                        workspace, stream);
    MUIR_PREP(64, 64) MUIR_PREP(64, 128) MUIR_PREP(64, 256)
    MUIR_PREP(128, 64) MUIR_PREP(128, 128) MUIR_PREP(128, 256)
#undef MUIR_PREP
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_prepare_state(const void *k, const float *a, const float *g, const float *r,
                                      int B, int T, int H, int d, int chunk, void *workspace,
                                      hipStream_t stream) {
    const LowRankGates none{nullptr, nullptr, nullptr, nullptr, nullptr};
    const int nchunks = (T + chunk - 1) / chunk;
    if (nchunks == 0) return hipSuccess;
    auto run = [&](auto dc, auto cc) {
        constexpr int D = decltype(dc)::value, C = decltype(cc)::value;
        auto kern = chunk_prepare_bf16_kernel<D, C, false, true>;
        constexpr size_t lds = Prep2Lds<D, C>::BYTES;
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(kern, dim3(nchunks, H, B), dim3(4 * D), lds, stream,
                           static_cast<const bf16_t *>(nullptr), static_cast<const bf16_t *>(k), a, g, r,
                           none, static_cast<unsigned char *>(workspace), T, H, nchunks);
        return hipGetLastError();
    };
    using I = std::integral_constant<int, 64>;
    using J = std::integral_constant<int, 128>;
    using K = std::integral_constant<int, 256>;
    if (d == 64 && chunk == 64) return run(I{}, I{});
    if (d == 64 && chunk == 128) return run(I{}, J{});
    if (d == 64 && chunk == 256) return run(I{}, K{});
    if (d == 128 && chunk == 64) return run(J{}, I{});
    if (d == 128 && chunk == 128) return run(J{}, J{});
    if (d == 128 && chunk == 256) return run(J{}, K{});
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_prepare_lowrank(const void *q, const void *k, const void *z,
                                        const void *Ua, const void *Ug, const float *ca,
                                        const float *cg, const float *r, int B, int T, int H,
                                        int d, int chunk, void *workspace, hipStream_t stream) {
    const LowRankGates lr{static_cast<const bf16_t *>(z), static_cast<const bf16_t *>(Ua),
                          static_cast<const bf16_t *>(Ug), ca, cg};
#define MUIR_PREP(D, C)                                                                        \
    if (d == D && chunk == C)                                                                  \
        return prepare_typed<bf16_t, bf16_t, D, C>(q, k, nullptr, nullptr, r, lr, B, T, H,      \
                                                   workspace, stream);
    MUIR_PREP(64, 64) MUIR_PREP(64, 128) MUIR_PREP(64, 256)
    MUIR_PREP(128, 64) MUIR_PREP(128, 128) MUIR_PREP(128, 256)
#undef MUIR_PREP
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_scan(const void *v, const float *e, const float *w, const float *og,
                             const float *s0, void *o, float *s_out, int B, int T, int H, int d,
                             int chunk, bool bf16, void *workspace, hipStream_t stream,
                             bool packed_ew) {
#define MUIR_SCAN(D, C)                                                                        \
    if (d == D && chunk == C)                                                                  \
        return bf16 ? scan_typed<bf16_t, bf16_t, D, C>(v, e, w, og, s0, o, s_out, B, T, H,      \
                                                       workspace, stream, packed_ew)           \
                    : scan_typed<float, float, D, C>(v, e, w, og, s0, o, s_out, B, T, H,        \
                                                     workspace, stream, packed_ew);
    MUIR_SCAN(64, 64) MUIR_SCAN(64, 128) MUIR_SCAN(64, 256)
    MUIR_SCAN(128, 64) MUIR_SCAN(128, 128) MUIR_SCAN(128, 256)
#undef MUIR_SCAN
    return hipErrorInvalidValue;
}

// With 16-column tiles and chunks of up to 128 tokens: there the gates' LDS (two chunks of
// e and w) keeps two workgroups per compute unit, as many as the registers allow. Larger
// chunks would halve that; with 8-column tiles (one workgroup per compute unit) the gate
// wavefront's z loads slowed the chain by more than the separate gate pass costs.
template <typename QT, int D, int C>
hipError_t scan_save_typed(const void *v, const float *e, const float *w, const float *s0,
                           void *o, float *s_out, const ScanSave &sv, int B, int T, int H,
                           const void *workspace, hipStream_t stream) {
    const int nchunks = (T + C - 1) / C;
    const int BH = B * H;
    const int groups = (BH + 7) / 8;
    auto run = [&](auto vc) {
        constexpr int VC = decltype(vc)::value;
        hipLaunchKernelGGL((chunk_scan_kernel<QT, QT, D, C, false, VC, false, true>),
                           dim3(groups * 8 * (D / (4 * VC))), dim3(128), 0, stream,
                           static_cast<const QT *>(v), e, w, nullptr, s0, static_cast<QT *>(o),
                           s_out, static_cast<const unsigned char *>(workspace), ScanGates{}, T,
                           H, BH, nchunks, sv);
        return hipGetLastError();
    };
    if (std::is_same_v<QT, bf16_t> && split_scan_applies(B, H, D))
        return launch_chunk_scan_split_save(v, e, w, s0, s_out, sv.u, sv.states, B, T, H, D, C,
                                            workspace, stream);
    if (std::is_same_v<QT, bf16_t> && scan_narrow_tiles(B, H, D)) return run(std::integral_constant<int, 2>{});
    return run(std::integral_constant<int, 4>{});
}

hipError_t launch_chunk_scan_save(const void *v, const float *e, const float *w, const float *s0,
                                  void *o, float *s_out, float *u_out, float *states, int B,
                                  int T, int H, int d, int chunk, bool bf16,
                                  const void *workspace, hipStream_t stream) {
    const ScanSave sv{u_out, states};
#define MUIR_SCAN_SV(D, C)                                                                        \
    if (d == D && chunk == C)                                                                     \
        return bf16 ? scan_save_typed<bf16_t, D, C>(v, e, w, s0, o, s_out, sv, B, T, H, workspace, \
                                                    stream)                                       \
                    : scan_save_typed<float, D, C>(v, e, w, s0, o, s_out, sv, B, T, H, workspace,  \
                                                   stream);
    MUIR_SCAN_SV(64, 64) MUIR_SCAN_SV(64, 128) MUIR_SCAN_SV(64, 256)
    MUIR_SCAN_SV(128, 64) MUIR_SCAN_SV(128, 128) MUIR_SCAN_SV(128, 256)
#undef MUIR_SCAN_SV
    return hipErrorInvalidValue;
}

bool scan_gates_in_kernel(int B, int H, int d, int chunk) {
    return !scan_narrow_tiles(B, H, d) && chunk <= 128;
}

hipError_t launch_chunk_scan_lowrank(const void *v, const void *z, const void *Ue, const void *Uw,
                                     const float *ce, const float *cw, const void *Uo,
                                     const float *co, const float *s0, void *o, float *s_out, int B,
                                     int T, int H, int d, int chunk, const void *workspace,
                                     hipStream_t stream) {
    if (!scan_gates_in_kernel(B, H, d, chunk)) return hipErrorNotSupported;
    const ScanGates sg{static_cast<const bf16_t *>(z), static_cast<const bf16_t *>(Ue),
                       static_cast<const bf16_t *>(Uw), ce, cw, static_cast<const bf16_t *>(Uo), co};
#define MUIR_SCAN_LR(D, C)                                                                        \
    if (d == D && chunk == C)                                                                     \
        return scan_vc<bf16_t, bf16_t, D, C, 4, true>(v, nullptr, nullptr, nullptr, s0, o, s_out, \
                                                      B, T, H, workspace, stream, sg);
    MUIR_SCAN_LR(64, 64) MUIR_SCAN_LR(64, 128) MUIR_SCAN_LR(128, 64) MUIR_SCAN_LR(128, 128)
#undef MUIR_SCAN_LR
    return hipErrorInvalidValue;
}

}  // namespace muir
