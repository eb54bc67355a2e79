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
// w_t * v_t, read with r * g_t * q_t).
//
// Two kernels:
//  * chunk_prepare_kernel (a1-a3), one workgroup per (chunk, head, batch), fully
//    parallel: decay products, the operands K*gamma, Qh*gamma, (K*beta)^T, gamma_C, and
//    the lower-triangular M and P in 16x16 blocks. Off-diagonal block (bt, bs) is one
//    MFMA product (K_bs * sigma_bs * D)(K_bt * pi_bt)^T pivoted at the start of block
//    bt: pi is the running product inside bt from its start, sigma the running product
//    inside bs after s, D the product of the whole blocks in between. The 16x16
//    diagonal blocks recurse further (pivots every 8, 4, 2, 1 tokens), each level one
//    masked MFMA tile, so the Gram work is all on the matrix cores.
//  * chunk_scan_kernel (a4-a6), one workgroup per (batch x head, 16 value columns),
//    sequential over chunks (value columns are exactly independent). Wave 0 carries the
//    serial chain: for leaf L (16 tokens) it subtracts E_L * (M_{L,<L} U_{<L}) from the
//    leaf's right-hand side on MFMA -- the off-diagonal products of the block-Neumann
//    recursion, grouped by the leaf they update -- then solves the 16x16 unit
//    lower-triangular leaf of every column by forward substitution. Waves 1-3 follow one
//    leaf behind: the readout O_L = (Qh*gamma)_L S0 + P_{L,<=L} U_{<=L} and the state
//    contribution (K*beta)_L^T U_L, both on MFMA. The chunk's Gram blocks M are copied
//    into LDS by direct global->LDS loads issued during the previous chunk.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace muir {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr size_t kLdsBudget = 160 * 1024 - 1024;

__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace slot of one (batch, head, chunk). M and P blocks are 16x16 row-major
// (row = later token t, column = earlier token s), lower-triangular block order.
template <typename OpT, int D, int C> struct Slot {
    static constexpr int NB = C / 16;
    static constexpr int NTRI = NB * (NB + 1) / 2;
    static constexpr size_t M_BYTES = size_t(NTRI) * 256 * sizeof(OpT);
    static constexpr size_t M_OFF = 0;
    // gamma_C sits right after M, inside a 1 KiB window, so one copy brings both into LDS.
    static constexpr size_t GC_OFF = M_OFF + M_BYTES;
    static constexpr size_t MG_BYTES = M_BYTES + 1024;
    static constexpr size_t P_OFF = GC_OFF + 1024;
    static constexpr size_t KG_OFF = align256(P_OFF + M_BYTES);
    static constexpr size_t QG_OFF = align256(KG_OFF + size_t(C) * D * sizeof(OpT));
    static constexpr size_t KBT_OFF = align256(QG_OFF + size_t(C) * D * sizeof(OpT));
    static constexpr size_t BYTES = align256(KBT_OFF + size_t(C) * D * sizeof(OpT));
    static_assert(M_BYTES % 1024 == 0 && D * 4 <= 1024, "M + gamma_C copy window");
    static __host__ __device__ constexpr int tri(int bt, int bs) { return bt * (bt + 1) / 2 + bs; }
};

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
    float *__restrict__ gGC = reinterpret_cast<float *>(slot + SL::GC_OFF);

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
        float G = 1.f, Gs = 1.f;
        for (int x = 0; x < bb; ++x) G *= sh_pi[x * D + ch];
        for (int x = bb + 1; x < NB; ++x) Gs *= sh_pi[x * D + ch];
        if (bb == 0) gGC[ch] = sh_pi[ch] * Gs;  // gamma_C
        float pi = 1.f;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int tt = 16 * bb + t;
            pi *= av[t];
            const float gam = G * pi;
            gKg[size_t(tt) * D + ch] = MM::from_f32(kv[t] * gam);
            gQg[size_t(tt) * D + ch] = MM::from_f32(qv[t] * gam);
        }
        float kbt[16];
        float sig = 1.f;
#pragma unroll
        for (int t = 15; t >= 0; --t) {
            kbt[t] = kv[t] * (sig * Gs);
            sh_bb[(16 * bb + t) * DB + ch] = MM::from_f32(kv[t] * sig);
            sig *= av[t];
        }
        OpT *dst = gKbT + size_t(ch) * C + 16 * bb;
#pragma unroll
        for (int t = 0; t < 16; t += 4)
            store4(dst + t, f32x4_t{kbt[t], kbt[t + 1], kbt[t + 2], kbt[t + 3]});
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
        store4(gM + size_t(SL::tri(bt, bt)) * 256 + tl * 16 + og, leafM);
        store4(gP + size_t(SL::tri(bt, bt)) * 256 + tl * 16 + og, leafP);
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
            store4(gM + size_t(SL::tri(bt, bs)) * 256 + tl * 16 + og, accM);
            store4(gP + size_t(SL::tri(bt, bs)) * 256 + tl * 16 + og, accP);
        }
    }
}

// ---------------------------------------------------------------------------------
// Phase S: sequential chunk scan.
// ---------------------------------------------------------------------------------
// Four (K*beta)^T values of one lane for a K = 16 step, kept packed and unconverted
// while the load is in flight.
template <typename OpT> struct KbFrag;
template <> struct KbFrag<bf16_t> {
    u16x4_t u;  // contraction indices 4*(lane/16) + [0, 4): one 8-byte load
    __device__ __forceinline__ void load(const bf16_t *row, int lane) {
        u = *reinterpret_cast<const u16x4_t *>(row + Mma<bf16_t>::k16idx(lane, 0));
    }
    __device__ __forceinline__ void get(float (&x)[4]) const {
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = bf16_to_f32(u[j]);
    }
};
template <> struct KbFrag<float> {
    float f[4];  // contraction indices 4*j + lane/16
    __device__ __forceinline__ void load(const float *row, int lane) {
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = row[Mma<float>::k16idx(lane, j)];
    }
    __device__ __forceinline__ void get(float (&x)[4]) const {
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = f[j];
    }
};

template <typename OpT, int D, int C> struct ScanLds {
    using SL = Slot<OpT, D, C>;
    static constexpr int CP = C + 4;                                  // padded token row
    static constexpr size_t TILE = size_t(16) * CP * 4;               // one [column][token] tile
    static constexpr size_t REST = 2 * TILE + size_t(D) * 16 * 4 + 256 * 4 + size_t(D) * 4;
    static constexpr bool M_IN_LDS = SL::MG_BYTES + REST <= kLdsBudget;
    static constexpr size_t M_SZ = M_IN_LDS ? SL::MG_BYTES : 0;   // M blocks + gamma_C window
    static constexpr size_t U_OFF = M_SZ;
    static constexpr size_t E_OFF = U_OFF + TILE;
    static constexpr size_t S_OFF = E_OFF + TILE;
    static constexpr size_t L_OFF = S_OFF + size_t(D) * 16 * 4;
    static constexpr size_t G_OFF = L_OFF + 256 * 4;              // gamma_C of this chunk
    static constexpr size_t BYTES = G_OFF + size_t(D) * 4;
    static_assert(BYTES <= kLdsBudget, "LDS budget");
};

typedef __attribute__((address_space(1))) const void gptr_t;
typedef __attribute__((address_space(3))) void lptr_t;

// Copy `bytes` (a multiple of 1 KiB) from global memory into LDS with direct
// global->LDS loads: every wave moves 1 KiB per instruction, 16 bytes per lane.
__device__ __forceinline__ void copy_to_lds(const void *gsrc, void *ldst, size_t bytes, int wave,
                                            int lane, int nwaves = kWaves) {
    const int n = static_cast<int>(bytes / 1024);
    for (int c = wave; c < n; c += nwaves) {
        const char *src = static_cast<const char *>(gsrc) + size_t(c) * 1024 + lane * 16;
        char *dst = static_cast<char *>(ldst) + size_t(c) * 1024;
        __builtin_amdgcn_global_load_lds((gptr_t *)src, (lptr_t *)dst, 16, 0, 0);
    }
}

// Leaves are numbered linearly over the whole sequence (leaf lam = chunk lam / NB, row
// block lam % NB), so every prefetch below may reach into the next chunk.
template <typename QT, typename OpT, int D, int C>
__global__ __launch_bounds__(kThreads) void chunk_scan_kernel(
    const QT *__restrict__ v, const float *__restrict__ e, const float *__restrict__ w,
    const float *__restrict__ s0, QT *__restrict__ o, float *__restrict__ s_out,
    const unsigned char *__restrict__ ws, int T, int H, int nchunks) {
    using SL = Slot<OpT, D, C>;
    using LY = ScanLds<OpT, D, C>;
    using MM = Mma<OpT>;
    using frag = typename MM::frag;
    constexpr int NB = C / 16;            // 16-token leaves per chunk
    constexpr int NCT = D / 16;           // 16-row channel tiles of the state
    constexpr int CP = LY::CP;
    constexpr int NKD = D / MM::KSTEP;
    constexpr int NKC = C / MM::KSTEP;    // k-steps over a whole chunk
    constexpr int VALS = MM::VALS;
    constexpr int CT_PER = (NCT + 2) / 3;  // state tiles per follower wave (waves 1..3)

    extern __shared__ __align__(16) unsigned char smem[];
    OpT *__restrict__ sh_M = reinterpret_cast<OpT *>(smem);
    float *__restrict__ sh_U = reinterpret_cast<float *>(smem + LY::U_OFF);  // [16][CP]
    float *__restrict__ sh_E = reinterpret_cast<float *>(smem + LY::E_OFF);  // [16][CP]
    float *__restrict__ sh_S = reinterpret_cast<float *>(smem + LY::S_OFF);  // [D][16]
    float *__restrict__ sh_L = reinterpret_cast<float *>(smem + LY::L_OFF);  // [16][16]
    float *__restrict__ sh_G = reinterpret_cast<float *>(smem + LY::G_OFF);  // [D]

    const int bh = blockIdx.x;
    const int b = bh / H, h = bh % H;
    const int j0 = 16 * blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int og = (lane >> 4) * 4, c16 = lane & 15;
    const size_t HD = size_t(H) * D;
    const size_t sbase = size_t(bh) * D * D;             // state [b,h] offset
    const size_t tb0 = size_t(b) * T * HD + size_t(h) * D + j0;  // token 0 of this tile
    const int nleaf = nchunks * NB;
    auto slot_of = [&](int ci) { return ws + (size_t(bh) * nchunks + ci) * SL::BYTES; };
    auto kg_of = [&](int ci) { return reinterpret_cast<const OpT *>(slot_of(ci) + SL::KG_OFF); };
    auto qg_of = [&](int ci) { return reinterpret_cast<const OpT *>(slot_of(ci) + SL::QG_OFF); };
    auto p_of = [&](int ci) { return reinterpret_cast<const OpT *>(slot_of(ci) + SL::P_OFF); };
    auto kbt_of = [&](int ci) { return reinterpret_cast<const OpT *>(slot_of(ci) + SL::KBT_OFF); };

    // --- prefetch helpers (global -> registers) ---
    // Every load is unconditional from a clamped, valid address; what lies past the end
    // of the sequence or outside a triangle is zeroed where it is consumed, so no branch
    // ever waits on a prefetch.
    auto leaf_pos = [&](int lam, int &ci, int &rt) {  // only called when nleaf >= 1
        const int lc = min(lam, nleaf - 1);
        ci = lc / NB;
        rt = lc % NB;
    };
    // Wave 0: (K*gamma) rows of leaf lam as the A operand, and its raw e, w, v.
    auto load_leaf = [&](int lam, frag (&kg)[NKD], float (&ee)[4], float (&ww)[4], QT (&vv)[4]) {
        int ci, rt;
        leaf_pos(lam, ci, rt);
        const OpT *src = kg_of(ci) + size_t(16 * rt + c16) * D + MM::kidx(lane, 0);
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk) kg[kk] = MM::load(src + kk * MM::KSTEP);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const size_t idx = tb0 + size_t(min(ci * C + 16 * rt + og + i, T - 1)) * HD + c16;
            ee[i] = e[idx];
            ww[i] = w[idx];
            vv[i] = v[idx];  // converted where it is used, so the load stays in flight
        }
    };
    // Readout owner: P row block of leaf lam (blocks past the diagonal are replaced by
    // the diagonal block and zeroed at use) and (Qh*gamma) rows of leaf lam.
    auto load_readout = [&](int lam, frag (&pp)[NKC], frag (&qg)[NKD]) {
        int ci, rt;
        leaf_pos(lam, ci, rt);
        const OpT *P = p_of(ci);
#pragma unroll
        for (int ks = 0; ks < NKC; ++ks) {
            const int s = ks * MM::KSTEP + MM::kidx(lane, 0);
            pp[ks] = MM::load(P + size_t(SL::tri(rt, min(s >> 4, rt))) * 256 + c16 * 16 + (s & 15));
        }
        const OpT *src = qg_of(ci) + size_t(16 * rt + c16) * D + MM::kidx(lane, 0);
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk) qg[kk] = MM::load(src + kk * MM::KSTEP);
    };
    // State followers: (K*beta)^T columns of leaf lam for the wave's channel tiles.
    auto load_kb = [&](int lam, KbFrag<OpT> (&dst)[CT_PER]) {
        int ci, rt;
        leaf_pos(lam, ci, rt);
        const OpT *K = kbt_of(ci);
#pragma unroll
        for (int x = 0; x < CT_PER; ++x) {
            const int ct = min(wave - 1 + 3 * x, NCT - 1);
            dst[x].load(K + size_t(16 * ct + c16) * C + 16 * rt, lane);
        }
    };

    // State tiles: waves 1..3 own channel tiles ct = (wave-1) + 3x, fp32, kept on chip.
    // The fp32 state lives in LDS (sh_S) between chunks; during a chunk the followers
    // accumulate (K*beta)^T U for their channel tiles in Sacc.
    f32x4_t Sacc[CT_PER];
#pragma unroll
    for (int x = 0; x < CT_PER; ++x) {
        Sacc[x] = zero4();
        const int ct = wave - 1 + 3 * x;
        if (wave > 0 && ct < NCT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch = 16 * ct + og + i;
                sh_S[ch * 16 + c16] = s0 ? s0[sbase + size_t(ch) * D + j0 + c16] : 0.f;
            }
        }
    }

    // Double-buffered prefetch state: buffer A serves even leaves, B odd leaves (chunks
    // hold an even number of leaves), so no in-flight register is ever copied.
    frag kgA[NKD], kgB[NKD];      // wave 0
    float eA[4], wA[4], eB[4], wB[4];
    QT vA[4], vB[4];
    frag pfP[NKC], pfQ[NKD];      // followers: next owned readout leaf
    KbFrag<OpT> kbA[CT_PER], kbB[CT_PER];
    // With no chunk (T == 0) nothing may be read: the workspace and the token tensors
    // are empty, and the clamped indices below would be -1.
    if (nchunks > 0) {
        if (wave == 0) {
            load_leaf(0, kgA, eA, wA, vA);
            load_leaf(1, kgB, eB, wB, vB);
        } else {
            load_readout(wave - 1, pfP, pfQ);
            load_kb(0, kbA);
            load_kb(1, kbB);
        }
        if constexpr (LY::M_IN_LDS) copy_to_lds(slot_of(0) + SL::M_OFF, sh_M, SL::MG_BYTES, wave, lane);
    }
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();

    for (int ci = 0; ci < nchunks; ++ci) {
        const unsigned char *slot = slot_of(ci);
        const OpT *__restrict__ gM = reinterpret_cast<const OpT *>(slot + SL::M_OFF);
        const float *__restrict__ gGC = reinterpret_cast<const float *>(slot + SL::GC_OFF);
        // M block (bt, bs), element row `row`, column `col` (the LDS copy when it fits).
        auto mptr = [&](int bt, int bs, int row, int col) -> const OpT * {
            const size_t off = size_t(SL::tri(bt, bs)) * 256 + row * 16 + col;
            if constexpr (LY::M_IN_LDS) return sh_M + off;
            else return gM + off;
        };

        // S0 of this chunk as the B operand (contraction = channel, column = value column).
        frag fS[NKD];
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk) {
            float x[VALS];
#pragma unroll
            for (int j = 0; j < VALS; ++j)
                x[j] = sh_S[(kk * MM::KSTEP + MM::kidx(lane, j)) * 16 + c16];
            fS[kk] = MM::pack(x);
        }
#pragma unroll
        for (int x = 0; x < CT_PER; ++x) Sacc[x] = zero4();
        // gamma_C of this chunk, kept apart from the copy window that the next chunk's
        // copy overwrites (read only after the chunk's last barrier).
        if (tid >= 64 && tid < 64 + D) {
            if constexpr (LY::M_IN_LDS) {
                sh_G[tid - 64] = reinterpret_cast<const float *>(smem + SL::GC_OFF)[tid - 64];
            } else {
                sh_G[tid - 64] = gGC[tid - 64];
            }
        }
        f32x4_t accH = zero4();  // wave 0: (K*gamma)_L S0 of the current leaf
        if (wave == 0) {
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) accH = MM::mma(kgA[kk], fS[kk], accH);
        }

        // One leaf. `kg/ee/ww/vv` hold leaf L and are refilled with leaf L + 2; `kgn` holds
        // leaf L + 1; `kb` holds leaf L's (K*beta)^T and is refilled with leaf L + 2.
        auto leaf_step = [&](int L, frag (&kg)[NKD], float (&ee)[4], float (&ww)[4],
                             QT (&vv)[4], const frag (&kgn)[NKD], KbFrag<OpT> (&kb)[CT_PER]) {
            const int lam = ci * NB + L;
            if (wave == 0) {
                // a4, serial chain. R_L = w*v - e * ((K*gamma)_L S0 + M_{L,<L} U_{<L}).
                // Straight-line over the whole chunk width: steps past 16*L read a valid
                // block and multiply a zeroed U fragment, so all LDS reads can be batched.
                f32x4_t acc0 = accH, acc1 = zero4();
                const int klen = 16 * L;
#pragma unroll
                for (int ks = 0; ks < NKC; ++ks) {
                    const int s = ks * MM::KSTEP + MM::kidx(lane, 0);
                    const bool in = s < klen;
                    const int sc = in ? s : 0;
                    float xa[VALS], xb[VALS];
                    load_vec<VALS>(mptr(L, sc >> 4, c16, sc & 15), xa);
                    load_vec<VALS>(sh_U + c16 * CP + sc, xb);
#pragma unroll
                    for (int j = 0; j < VALS; ++j) xb[j] = in ? xb[j] : 0.f;
                    if (ks & 1) acc1 = MM::mma(MM::pack(xa), MM::pack(xb), acc1);
                    else acc0 = MM::mma(MM::pack(xa), MM::pack(xb), acc0);
                }
                const f32x4_t acc = acc0 + acc1;
                const int cell = c16 * CP + 16 * L + og;
                float rr[4], er[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool in = ci * C + 16 * L + og + i < T;
                    er[i] = in ? ee[i] : 0.f;
                    rr[i] = (in ? ww[i] * to_f32(vv[i]) : 0.f) - er[i] * acc[i];
                }
                store4(sh_U + cell, f32x4_t{rr[0], rr[1], rr[2], rr[3]});
                store4(sh_E + cell, f32x4_t{er[0], er[1], er[2], er[3]});
                // Refill this buffer two leaves ahead and start the next leaf's
                // (K*gamma) S0 on the matrix cores while this leaf is substituted.
                load_leaf(lam + 2, kg, ee, ww, vv);
                accH = zero4();
                if (L + 1 < NB) {
#pragma unroll
                    for (int kk = 0; kk < NKD; ++kk) accH = MM::mma(kgn[kk], fS[kk], accH);
                }
                {   // leaf block of M in fp32, stored transposed: sh_L[s * 16 + t] = M_ts
                    float x4[4];
                    load_vec<4>(mptr(L, L, 0, 0) + lane * 4, x4);  // row lane/4, cols 4(lane%4)+i
#pragma unroll
                    for (int i = 0; i < 4; ++i) sh_L[(4 * (lane & 3) + i) * 16 + (lane >> 2)] = x4[i];
                }
                wave_lds_sync();
                if (lane < 16) {
                    // (I + Diag(e_j) M_LL) u_j = r_j by forward substitution, column j = lane.
                    // Column s of the leaf is read as four broadcast 16-byte LDS loads, one
                    // column ahead of its use.
                    float rv[16], ev[16], p[16];
                    const float4 *ru = reinterpret_cast<const float4 *>(sh_U + lane * CP + 16 * L);
                    const float4 *re = reinterpret_cast<const float4 *>(sh_E + lane * CP + 16 * L);
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const float4 a4 = ru[x], b4 = re[x];
                        rv[4 * x] = a4.x; rv[4 * x + 1] = a4.y; rv[4 * x + 2] = a4.z; rv[4 * x + 3] = a4.w;
                        ev[4 * x] = b4.x; ev[4 * x + 1] = b4.y; ev[4 * x + 2] = b4.z; ev[4 * x + 3] = b4.w;
                    }
#pragma unroll
                    for (int t = 0; t < 16; ++t) p[t] = 0.f;
                    const float4 *lt = reinterpret_cast<const float4 *>(sh_L);
                    float4 col[4], nxt[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) col[x] = lt[x];
#pragma unroll
                    for (int s = 0; s < 16; ++s) {
                        if (s + 1 < 16) {
#pragma unroll
                            for (int x = (s + 1) / 4; x < 4; ++x) nxt[x] = lt[(s + 1) * 4 + x];
                        }
                        const float u = rv[s] - ev[s] * p[s];
                        rv[s] = u;
                        const float *c = reinterpret_cast<const float *>(col);
#pragma unroll
                        for (int t = s + 1; t < 16; ++t) p[t] += c[t] * u;
#pragma unroll
                        for (int x = 0; x < 4; ++x) col[x] = nxt[x];
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    float4 *wu = reinterpret_cast<float4 *>(sh_U + lane * CP + 16 * L);
#pragma unroll
                    for (int x = 0; x < 4; ++x)
                        wu[x] = make_float4(rv[4 * x], rv[4 * x + 1], rv[4 * x + 2], rv[4 * x + 3]);
                }
            }
            lds_barrier();
            if (wave > 0) {
                // a6: readout of leaf L by its owner: O_L = (Qh*gamma)_L S0 + P_{L,<=L} U.
                if (wave - 1 == lam % 3) {
                    f32x4_t acc0 = zero4(), acc1 = zero4();
#pragma unroll
                    for (int kk = 0; kk < NKD; ++kk) acc0 = MM::mma(pfQ[kk], fS[kk], acc0);
                    const int klen = 16 * (L + 1);
#pragma unroll
                    for (int ks = 0; ks < NKC; ++ks) {
                        const int s = ks * MM::KSTEP + MM::kidx(lane, 0);
                        const bool in = s < klen;
                        float xb[VALS];
                        load_vec<VALS>(sh_U + c16 * CP + (in ? s : 0), xb);
#pragma unroll
                        for (int j = 0; j < VALS; ++j) xb[j] = in ? xb[j] : 0.f;
                        const frag fa = in ? pfP[ks] : MM::zero();
                        if (ks & 1) acc1 = MM::mma(fa, MM::pack(xb), acc1);
                        else acc0 = MM::mma(fa, MM::pack(xb), acc0);
                    }
                    const f32x4_t acc = acc0 + acc1;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = ci * C + 16 * L + og + i;
                        if (t < T) elem<QT>::store(o, tb0 + size_t(t) * HD + c16, acc[i]);
                    }
                    load_readout(lam + 3, pfP, pfQ);
                }
                // a5, leaf L's share of the state carry: Sacc += (K*beta)_L^T U_L.
                float ub[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) ub[j] = sh_U[c16 * CP + 16 * L + MM::k16idx(lane, j)];
#pragma unroll
                for (int x = 0; x < CT_PER; ++x) {
                    float ka[4];
                    kb[x].get(ka);
                    if (wave - 1 + 3 * x < NCT) Sacc[x] = MM::mma_k16(ka, ub, Sacc[x]);
                }
                load_kb(lam + 2, kb);
            }
        };

        for (int L = 0; L < NB; L += 2) {
            leaf_step(L, kgA, eA, wA, vA, kgB, kbA);
            leaf_step(L + 1, kgB, eB, wB, vB, kgA, kbB);
        }
        // Wave 0 finished with this chunk's M before the last barrier of the loop: the
        // next chunk's M (and gamma_C) streams into LDS while the state is finished.
        if constexpr (LY::M_IN_LDS) {
            if (ci + 1 < nchunks && wave > 0)
                copy_to_lds(slot_of(ci + 1) + SL::M_OFF, sh_M, SL::MG_BYTES, wave - 1, lane,
                            kWaves - 1);
        }
        // S_C = Diag(gamma_C) S0 + (K*beta)^T U.
        if (wave > 0) {
#pragma unroll
            for (int x = 0; x < CT_PER; ++x) {
                const int ct = wave - 1 + 3 * x;
                if (ct >= NCT) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ch = 16 * ct + og + i;
                    sh_S[ch * 16 + c16] = sh_G[ch] * sh_S[ch * 16 + c16] + Sacc[x][i];
                }
            }
        }
        if constexpr (LY::M_IN_LDS) __builtin_amdgcn_s_waitcnt(0);
        lds_barrier();
    }

    if (s_out && wave > 0) {
#pragma unroll
        for (int x = 0; x < CT_PER; ++x) {
            const int ct = wave - 1 + 3 * x;
            if (ct >= NCT) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch = 16 * ct + og + i;
                s_out[sbase + size_t(ch) * D + j0 + c16] = sh_S[ch * 16 + c16];
            }
        }
    }
}

template <typename OpT, int D, int C>
size_t slot_bytes() { return Slot<OpT, D, C>::BYTES; }

size_t slot_bytes_rt(bool bf16, int d, int chunk) {
#define MUIR_SLOT(D, C) \
    if (d == D && chunk == C) return bf16 ? slot_bytes<bf16_t, D, C>() : slot_bytes<float, D, C>();
    MUIR_SLOT(64, 64) MUIR_SLOT(64, 128) MUIR_SLOT(64, 256)
    MUIR_SLOT(128, 64) MUIR_SLOT(128, 128) MUIR_SLOT(128, 256)
#undef MUIR_SLOT
    return 0;
}

template <typename QT, typename OpT, int D, int C>
hipError_t prepare_typed(const void *q, const void *k, const float *a, const float *g,
                         const float *r, int B, int T, int H, void *workspace,
                         hipStream_t stream) {
    const int nchunks = (T + C - 1) / C;
    if (nchunks == 0) return hipSuccess;
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

template <typename QT, typename OpT, int D, int C>
hipError_t scan_typed(const void *v, const float *e, const float *w, const float *s0, void *o,
                      float *s_out, int B, int T, int H, const void *workspace,
                      hipStream_t stream) {
    const int nchunks = (T + C - 1) / C;
    using LY = ScanLds<OpT, D, C>;
    auto kern = chunk_scan_kernel<QT, OpT, D, C>;
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(LY::BYTES));
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(B * H, D / 16), dim3(kThreads), LY::BYTES, stream,
                       static_cast<const QT *>(v), e, w, s0, static_cast<QT *>(o), s_out,
                       static_cast<const unsigned char *>(workspace), T, H, nchunks);
    return hipGetLastError();
}

}  // namespace

size_t chunk_workspace_bytes(int B, int T, int H, int d, int chunk, bool bf16) {
    const size_t slot = slot_bytes_rt(bf16, d, chunk);
    if (slot == 0 || B < 1 || H < 1 || T < 0) return 0;
    const size_t nchunks = (size_t(T) + chunk - 1) / chunk;
    const size_t n = size_t(B) * size_t(H) * nchunks;
    if (n != 0 && slot > SIZE_MAX / n) return 0;
    return n * slot;
}

hipError_t launch_chunk_prepare(const void *q, const void *k, const float *a, const float *g,
                                const float *r, int B, int T, int H, int d, int chunk, bool bf16,
                                void *workspace, hipStream_t stream) {
#define MUIR_PREP(D, C)                                                                        \
    if (d == D && chunk == C)                                                                  \
        return bf16 ? prepare_typed<bf16_t, bf16_t, D, C>(q, k, a, g, r, B, T, H, workspace,    \
                                                          stream)                              \
                    : prepare_typed<float, float, D, C>(q, k, a, g, r, B, T, H, workspace, stream);
    MUIR_PREP(64, 64) MUIR_PREP(64, 128) MUIR_PREP(64, 256)
    MUIR_PREP(128, 64) MUIR_PREP(128, 128) MUIR_PREP(128, 256)
#undef MUIR_PREP
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_scan(const void *v, const float *e, const float *w, const float *s0,
                             void *o, float *s_out, int B, int T, int H, int d, int chunk,
                             bool bf16, const void *workspace, hipStream_t stream) {
#define MUIR_SCAN(D, C)                                                                        \
    if (d == D && chunk == C)                                                                  \
        return bf16 ? scan_typed<bf16_t, bf16_t, D, C>(v, e, w, s0, o, s_out, B, T, H,          \
                                                       workspace, stream)                      \
                    : scan_typed<float, float, D, C>(v, e, w, s0, o, s_out, B, T, H, workspace, \
                                                     stream);
    MUIR_SCAN(64, 64) MUIR_SCAN(64, 128) MUIR_SCAN(64, 256)
    MUIR_SCAN(128, 64) MUIR_SCAN(128, 128) MUIR_SCAN(128, 256)
#undef MUIR_SCAN
    return hipErrorInvalidValue;
}

}  // namespace muir
