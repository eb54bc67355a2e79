// Chunkwise-parallel forward of the gated delta rule with matched-filter readout.
//
// The pages' stable large-chunk scheme (liuch.name summary of arXiv 2611.08376, third
// bullet; openai-hub news page, section on rewriting the long-sequence parallel
// algorithm for TPU): every decay that crosses a block boundary is split into two
// running products pivoted at that boundary, both in (0, 1], so nothing is ever
// divided by a cumulative decay; the intra-chunk unit lower-triangular system is solved
// by recursive block-Neumann halving with its off-diagonal products on the matrix
// cores; chunks are chained by carrying the fp32 state.
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
//  * chunk_gram_kernel (a1-a3), one workgroup per (chunk, head, batch), fully
//    parallel: decay products, the operands K*gamma, Qh*gamma, (K*beta)^T, gamma_C, and
//    the lower-triangular M and P in 16x16 blocks. Off-diagonal block (bt, bs) is one
//    MFMA product (K_bt * pi_bt) Diag(D) (K_bs * sigma_bs)^T pivoted at the start of
//    block bt: pi is the running product inside bt from its start, sigma the running
//    product inside bs after s, D the product of the whole blocks in between. The
//    16x16 diagonal blocks recurse further (pivots every 8, 4, 2, 1 tokens), each
//    level one masked MFMA tile, so the Gram work is all on the matrix cores.
//  * chunk_scan_kernel (a4-a6), one workgroup per (batch x head, 16 value columns),
//    sequential over chunks (value columns are exactly independent): H and Qh*gamma*S0
//    on MFMA, the recursive block-Neumann solve of each column's system (16-token
//    leaves by forward substitution, off-diagonal updates R2 -= E2 * (M21 X1) on MFMA),
//    the readout P U and the state update on MFMA, fp32 state kept on chip.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace muir {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr size_t kLdsBudget = 160 * 1024 - 1024;

__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace slot of one (batch, head, chunk).
template <typename OpT, int D, int C> struct Slot {
    static constexpr int NB = C / 16;
    static constexpr int NTRI = NB * (NB + 1) / 2;
    static constexpr size_t M_OFF = 0;
    static constexpr size_t P_OFF = align256(M_OFF + size_t(NTRI) * 256 * sizeof(OpT));
    static constexpr size_t KG_OFF = align256(P_OFF + size_t(NTRI) * 256 * sizeof(OpT));
    static constexpr size_t QG_OFF = align256(KG_OFF + size_t(C) * D * sizeof(OpT));
    static constexpr size_t KBT_OFF = align256(QG_OFF + size_t(C) * D * sizeof(OpT));
    static constexpr size_t GC_OFF = align256(KBT_OFF + size_t(C) * D * sizeof(OpT));
    static constexpr size_t BYTES = align256(GC_OFF + size_t(D) * 4);
    static __device__ __forceinline__ int tri(int bt, int bs) { return bt * (bt + 1) / 2 + bs; }
};

template <typename OpT, int D, int C> struct GramLds {
    static constexpr size_t PI = size_t(C / 16) * D * 4;            // block totals
    static constexpr size_t BB = size_t(C) * D * sizeof(OpT);       // K * sigma
    static constexpr size_t SCR = size_t(16) * D * 4;               // per-wave table
    static constexpr int NW_FIT = int((kLdsBudget - PI - BB) / SCR);
    static constexpr int NW = NW_FIT < kWaves ? NW_FIT : kWaves;    // waves in phase 2
    static constexpr size_t BYTES = PI + BB + size_t(NW) * SCR;
    static_assert(NW >= 1, "LDS budget");
};

// ---------------------------------------------------------------------------------
// Phase P: decay products, pivoted operands and the intra-chunk Gram blocks.
// ---------------------------------------------------------------------------------
template <typename QT, typename OpT, int D, int C>
__global__ __launch_bounds__(kThreads) void chunk_gram_kernel(
    const QT *__restrict__ q, const QT *__restrict__ k, const float *__restrict__ a,
    const float *__restrict__ g, const float *__restrict__ r, unsigned char *__restrict__ ws,
    int T, int H, int nchunks) {
    using SL = Slot<OpT, D, C>;
    using LDS = GramLds<OpT, D, C>;
    using MM = Mma<OpT>;
    constexpr int NB = C / 16;
    constexpr int NK = D / MM::KSTEP;  // k-steps over the channels
    constexpr int VALS = MM::VALS;

    extern __shared__ __align__(16) unsigned char smem[];
    float *sh_pi = reinterpret_cast<float *>(smem);                              // [NB][D]
    OpT *sh_bb = reinterpret_cast<OpT *>(smem + LDS::PI);                        // [C][D]
    float *sh_scr = reinterpret_cast<float *>(smem + LDS::PI + LDS::BB);         // [NW][16][D]

    const int ci = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    unsigned char *slot = ws + ((size_t(b) * H + h) * nchunks + ci) * SL::BYTES;
    OpT *gM = reinterpret_cast<OpT *>(slot + SL::M_OFF);
    OpT *gP = reinterpret_cast<OpT *>(slot + SL::P_OFF);
    OpT *gKg = reinterpret_cast<OpT *>(slot + SL::KG_OFF);
    OpT *gQg = reinterpret_cast<OpT *>(slot + SL::QG_OFF);
    OpT *gKbT = reinterpret_cast<OpT *>(slot + SL::KBT_OFF);
    float *gGC = reinterpret_cast<float *>(slot + SL::GC_OFF);

    const int t0 = ci * C;
    const int nreal = min(C, T - t0);
    const size_t HD = size_t(H) * D;
    const size_t base = (size_t(b) * T + t0) * HD + size_t(h) * D;  // token t0, channel 0
    const float *rh = r + size_t(h) * D;
    const int tid = threadIdx.x;

    // Padded tokens (t >= nreal) behave as a = 1, k = q = 0: they add nothing and
    // leave every decay product of the real tokens unchanged.
    auto ld_a = [&](int t, int ch) -> float { return t < nreal ? a[base + t * HD + ch] : 1.f; };
    auto ld_k = [&](int t, int ch) -> float {
        return t < nreal ? elem<QT>::load(k, base + t * HD + ch) : 0.f;
    };
    auto ld_qh = [&](int t, int ch) -> float {
        return t < nreal ? rh[ch] * g[base + t * HD + ch] * elem<QT>::load(q, base + t * HD + ch)
                         : 0.f;
    };

    // a1: whole-block decay products Pi_b = prod of the 16 decays of block b, per row.
    for (int idx = tid; idx < NB * D; idx += kThreads) {
        const int bb = idx / D, ch = idx % D;
        float p = 1.f;
#pragma unroll
        for (int t = 0; t < 16; ++t) p *= ld_a(16 * bb + t, ch);
        sh_pi[idx] = p;
    }
    __syncthreads();

    // a1/a2: per (block, row): pi (running product from the block start, inclusive) and
    // sigma (running product after s to the block end). gamma_t = G_b * pi_t with G_b the
    // product of the earlier blocks; beta_s = sigma_s * Gs_b with Gs_b the product of the
    // later blocks. All factors lie in [0, 1]; nothing is divided.
    for (int idx = tid; idx < NB * D; idx += kThreads) {
        const int bb = idx / D, ch = idx % D;
        float G = 1.f, Gs = 1.f;
        for (int x = 0; x < bb; ++x) G *= sh_pi[x * D + ch];
        for (int x = bb + 1; x < NB; ++x) Gs *= sh_pi[x * D + ch];
        if (bb == 0) gGC[ch] = G * sh_pi[ch] * Gs;  // gamma_C (G = 1 here)
        float av[16], kv[16];
        float pi = 1.f;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int tt = 16 * bb + t;
            av[t] = ld_a(tt, ch);
            kv[t] = ld_k(tt, ch);
            pi *= av[t];
            const float gam = G * pi;
            gKg[size_t(tt) * D + ch] = MM::from_f32(kv[t] * gam);
            gQg[size_t(tt) * D + ch] = MM::from_f32(ld_qh(tt, ch) * gam);
        }
        float sig = 1.f;
#pragma unroll
        for (int t = 15; t >= 0; --t) {
            const int tt = 16 * bb + t;
            gKbT[size_t(ch) * C + tt] = MM::from_f32(kv[t] * (sig * Gs));
            sh_bb[size_t(tt) * D + ch] = MM::from_f32(kv[t] * sig);
            sig *= av[t];
        }
    }
    __syncthreads();

    // a3: Gram blocks. Wave w handles row blocks bt = w, w + NW, ...
    const int wave = tid >> 6, lane = tid & 63;
    if (wave >= LDS::NW) return;
    float *scr = sh_scr + size_t(wave) * 16 * D;
    const int tl = lane & 15;         // fragment row (token within the block)
    const int orow = (lane >> 4) * 4; // accumulator rows orow..orow+3
    const int ocol = lane & 15;       // accumulator column
    constexpr int CPL = D / 64;       // channels per lane for the running products

    for (int bt = wave; bt < NB; bt += LDS::NW) {
        // Block data: decays per (lane channel, token), k and qh in fragment layout.
        float av[CPL][16];
#pragma unroll
        for (int m = 0; m < CPL; ++m)
#pragma unroll
            for (int t = 0; t < 16; ++t) av[m][t] = ld_a(16 * bt + t, lane + 64 * m);
        float kf[NK][VALS], qf[NK][VALS];
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
#pragma unroll
            for (int j = 0; j < VALS; ++j) {
                const int ch = kk * MM::KSTEP + MM::kidx(lane, j);
                kf[kk][j] = ld_k(16 * bt + tl, ch);
                qf[kk][j] = ld_qh(16 * bt + tl, ch);
            }

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
                        scr[t * D + ch] = run;
                    }
                    run = 1.f;
#pragma unroll
                    for (int s = n0 + half - 1; s >= n0; --s) {
                        scr[s * D + ch] = run;
                        run *= av[m][s];
                    }
                }
            }
            wave_lds_sync();
            f32x4_t accM = zero4(), accP = zero4();
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                float xk[VALS], xq[VALS];
#pragma unroll
                for (int j = 0; j < VALS; ++j) {
                    const float f = scr[tl * D + kk * MM::KSTEP + MM::kidx(lane, j)];
                    xk[j] = kf[kk][j] * f;
                    xq[j] = qf[kk][j] * f;
                }
                const auto fk = MM::pack(xk);
                const auto fq = MM::pack(xq);
                accM = MM::mma(fk, fk, accM);
                accP = MM::mma(fq, fk, accP);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = orow + i, s = ocol;
                const bool valid = ((t ^ s) < 2 * half) && (t & half) && !(s & half);
                leafM[i] += valid ? accM[i] : 0.f;
                leafP[i] += valid ? accP[i] : 0.f;
            }
            wave_lds_sync();
        }
        {   // diagonal of P: qh_t . k_t
            f32x4_t accD = zero4();
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) accD = MM::mma(MM::pack(qf[kk]), MM::pack(kf[kk]), accD);
#pragma unroll
            for (int i = 0; i < 4; ++i) leafP[i] += (orow + i == ocol) ? accD[i] : 0.f;
        }
        {
            OpT *mb = gM + size_t(SL::tri(bt, bt)) * 256;
            OpT *pb = gP + size_t(SL::tri(bt, bt)) * 256;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                mb[(orow + i) * 16 + ocol] = MM::from_f32(leafM[i]);
                pb[(orow + i) * 16 + ocol] = MM::from_f32(leafP[i]);
            }
        }
        if (bt == 0) continue;

        // Off-diagonal blocks (bt, bs), bs < bt, pivot at the start of block bt:
        // A = K_bt * pi_bt (and Qh_bt * pi_bt), B = K_bs * sigma_bs * D(bs, bt).
#pragma unroll
        for (int m = 0; m < CPL; ++m) {
            float run = 1.f;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                run *= av[m][t];
                scr[t * D + lane + 64 * m] = run;
            }
        }
        wave_lds_sync();
        typename MM::frag fAk[NK], fAq[NK];
        float dm[NK][VALS];
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            float xk[VALS], xq[VALS];
#pragma unroll
            for (int j = 0; j < VALS; ++j) {
                const float f = scr[tl * D + kk * MM::KSTEP + MM::kidx(lane, j)];
                xk[j] = kf[kk][j] * f;
                xq[j] = qf[kk][j] * f;
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
                float xb[VALS];
#pragma unroll
                for (int j = 0; j < VALS; ++j) {
                    const int ch = kk * MM::KSTEP + MM::kidx(lane, j);
                    xb[j] = MM::to_f32(sh_bb[size_t(16 * bs + tl) * D + ch]) * dm[kk][j];
                    dm[kk][j] *= sh_pi[bs * D + ch];
                }
                const auto fb = MM::pack(xb);
                accM = MM::mma(fAk[kk], fb, accM);
                accP = MM::mma(fAq[kk], fb, accP);
            }
            OpT *mb = gM + size_t(SL::tri(bt, bs)) * 256;
            OpT *pb = gP + size_t(SL::tri(bt, bs)) * 256;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                mb[(orow + i) * 16 + ocol] = MM::from_f32(accM[i]);
                pb[(orow + i) * 16 + ocol] = MM::from_f32(accP[i]);
            }
        }
    }
}

// ---------------------------------------------------------------------------------
// Phase S: sequential chunk scan with the per-column recursive block-Neumann solve.
// ---------------------------------------------------------------------------------
template <typename QT, typename OpT, int D, int C>
__global__ __launch_bounds__(kThreads) void chunk_scan_kernel(
    const QT *__restrict__ v, const float *__restrict__ e, const float *__restrict__ w,
    const float *__restrict__ s0, QT *__restrict__ o, float *__restrict__ s_out,
    const unsigned char *__restrict__ ws, int T, int H, int nchunks) {
    using SL = Slot<OpT, D, C>;
    using MM = Mma<OpT>;
    constexpr int NB = C / 16;            // 16-token blocks per chunk
    constexpr int NCT = D / 16;           // 16-row channel tiles of the state
    constexpr int CP = C + 4;             // padded row of the [column][token] LDS tiles
    constexpr int RT_PER_WAVE = (NB + kWaves - 1) / kWaves;
    constexpr int CT_PER_WAVE = (NCT + kWaves - 1) / kWaves;
    constexpr int NKD = D / MM::KSTEP;
    constexpr int VALS = MM::VALS;

    __shared__ __align__(16) float sh_S[D * 16];   // state tile [channel][column]
    __shared__ __align__(16) float sh_U[16 * CP];  // RHS, then solution [column][token]
    __shared__ __align__(16) float sh_E[16 * CP];  // erase gate [column][token]
    __shared__ __align__(16) float sh_L[16 * 16];  // current leaf of M, fp32

    const int bh = blockIdx.x;
    const int b = bh / H, h = bh % H;
    const int j0 = 16 * blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int orow = (lane >> 4) * 4, ocol = lane & 15, frow = lane & 15;
    const size_t HD = size_t(H) * D;
    const size_t sbase = size_t(bh) * D * D;  // state [b,h] offset

    f32x4_t Sreg[CT_PER_WAVE];
#pragma unroll
    for (int x = 0; x < CT_PER_WAVE; ++x) {
        const int ct = wave + kWaves * x;
        if (ct < NCT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch = 16 * ct + orow + i;
                const float val = s0 ? s0[sbase + size_t(ch) * D + j0 + ocol] : 0.f;
                Sreg[x][i] = val;
                sh_S[ch * 16 + ocol] = val;
            }
        }
    }
    __syncthreads();

    for (int ci = 0; ci < nchunks; ++ci) {
        const unsigned char *slot = ws + (size_t(bh) * nchunks + ci) * SL::BYTES;
        const OpT *gM = reinterpret_cast<const OpT *>(slot + SL::M_OFF);
        const OpT *gP = reinterpret_cast<const OpT *>(slot + SL::P_OFF);
        const OpT *gKg = reinterpret_cast<const OpT *>(slot + SL::KG_OFF);
        const OpT *gQg = reinterpret_cast<const OpT *>(slot + SL::QG_OFF);
        const OpT *gKbT = reinterpret_cast<const OpT *>(slot + SL::KBT_OFF);
        const float *gGC = reinterpret_cast<const float *>(slot + SL::GC_OFF);
        const int t0 = ci * C;
        const int nreal = min(C, T - t0);
        const size_t tbase = (size_t(b) * T + t0) * HD + size_t(h) * D + j0;

        // S0 as the B operand (contraction = channel, column = value column).
        typename MM::frag fS[NKD];
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk) {
            float x[VALS];
#pragma unroll
            for (int j = 0; j < VALS; ++j)
                x[j] = sh_S[(kk * MM::KSTEP + MM::kidx(lane, j)) * 16 + frow];
            fS[kk] = MM::pack(x);
        }

        // a5 (first half): H = (K*gamma) S0 and the inter-chunk readout (Qh*gamma) S0;
        // right-hand side R = w*v - e*H.
        f32x4_t Oin[RT_PER_WAVE];
#pragma unroll
        for (int x = 0; x < RT_PER_WAVE; ++x) {
            const int rt = wave + kWaves * x;
            if (rt >= NB) continue;
            f32x4_t accH = zero4(), accO = zero4();
#pragma unroll
            for (int kk = 0; kk < NKD; ++kk) {
                const size_t off = size_t(16 * rt + frow) * D + kk * MM::KSTEP + MM::kidx(lane, 0);
                accH = MM::mma(MM::load(gKg + off), fS[kk], accH);
                accO = MM::mma(MM::load(gQg + off), fS[kk], accO);
            }
            Oin[x] = accO;
            float4 rr, ee;
            float *rp = &rr.x, *ep = &ee.x;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * rt + orow + i;
                float ev = 0.f, bv = 0.f;
                if (t < nreal) {
                    const size_t idx = tbase + size_t(t) * HD + ocol;
                    ev = e[idx];
                    bv = w[idx] * elem<QT>::load(v, idx);
                }
                rp[i] = bv - ev * accH[i];
                ep[i] = ev;
            }
            *reinterpret_cast<float4 *>(&sh_U[ocol * CP + 16 * rt + orow]) = rr;
            *reinterpret_cast<float4 *>(&sh_E[ocol * CP + 16 * rt + orow]) = ee;
        }
        __syncthreads();

        // a4: recursive block-Neumann solve, leaf by leaf. After leaf L the left node that
        // just completed is [L+1-z, L+1) (z = lowest set bit of L+1, in blocks); its
        // product with M updates the right node [L+1, L+1+z): R2 -= E2 * (M21 X1).
        for (int L = 0; L < NB; ++L) {
            if (wave == 0) {
                const OpT *mb = gM + size_t(SL::tri(L, L)) * 256;
#pragma unroll
                for (int i = 0; i < 4; ++i) sh_L[lane * 4 + i] = MM::to_f32(mb[lane * 4 + i]);
                wave_lds_sync();
                if (lane < 16) {
                    float rv[16], ev[16], p[16];
                    const float4 *ru = reinterpret_cast<const float4 *>(&sh_U[lane * CP + 16 * L]);
                    const float4 *re = reinterpret_cast<const float4 *>(&sh_E[lane * CP + 16 * L]);
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const float4 a4 = ru[x], b4 = re[x];
                        rv[4 * x] = a4.x; rv[4 * x + 1] = a4.y; rv[4 * x + 2] = a4.z; rv[4 * x + 3] = a4.w;
                        ev[4 * x] = b4.x; ev[4 * x + 1] = b4.y; ev[4 * x + 2] = b4.z; ev[4 * x + 3] = b4.w;
                    }
#pragma unroll
                    for (int t = 0; t < 16; ++t) p[t] = 0.f;
#pragma unroll
                    for (int s = 0; s < 16; ++s) {
                        const float u = rv[s] - ev[s] * p[s];
                        rv[s] = u;
#pragma unroll
                        for (int t = s + 1; t < 16; ++t) p[t] += sh_L[t * 16 + s] * u;
                    }
                    float4 *wu = reinterpret_cast<float4 *>(&sh_U[lane * CP + 16 * L]);
#pragma unroll
                    for (int x = 0; x < 4; ++x)
                        wu[x] = make_float4(rv[4 * x], rv[4 * x + 1], rv[4 * x + 2], rv[4 * x + 3]);
                }
            }
            __syncthreads();
            const int z = (L + 1) & -(L + 1);
            if (L + 1 < NB) {
                const int s_lo = 16 * (L + 1 - z);  // left node tokens [s_lo, s_lo + 16z)
                const int klen = 16 * z;
                const int nks = (klen + MM::KSTEP - 1) / MM::KSTEP;
                for (int rt = L + 1 + wave; rt < L + 1 + z && rt < NB; rt += kWaves) {
                    f32x4_t acc = zero4();
                    for (int ks = 0; ks < nks; ++ks) {
                        const int kap = ks * MM::KSTEP + MM::kidx(lane, 0);
                        typename MM::frag fa, fb;
                        if (kap < klen) {
                            const int s = s_lo + kap;
                            fa = MM::load(gM + size_t(SL::tri(rt, s >> 4)) * 256 + frow * 16 + (s & 15));
                            float x[VALS];
#pragma unroll
                            for (int j = 0; j < VALS; ++j) x[j] = sh_U[frow * CP + s + j];
                            fb = MM::pack(x);
                        } else {
                            fa = MM::zero();
                            fb = MM::zero();
                        }
                        acc = MM::mma(fa, fb, acc);
                    }
                    float4 *up = reinterpret_cast<float4 *>(&sh_U[ocol * CP + 16 * rt + orow]);
                    const float4 ev = *reinterpret_cast<const float4 *>(&sh_E[ocol * CP + 16 * rt + orow]);
                    float4 uv = *up;
                    uv.x -= ev.x * acc[0];
                    uv.y -= ev.y * acc[1];
                    uv.z -= ev.z * acc[2];
                    uv.w -= ev.w * acc[3];
                    *up = uv;
                }
                __syncthreads();
            }
        }

        // a6: readout O = (Qh*gamma) S0 + P U, cast and store.
#pragma unroll
        for (int x = 0; x < RT_PER_WAVE; ++x) {
            const int rt = wave + kWaves * x;
            if (rt >= NB) continue;
            f32x4_t acc = Oin[x];
            const int klen = 16 * (rt + 1);
            const int nks = (klen + MM::KSTEP - 1) / MM::KSTEP;
            for (int ks = 0; ks < nks; ++ks) {
                const int s = ks * MM::KSTEP + MM::kidx(lane, 0);
                typename MM::frag fa, fb;
                if (s < klen) {
                    fa = MM::load(gP + size_t(SL::tri(rt, s >> 4)) * 256 + frow * 16 + (s & 15));
                    float xx[VALS];
#pragma unroll
                    for (int j = 0; j < VALS; ++j) xx[j] = sh_U[frow * CP + s + j];
                    fb = MM::pack(xx);
                } else {
                    fa = MM::zero();
                    fb = MM::zero();
                }
                acc = MM::mma(fa, fb, acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * rt + orow + i;
                if (t < nreal) elem<QT>::store(o, tbase + size_t(t) * HD + ocol, acc[i]);
            }
        }

        // a5 (second half): S_C = Diag(gamma_C) S0 + (K*beta)^T U.
        f32x4_t Snew[CT_PER_WAVE];
#pragma unroll
        for (int x = 0; x < CT_PER_WAVE; ++x) {
            const int ct = wave + kWaves * x;
            if (ct >= NCT) continue;
            f32x4_t acc = zero4();
#pragma unroll 4
            for (int ks = 0; ks < C / MM::KSTEP; ++ks) {
                const int s = ks * MM::KSTEP + MM::kidx(lane, 0);
                const auto fa = MM::load(gKbT + size_t(16 * ct + frow) * C + s);
                float xx[VALS];
#pragma unroll
                for (int j = 0; j < VALS; ++j) xx[j] = sh_U[frow * CP + s + j];
                acc = MM::mma(fa, MM::pack(xx), acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) Snew[x][i] = gGC[16 * ct + orow + i] * Sreg[x][i] + acc[i];
        }
        __syncthreads();
#pragma unroll
        for (int x = 0; x < CT_PER_WAVE; ++x) {
            const int ct = wave + kWaves * x;
            if (ct >= NCT) continue;
            Sreg[x] = Snew[x];
#pragma unroll
            for (int i = 0; i < 4; ++i) sh_S[(16 * ct + orow + i) * 16 + ocol] = Snew[x][i];
        }
        __syncthreads();
    }

    if (s_out) {
#pragma unroll
        for (int x = 0; x < CT_PER_WAVE; ++x) {
            const int ct = wave + kWaves * x;
            if (ct >= NCT) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s_out[sbase + size_t(16 * ct + orow + i) * D + j0 + ocol] = Sreg[x][i];
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
    using LDS = GramLds<OpT, D, C>;
    auto kg = chunk_gram_kernel<QT, OpT, D, C>;
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kg),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(LDS::BYTES));
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kg, dim3(nchunks, H, B), dim3(kThreads), LDS::BYTES, stream,
                       static_cast<const QT *>(q), static_cast<const QT *>(k), a, g, r,
                       static_cast<unsigned char *>(workspace), T, H, nchunks);
    return hipGetLastError();
}

template <typename QT, typename OpT, int D, int C>
hipError_t scan_typed(const void *v, const float *e, const float *w, const float *s0, void *o,
                      float *s_out, int B, int T, int H, const void *workspace,
                      hipStream_t stream) {
    const int nchunks = (T + C - 1) / C;
    hipLaunchKernelGGL((chunk_scan_kernel<QT, OpT, D, C>), dim3(B * H, D / 16), dim3(kThreads), 0,
                       stream, static_cast<const QT *>(v), e, w, s0, static_cast<QT *>(o), s_out,
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
