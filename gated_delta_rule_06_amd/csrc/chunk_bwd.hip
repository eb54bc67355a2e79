// Backward pass of the chunkwise gated delta rule with matched-filter readout, for gfx950.
//
// Method: Muir abstract (Astral Feed page, "Full text") for the recurrence; liuch.name summary
// (third bullet) and the openai-hub page (section on the chunkwise algorithm) for the chunk
// form whose reverse mode this is. Per head, with q_hat = r * g * q, b = w * v, the state S
// (dk x dv) is decayed per row, the prediction p_t = S^T k_t is erased under the value gate,
// u_t = b_t - e_t * p_t is written, and o_t = S^T q_hat_t is read. Given dO and dS_T, the
// adjoint lambda = dL/dS runs backwards. Per chunk of C tokens, with gamma_t the decay product
// from the chunk start through t, beta_t the product after t to the chunk end, Gamma_ts the
// product over s < tau <= t, M_ts = sum_i k_ti Gamma_tsi k_si (s < t) and P_ts = sum_i
// q_hat_ti Gamma_tsi k_si (s <= t):
//
//   (I + M^T Diag(e_j)) dU_j = (K*beta) lambda_C + P^T dO        per value column j
//   dP = -E * dU,   dv = w * dU,   dw = v * dU,   de = -p * dU
//   lambda_0 = Diag(gamma_C) lambda_C + (Q_hat*gamma)^T dO + (K*gamma)^T dP
//   dq_hat_t = gamma_t * (S0 do_t) + sum_{s<=t} Gamma_ts * k_s (u_s . do_t)
//   dk_t     = gamma_t * (S0 dp_t) + sum_{s<t} Gamma_ts * k_s (u_s . dp_t)          (read)
//            + beta_t * (lambda_C u_t) + sum_{t'>=t} Gamma_t't * q_hat_t' (do_t' . u_t)
//            + sum_{t'>t} Gamma_t't * k_t' (dp_t' . u_t)                              (write)
//   a * dL/da at token tau = sum_{t>=tau in chunk} [q_hat*dq_hat + k*dk_read - k*dk_write]_t
//                            + rowsum(S_C * lambda_C)
//
// No decay is ever divided by. A pair's decay Gamma_ts is split into factors in (0, 1] at
// 16-token block boundaries (prefix of t's block, whole blocks between, suffix of s's block),
// inside one block at 4-token sub-block boundaries the same way, and inside one sub-block at its
// halves (the prepare) or as a direct product of at most three factors (the gradient kernel). The
// split forms make the decayed pair sums products on the fp32 matrix cores, one per block pair,
// sub-block gap or half split.
//
// Kernels, in launch order (after the forward's prepare and its scan, which also writes u and
// the chunk start states):
//   bwd_prepare_kernel  one workgroup per (b, h, chunk): K*beta, K*gamma and Q_hat*gamma (the
//                       last two channel-major), gamma_C, M and P transposed, and p.
//   bwd_scan_kernel     one workgroup per (b, h, 16 value columns), chunks in reverse: the
//                       transposed triangular solve, the adjoint carry, dv, dw, de.
//   bwd_grads_kernel    one workgroup per (b, h, chunk): O U^T, dP U^T and the state products,
//                       then the decayed pair sums for dq_hat and dk, then dq, dk, dg and
//                       a * dL/da (a reverse cumulative sum per channel).
//   bwd_dr_kernel       dr summed over batch and chunks.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace muir {

namespace {

constexpr int kC = 64;        // tokens per chunk
constexpr int kNB = kC / 16;  // 16-token blocks per chunk
constexpr int kBwdThreads = 256;

// D[16x16] += A[16xK] B[Kx16] on the fp32 matrix cores: fa(r, k) = A[r][k], fb(c, k) = B[k][c].
// Lane l holds output rows 4 (l / 16) .. + 3 of column l % 16.
template <int K, typename FA, typename FB>
__device__ __forceinline__ f32x4_t mm16(FA fa, FB fb, f32x4_t acc) {
    const int lane = threadIdx.x & 63, r = lane & 15, kq = lane >> 4;
#pragma unroll 8
    for (int m = 0; m < K / 4; ++m) {
        const int kk = 4 * m + kq;
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa(r, kk), fb(r, kk), acc, 0, 0, 0);
    }
    return acc;
}

template <typename QT> __device__ __forceinline__ float ld(const QT *p, size_t i) { return to_f32(p[i]); }

// Four consecutive elements (16-byte aligned for fp32, 8-byte for bf16) as floats.
__device__ __forceinline__ f32x4_t ld4(const float *p, size_t i) {
    return *reinterpret_cast<const f32x4_t *>(p + i);
}
__device__ __forceinline__ f32x4_t ld4(const bf16_t *p, size_t i) {
    const u16x4_t u = *reinterpret_cast<const u16x4_t *>(p + i);
    return f32x4_t{bf16_to_f32(u[0]), bf16_to_f32(u[1]), bf16_to_f32(u[2]), bf16_to_f32(u[3])};
}

// ------------------------------------------------------------------------------------------
// Prepare. LDS: M and P [C][C + 1], K*gamma [C][D + 4] for the prediction, and the pivot
// pass arrays (per 64-channel pass: a, k, q_hat, prefix F and suffix R [C][65] inside each
// 16-token block, then inside each 4-token sub-block, and the products of whole blocks,
// then of whole sub-blocks [16][64]).
//
// Pivots. For s < t in different 16-token blocks, Gamma_ts = F_t * (whole blocks between) *
// R_s, so each cross-block 16x16 tile of M or P is one matrix-core product over channels with
// the middle factor folded into the s side. Inside a 16-token block the same split at 4-token
// sub-blocks gives Gamma_ts = F4_t * (whole sub-blocks between) * R4_s; the middle factor
// depends only on s's sub-block and the gap (1, 2 or 3 sub-blocks), so each gap is one masked
// product. Pairs inside one sub-block (at most 3 factors) are direct products.
// ------------------------------------------------------------------------------------------
template <int D> struct PrepBwdLds {
    static constexpr int LDM = kC + 1;
    static constexpr int DH = 64;
    static constexpr int LDH = DH + 1;
    static constexpr int MP = 2 * kC * LDM;
    static constexpr int PASS = 5 * kC * LDH + 16 * DH;
    static constexpr int KGL = kC * (D + 4);
    static constexpr int FLOATS = MP + KGL + PASS;
    static constexpr size_t BYTES = size_t(FLOATS) * 4;
};

template <typename QT, int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_prepare_kernel(
    const QT *__restrict__ q, const QT *__restrict__ k, const float *__restrict__ a,
    const float *__restrict__ g, const float *__restrict__ r, const float *__restrict__ states,
    const float *__restrict__ u, float *__restrict__ kb, float *__restrict__ kg,
    float *__restrict__ qg, float *__restrict__ gC, float *__restrict__ Mw,
    float *__restrict__ Pw, float *__restrict__ pred, int T, int H, int nchunks) {
    using L = PrepBwdLds<D>;
    constexpr int C = kC, LDM = L::LDM, DH = L::DH, LDH = L::LDH;
    extern __shared__ float lds[];
    float *sM = lds, *sP = lds + kC * LDM;
    float *sKG = lds + L::MP;
    float *pass = sKG + L::KGL;
    float *sA = pass, *sK = sA + C * LDH, *sQ = sK + C * LDH, *sF = sQ + C * LDH,
          *sR = sF + C * LDH, *sMid = sR + C * LDH;

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int bh = b * H + h;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const size_t HD = size_t(H) * D;
    const int c0 = c * C;
    const int nval = min(C, T - c0);
    const size_t tok0 = (size_t(b) * T + c0) * HD + size_t(h) * D;
    const size_t slot = size_t(bh) * nchunks + c;
    const float *rh = r + size_t(h) * D;

    for (int idx = tid; idx < 2 * C * LDM; idx += kBwdThreads) lds[idx] = 0.f;

    // Cross-block tiles of M and P: pair p = (bt, bs), bs < bt, pair index bt (bt - 1) / 2 + bs;
    // tile job j < 12: matrix j / 6 (0: M, 1: P), pair j % 6. Wave w owns jobs w, w + 4, w + 8.
    f32x4_t acc[3] = {zero4(), zero4(), zero4()};
    // Diagonal 16x16 tiles: wave w owns tile jobs w and w + 4 (job: matrix j / 4, block j % 4),
    // accumulated over the passes.
    f32x4_t dacc[2] = {zero4(), zero4()};

    for (int p0 = 0; p0 < D; p0 += DH) {
        __syncthreads();
        {
            // All of the pass's loads are issued before the first LDS store.
            constexpr int N4 = C * DH / 4 / kBwdThreads;
            f32x4_t va[N4], vk[N4], vq[N4];
#pragma unroll
            for (int j = 0; j < N4; ++j) {
                const int e0 = 4 * (tid + kBwdThreads * j), t = e0 / DH, ii = e0 % DH;
                const size_t o = tok0 + size_t(t) * HD + p0 + ii;
                if (t < nval) {
                    va[j] = ld4(a, o);
                    vk[j] = ld4(k, o);
                    vq[j] = ld4(g, o) * ld4(q, o) * ld4(rh, p0 + ii);
                } else {
                    va[j] = f32x4_t{1.f, 1.f, 1.f, 1.f};
                    vk[j] = vq[j] = zero4();
                }
            }
#pragma unroll
            for (int j = 0; j < N4; ++j) {
                const int e0 = 4 * (tid + kBwdThreads * j), t = e0 / DH, ii = e0 % DH;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    sA[t * LDH + ii + q4] = va[j][q4];
                    sK[t * LDH + ii + q4] = vk[j][q4];
                    sQ[t * LDH + ii + q4] = vq[j][q4];
                }
            }
        }
        __syncthreads();
        float *sBp = sMid + 6 * DH;  // whole-block decay products per channel
        {
            // Thread (channel, 16-token block): prefix F and suffix R inside the block.
            const int ii = tid % DH, bb = tid / DH;
            float run = 1.f;
#pragma unroll
            for (int tl = 0; tl < 16; ++tl) {
                run *= sA[(16 * bb + tl) * LDH + ii];
                sF[(16 * bb + tl) * LDH + ii] = run;
            }
            run = 1.f;
#pragma unroll
            for (int tl = 15; tl >= 0; --tl) {
                sR[(16 * bb + tl) * LDH + ii] = run;
                run *= sA[(16 * bb + tl) * LDH + ii];
            }
            sBp[bb * DH + ii] = run;
        }
        __syncthreads();
        {
            // Thread (channel, block bb): products of the whole blocks between bb and each
            // earlier block; gamma and beta of its tokens and the scaled operands K*gamma,
            // Q_hat*gamma, K*beta; gamma_C.
            const int ii = tid % DH, bb = tid / DH, i = p0 + ii;
            float bp[kNB];
#pragma unroll
            for (int b2 = 0; b2 < kNB; ++b2) bp[b2] = sBp[b2 * DH + ii];
            float mid = 1.f, before = 1.f, after = 1.f;
            for (int bs = bb - 1; bs >= 0; --bs) {
                sMid[(bb * (bb - 1) / 2 + bs) * DH + ii] = mid;
                mid *= bp[bs];
            }
#pragma unroll
            for (int b2 = 0; b2 < kNB; ++b2) {
                if (b2 < bb) before *= bp[b2];
                if (b2 > bb) after *= bp[b2];
            }
#pragma unroll
            for (int tl = 0; tl < 16; ++tl) {
                const int t = 16 * bb + tl;
                const float gm = before * sF[t * LDH + ii];
                const float kt = sK[t * LDH + ii];
                kg[(slot * D + i) * C + t] = kt * gm;
                qg[(slot * D + i) * C + t] = sQ[t * LDH + ii] * gm;
                sKG[t * (D + 4) + i] = kt * gm;
                kb[(slot * C + t) * D + i] = kt * sR[t * LDH + ii] * after;
            }
            if (bb == kNB - 1) gC[slot * D + i] = before * bp[kNB - 1];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int job = wave + 4 * j;
            const int mat = job / 6, pr = job % 6;
            const int bt = pr < 1 ? 1 : (pr < 3 ? 2 : 3);
            const int bs = pr - bt * (bt - 1) / 2;
            const float *sX = mat == 0 ? sK : sQ;
            acc[j] = mm16<DH>(
                [&](int rr, int kk) { return sX[(16 * bt + rr) * LDH + kk] * sF[(16 * bt + rr) * LDH + kk]; },
                [&](int cc, int kk) {
                    return sK[(16 * bs + cc) * LDH + kk] * sR[(16 * bs + cc) * LDH + kk] * sMid[pr * DH + kk];
                },
                acc[j]);
        }
        __syncthreads();
        // Sub-block pivots (replacing the block ones): F4, R4 and whole-sub-block products B4.
        float *sB4 = sMid;
        {
            // Thread (channel, block): its four sub-blocks.
            const int ii = tid % DH, bb = tid / DH;
#pragma unroll
            for (int u = 4 * bb; u < 4 * bb + 4; ++u) {
                float run = 1.f;
#pragma unroll
                for (int tl = 0; tl < 4; ++tl) {
                    run *= sA[(4 * u + tl) * LDH + ii];
                    sF[(4 * u + tl) * LDH + ii] = run;
                }
                run = 1.f;
#pragma unroll
                for (int tl = 3; tl >= 0; --tl) {
                    sR[(4 * u + tl) * LDH + ii] = run;
                    run *= sA[(4 * u + tl) * LDH + ii];
                }
                sB4[u * DH + ii] = run;
            }
        }
        __syncthreads();
        // Cross-sub-block entries of the diagonal tiles: for gap g (ut = us + g), the s side
        // carries K * R4 times the products of the g - 1 whole sub-blocks after s's.
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int job = wave + 4 * j;
            const int mat = job / 4, bb = job % 4;
            const float *sX = mat == 0 ? sK : sQ;
            const int rr = lane & 15, kq = lane >> 4;
            const int us = rr >> 2;  // the B row (column s = 16 bb + rr) sub-block in the block
            // Inside one sub-block the split repeats at its halves: t in the upper half, s in
            // the lower takes (a from the half's start through t) x (a after s to the half's
            // end); t = s + 1 in one half takes a_t; t = s takes 1.
            const int sub = rr & 3;  // the A row's (and B column's) place in its sub-block
            f32x4_t y[6] = {zero4(), zero4(), zero4(), zero4(), zero4(), zero4()};
#pragma unroll 4
            for (int m = 0; m < DH / 4; ++m) {
                const int kk = 4 * m + kq;
                const int ta = 16 * bb + rr;
                const float xt = sX[ta * LDH + kk], ks = sK[ta * LDH + kk];
                const float at = sA[ta * LDH + kk];
                const float aprev = sA[(sub > 0 ? ta - 1 : ta) * LDH + kk];
                const float anext = sA[(sub < 3 ? ta + 1 : ta) * LDH + kk];
                const float av = xt * sF[ta * LDH + kk];
                const float b1 = ks * sR[ta * LDH + kk];
                const int u0 = 4 * bb + us;  // s's sub-block in the chunk
                const float m1 = us + 1 < 4 ? sB4[(u0 + 1) * DH + kk] : 0.f;
                const float m2 = us + 2 < 4 ? sB4[(u0 + 2) * DH + kk] : 0.f;
                const float b2 = b1 * m1, b3 = b2 * m2;
                const float f2 = sub == 2 ? at : (sub == 3 ? aprev * at : 0.f);
                const float r2 = sub == 0 ? anext : (sub == 1 ? 1.f : 0.f);
                y[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b1, y[0], 0, 0, 0);
                y[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b2, y[1], 0, 0, 0);
                y[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b3, y[2], 0, 0, 0);
                y[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(xt * f2, ks * r2, y[3], 0, 0, 0);
                y[4] = __builtin_amdgcn_mfma_f32_16x16x4f32(xt * at, ks, y[4], 0, 0, 0);
                y[5] = __builtin_amdgcn_mfma_f32_16x16x4f32(xt, ks, y[5], 0, 0, 0);
            }
            // Output lane l: rows 4 (l / 16) + i (sub-block l / 16), column l % 16.
            const int ut = lane >> 4, sc = lane & 15, usc = sc >> 2;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tr = 4 * ut + i;  // row within the block
                const int gap = ut - usc;
                float add = gap == 1 ? y[0][i] : (gap == 2 ? y[1][i] : (gap == 3 ? y[2][i] : 0.f));
                if (gap == 0) {
                    if ((tr & 3) >= 2 && (sc & 3) < 2) add = y[3][i];
                    else if ((tr & 1) == 1 && sc == tr - 1) add = y[4][i];
                    else if (sc == tr && mat == 1) add = y[5][i];
                }
                dacc[j][i] += add;
            }
        }
    }
    __syncthreads();
    // M and P into LDS (the upper parts and M's diagonal stay zero).
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int job = wave + 4 * j;
        const int mat = job / 6, pr = job % 6;
        const int bt = pr < 1 ? 1 : (pr < 3 ? 2 : 3);
        const int bs = pr - bt * (bt - 1) / 2;
        float *dst = mat == 0 ? sM : sP;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(16 * bt + 4 * (lane >> 4) + i) * LDM + 16 * bs + (lane & 15)] = acc[j][i];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int job = wave + 4 * j;
        const int mat = job / 4, bb = job % 4;
        float *dst = mat == 0 ? sM : sP;
        const int ut = lane >> 4, sc = lane & 15;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (sc <= 4 * ut + i) dst[(16 * bb + 4 * ut + i) * LDM + 16 * bb + sc] = dacc[j][i];
    }
    __syncthreads();
    for (int idx = tid; idx < C * C; idx += kBwdThreads) {
        const int t = idx / C, s = idx % C;
        Mw[slot * C * C + idx] = sM[t * LDM + s];
        Pw[slot * C * C + idx] = sP[s * LDM + t];  // P transposed: row t holds P[., t]
    }
    // p = (K*gamma) S0 + M U, [C x D]: wave w owns value-column tiles w, w + 4, ...
    const float *S0 = states + (size_t(bh) * (nchunks + 1) + c) * D * D;
    const float *Ub = u + (size_t(b) * T + c0) * HD + size_t(h) * D;
    for (int jt = wave; jt < D / 16; jt += 4) {
        // This lane's B operands of every contraction step, loaded together.
        const int cc = lane & 15, kq = lane >> 4;
        float bS[D / 4], bU[C / 4];
#pragma unroll
        for (int m = 0; m < D / 4; ++m) bS[m] = S0[size_t(4 * m + kq) * D + 16 * jt + cc];
#pragma unroll
        for (int m = 0; m < C / 4; ++m)
            bU[m] = 4 * m + kq < nval ? Ub[size_t(4 * m + kq) * HD + 16 * jt + cc] : 0.f;
#pragma unroll
        for (int tt = 0; tt < kNB; ++tt) {
            f32x4_t y = zero4();
#pragma unroll
            for (int m = 0; m < D / 4; ++m)
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(sKG[(16 * tt + cc) * (D + 4) + 4 * m + kq], bS[m], y, 0, 0, 0);
#pragma unroll
            for (int m = 0; m < C / 4; ++m)
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(sM[(16 * tt + cc) * LDM + 4 * m + kq], bU[m], y, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tt + 4 * (lane >> 4) + i;
                if (t < nval) pred[tok0 + size_t(t) * HD + 16 * jt + (lane & 15)] = y[i];
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// Reverse scan over chunks, per (b, h, 16 value columns); four wavefronts.
//   right-hand side  (K*beta) lambda_C + P^T dO: fp32 matrix cores, wave w owns tokens
//                    16w .. 16w + 15; its A operands come straight from memory into registers,
//                    loaded while the previous chunk is finished.
//   solve            back substitution, wave w owns columns 4w .. 4w + 3, lane = token.
//   adjoint carry    lambda <- Diag(gamma_C) lambda + (Q_hat*gamma)^T dO + (K*gamma)^T dP:
//                    matrix cores, wave w owns channel tiles w, w + 4, ...
// Matrix-core contraction order: step (mo, mi) of lane group kq takes k = 16 mo + 4 kq + mi, so
// a lane's four A values of one mo are adjacent in memory (one 16-byte load) and the B reads
// from rows of 20 floats fall in distinct LDS banks.
// LDS: lambda [D][20], dO and dP [C][20], M [C][C + 1], per-token tiles [C][17] of e, w, v, p
// and the right-hand side, gamma_C [D].
// ------------------------------------------------------------------------------------------
constexpr int kVTS = 16;  // value columns per scan workgroup
template <int D> struct ScanBwdLds {
    static constexpr int LDM = kC + 1, LDT = kVTS + 1, LDB = kVTS + 4;
    static constexpr int FLOATS = D * LDB + 2 * kC * LDB + kC * LDM + 5 * kC * LDT + D;
    static constexpr size_t BYTES = size_t(FLOATS) * 4;
};

template <typename QT, int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_scan_kernel(
    const QT *__restrict__ dout, const QT *__restrict__ v, const float *__restrict__ e,
    const float *__restrict__ w, const float *__restrict__ kb, const float *__restrict__ kg,
    const float *__restrict__ qg, const float *__restrict__ gC, const float *__restrict__ Mw,
    const float *__restrict__ Pw, const float *__restrict__ pred, const float *__restrict__ dsT,
    float *__restrict__ dU, float *__restrict__ lamC, float *__restrict__ dv,
    float *__restrict__ dw, float *__restrict__ de, float *__restrict__ ds0, int T, int H, int BH,
    int nchunks) {
    using L = ScanBwdLds<D>;
    constexpr int C = kC, VT = kVTS, NVT = D / VT, LDM = L::LDM, LDT = L::LDT, LDB = L::LDB;
    constexpr int NIT = D / 64;  // channel tiles per wave in the adjoint carry
    extern __shared__ float lds[];
    float *sLam = lds, *sdO = sLam + D * LDB, *sdP = sdO + C * LDB, *sM = sdP + C * LDB;
    float *sE = sM + C * LDM, *sW = sE + C * LDT, *sV = sW + C * LDT, *sPr = sV + C * LDT;
    float *sRhs = sPr + C * LDT, *sGC = sRhs + C * LDT;

    // The value tiles of one head get ids equal mod 8, so they share an XCD and its L2.
    const int id = blockIdx.x;
    const int bh = (id >> 3) / NVT * 8 + (id & 7);
    const int ct = (id >> 3) % NVT;
    if (bh >= BH) return;
    const int b = bh / H, h = bh % H;
    const int j0 = VT * ct;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    const size_t HD = size_t(H) * D;
    auto tok_base = [&](int c) { return (size_t(b) * T + size_t(c) * C) * HD + size_t(h) * D + j0; };
    auto slot_of = [&](int c) { return size_t(bh) * nchunks + c; };

    // Matrix-core A operands: K*beta and P^T rows of this wave's tokens; Q_hat*gamma and
    // K*gamma (channel-major) rows of this wave's channel tiles.
    f32x4_t aKB[D / 16], aP[C / 16], aQG[NIT][C / 16], aKG[NIT][C / 16];
    auto load_rhsA = [&](int c) {
        const size_t sl = slot_of(c);
#pragma unroll
        for (int mo = 0; mo < D / 16; ++mo) aKB[mo] = ld4(kb, (sl * C + 16 * wave + r) * D + 16 * mo + 4 * kq);
#pragma unroll
        for (int mo = 0; mo < C / 16; ++mo) aP[mo] = ld4(Pw, (sl * C + 16 * wave + r) * C + 16 * mo + 4 * kq);
    };
    auto load_lamA = [&](int c) {
        const size_t sl = slot_of(c);
#pragma unroll
        for (int n = 0; n < NIT; ++n)
#pragma unroll
            for (int mo = 0; mo < C / 16; ++mo) {
                const size_t o = (sl * D + 16 * (wave + 4 * n) + r) * C + 16 * mo + 4 * kq;
                aQG[n][mo] = ld4(qg, o);
                aKG[n][mo] = ld4(kg, o);
            }
    };
    // Staged through LDS: M, the per-token tiles (thread: token tid / 4, columns 4 (tid % 4)
    // .. + 3) and gamma_C.
    struct Stage {
        f32x4_t m[C * C / 4 / kBwdThreads];
        f32x4_t dO, e, w, v, pr;
        float gc;
    } st;
    auto load_stage = [&](int c) {
        const size_t sl = slot_of(c);
        const f32x4_t *M4 = reinterpret_cast<const f32x4_t *>(Mw + sl * C * C);
#pragma unroll
        for (int j = 0; j < C * C / 4 / kBwdThreads; ++j) st.m[j] = M4[tid + kBwdThreads * j];
        const int t = tid >> 2, c4 = 4 * (tid & 3);
        if (t < min(C, T - c * C)) {
            const size_t o = tok_base(c) + size_t(t) * HD + c4;
            st.dO = ld4(dout, o);
            st.e = ld4(e, o);
            st.w = ld4(w, o);
            st.v = ld4(v, o);
            st.pr = ld4(pred, o);
        } else {
            st.dO = st.e = st.w = st.v = st.pr = zero4();
        }
        st.gc = tid < D ? gC[sl * D + tid] : 0.f;
    };
    auto store_stage = [&]() {
#pragma unroll
        for (int j = 0; j < C * C / 4 / kBwdThreads; ++j) {
            const int e0 = 4 * (tid + kBwdThreads * j), t = e0 / C, s = e0 % C;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) sM[t * LDM + s + q4] = st.m[j][q4];
        }
        const int t = tid >> 2, c4 = 4 * (tid & 3);
        *reinterpret_cast<f32x4_t *>(&sdO[t * LDB + c4]) = st.dO;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            sE[t * LDT + c4 + q4] = st.e[q4];
            sW[t * LDT + c4 + q4] = st.w[q4];
            sV[t * LDT + c4 + q4] = st.v[q4];
            sPr[t * LDT + c4 + q4] = st.pr[q4];
        }
        if (tid < D) sGC[tid] = st.gc;
    };

    for (int idx = tid; idx < D * VT; idx += kBwdThreads) {
        const int i = idx / VT, j = idx % VT;
        sLam[i * LDB + j] = dsT ? dsT[(size_t(bh) * D + i) * D + j0 + j] : 0.f;
    }
    if (nchunks > 0) {
        load_stage(nchunks - 1);
        load_rhsA(nchunks - 1);
        load_lamA(nchunks - 1);
    }
    for (int c = nchunks - 1; c >= 0; --c) {
        const int nval = min(C, T - c * C);
        const size_t tok0 = tok_base(c);
        const size_t slot = slot_of(c);
        __syncthreads();
        store_stage();
        for (int idx = tid; idx < D * VT; idx += kBwdThreads) {
            const int i = idx / VT, j = idx % VT;
            lamC[(slot * D + i) * D + j0 + j] = sLam[i * LDB + j];
        }
        __syncthreads();
        if (c > 0) load_stage(c - 1);
        // Right-hand side of this wave's 16 tokens.
        {
            f32x4_t y = zero4();
#pragma unroll
            for (int mo = 0; mo < D / 16; ++mo)
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
                    y = __builtin_amdgcn_mfma_f32_16x16x4f32(aKB[mo][mi], sLam[(16 * mo + 4 * kq + mi) * LDB + r], y, 0, 0, 0);
#pragma unroll
            for (int mo = 0; mo < C / 16; ++mo)
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
                    y = __builtin_amdgcn_mfma_f32_16x16x4f32(aP[mo][mi], sdO[(16 * mo + 4 * kq + mi) * LDB + r], y, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) sRhs[(16 * wave + 4 * kq + i) * LDT + r] = y[i];
        }
        if (c > 0) load_rhsA(c - 1);
        __syncthreads();
        // Back substitution. With y = e * dU, dU_t = rhs_t - sum_{s > t} M_st y_s; lanes t >= s
        // read M_st = 0.
        {
            const int j = 4 * wave;
            float x[4], ev[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                x[q4] = sRhs[lane * LDT + j + q4];
                ev[q4] = sE[lane * LDT + j + q4];
            }
#pragma unroll
            for (int s = C - 1; s >= 0; --s) {
                const float m = sM[s * LDM + lane];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const float ys = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ev[q4] * x[q4]), s));
                    x[q4] = fmaf(-m, ys, x[q4]);
                }
            }
            f32x4_t xu, xv, xw, xe;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                sdP[lane * LDB + j + q4] = -ev[q4] * x[q4];
                xu[q4] = x[q4];
                xv[q4] = sW[lane * LDT + j + q4] * x[q4];
                xw[q4] = sV[lane * LDT + j + q4] * x[q4];
                xe[q4] = -sPr[lane * LDT + j + q4] * x[q4];
            }
            if (lane < nval) {
                const size_t o = tok0 + size_t(lane) * HD + j;
                *reinterpret_cast<f32x4_t *>(dU + o) = xu;
                *reinterpret_cast<f32x4_t *>(dv + o) = xv;
                *reinterpret_cast<f32x4_t *>(dw + o) = xw;
                *reinterpret_cast<f32x4_t *>(de + o) = xe;
            }
        }
        __syncthreads();
        // Adjoint carry for this wave's channel tiles.
#pragma unroll
        for (int n = 0; n < NIT; ++n) {
            const int i0 = 16 * (wave + 4 * n);
            f32x4_t y;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ii = i0 + 4 * kq + i;
                y[i] = sGC[ii] * sLam[ii * LDB + r];
            }
#pragma unroll
            for (int mo = 0; mo < C / 16; ++mo)
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    const int tt = 16 * mo + 4 * kq + mi;
                    y = __builtin_amdgcn_mfma_f32_16x16x4f32(aQG[n][mo][mi], sdO[tt * LDB + r], y, 0, 0, 0);
                    y = __builtin_amdgcn_mfma_f32_16x16x4f32(aKG[n][mo][mi], sdP[tt * LDB + r], y, 0, 0, 0);
                }
#pragma unroll
            for (int i = 0; i < 4; ++i) sLam[(i0 + 4 * kq + i) * LDB + r] = y[i];
        }
        if (c > 0) load_lamA(c - 1);
    }
    __syncthreads();
    if (ds0) {
        for (int idx = tid; idx < D * VT; idx += kBwdThreads) {
            const int i = idx / VT, j = idx % VT;
            ds0[(size_t(bh) * D + i) * D + j0 + j] = sLam[i * LDB + j];
        }
    }
}

// ------------------------------------------------------------------------------------------
// Chunk-parallel gradients. LDS: O U^T and dP U^T [C][C + 1]; then a union of U, dO, dP
// [C][D + 4] (products) and k, a, q_hat channel-major [D][C + 1] (decayed sums).
// ------------------------------------------------------------------------------------------
template <int D> struct GradLds {
    // Rows of DH = 16 floats: a matrix-core step reads 4 rows x 16 channels, one bank each.
    static constexpr int LDM = kC + 1, DH = 16, LDH = DH;
    static constexpr int OUPU = 2 * kC * LDM;
    // Per 16-channel pass: a, k, q_hat, F, R (16-token blocks), F4, R4 (4-token sub-blocks)
    // [C][16]; products of whole blocks between (6 pairs), of whole sub-blocks (16), of the
    // blocks before and after each block (4 + 4), per channel. About 67 KB in all for d = 128,
    // so two workgroups share a compute unit.
    static constexpr int P2 = 7 * kC * LDH + (6 + 16 + 4 + 4) * DH;
    static constexpr int FLOATS = OUPU + 2 * D + (P2 > kBwdThreads ? P2 : kBwdThreads) + kNB * DH;
    static constexpr size_t BYTES = size_t(FLOATS) * 4;
};

template <typename QT, int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_grads_kernel(
    const QT *__restrict__ q, const QT *__restrict__ k, const QT *__restrict__ dout,
    const float *__restrict__ a, const float *__restrict__ g, const float *__restrict__ e,
    const float *__restrict__ r, const float *__restrict__ U, const float *__restrict__ dU,
    const float *__restrict__ states, const float *__restrict__ lamC, float *__restrict__ X3,
    float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dg,
    float *__restrict__ dla, float *__restrict__ drp, int T, int H, int nchunks) {
    using L = GradLds<D>;
    constexpr int C = kC, LDM = L::LDM, LDH = L::LDH, DH = L::DH;
    extern __shared__ float lds[];
    float *sOU = lds, *sPU = lds + C * LDM;
    float *sRS = lds + L::OUPU;  // rowsum(S_C * lambda_C) per channel
    float *sDr = sRS + D;        // sum over tokens of g * q * dq_hat per channel
    float *un = sDr + D;
    float *sA = un, *sK = sA + C * LDH, *sQ = sK + C * LDH, *sF = sQ + C * LDH, *sR = sF + C * LDH,
          *sF4 = sR + C * LDH, *sR4 = sF4 + C * LDH, *sMid = sR4 + C * LDH, *sB4 = sMid + 6 * DH,
          *sGb = sB4 + 16 * DH, *sBa = sGb + 4 * DH;
    float *sBp = lds + L::FLOATS - kNB * DH;  // whole-block decay products per channel

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int bh = b * H + h;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const size_t HD = size_t(H) * D;
    const int c0 = c * C;
    const int nval = min(C, T - c0);
    const size_t tok0 = (size_t(b) * T + c0) * HD + size_t(h) * D;
    const size_t slot = size_t(bh) * nchunks + c;
    const float *S0 = states + (size_t(bh) * (nchunks + 1) + c) * D * D;
    const float *SC = S0 + size_t(D) * D;
    const float *lam = lamC + slot * D * D;

    // Rows of U, dO and dP = -e * dU as matrix-core operands straight from memory: 16 bytes per
    // load, contraction step (mo, mi) of lane group kq taking k = 16 mo + 4 kq + mi. Tokens past
    // the sequence read as zero.
    const int rr = lane & 15, kq = lane >> 4;
    auto rowU = [&](int t, f32x4_t (&x)[D / 16]) {
#pragma unroll
        for (int mo = 0; mo < D / 16; ++mo)
            x[mo] = t < nval ? ld4(U, tok0 + size_t(t) * HD + 16 * mo + 4 * kq) : zero4();
    };
    auto rowO = [&](int t, f32x4_t (&x)[D / 16]) {
#pragma unroll
        for (int mo = 0; mo < D / 16; ++mo)
            x[mo] = t < nval ? ld4(dout, tok0 + size_t(t) * HD + 16 * mo + 4 * kq) : zero4();
    };
    auto rowP = [&](int t, f32x4_t (&x)[D / 16]) {
#pragma unroll
        for (int mo = 0; mo < D / 16; ++mo) {
            const size_t o = tok0 + size_t(t) * HD + 16 * mo + 4 * kq;
            x[mo] = t < nval ? -ld4(e, o) * ld4(dU, o) : zero4();
        }
    };
    // rowsum(S_C * lambda_C): thread (row, part) sums a contiguous segment of the row, every
    // load issued before the first use; the parts meet through LDS atomics.
    {
        constexpr int TPR = kBwdThreads / D;  // threads per row
        constexpr int SEG = D / TPR;          // elements per thread
        const int i = tid / TPR, part = tid % TPR;
        f32x4_t xs[SEG / 4], xl[SEG / 4];
#pragma unroll
        for (int j = 0; j < SEG / 4; ++j) {
            xs[j] = ld4(SC, size_t(i) * D + part * SEG + 4 * j);
            xl[j] = ld4(lam, size_t(i) * D + part * SEG + 4 * j);
        }
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < SEG / 4; ++j)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) acc = fmaf(xs[j][q4], xl[j][q4], acc);
        if (part == 0) sRS[i] = 0.f;
        __syncthreads();
        atomicAdd(&sRS[i], acc);
    }
    for (int i = tid; i < D; i += kBwdThreads) sDr[i] = 0.f;
    __syncthreads();
    // O U^T (s <= t) and dP U^T (s < t), lower 16x16 tiles; job j < 20: matrix j / 10, tile
    // j % 10 = bt (bt + 1) / 2 + bs.
    for (int job = wave; job < 20; job += 4) {
        const int mat = job / 10, tl = job % 10;
        const int bt = tl < 1 ? 0 : (tl < 3 ? 1 : (tl < 6 ? 2 : 3));
        const int bs = tl - bt * (bt + 1) / 2;
        f32x4_t xa[D / 16], xb[D / 16];
        if (mat == 0) rowO(16 * bt + rr, xa);
        else rowP(16 * bt + rr, xa);
        rowU(16 * bs + rr, xb);
        f32x4_t y = zero4();
#pragma unroll
        for (int mo = 0; mo < D / 16; ++mo)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) y = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[mo][mi], xb[mo][mi], y, 0, 0, 0);
        float *dst = mat == 0 ? sOU : sPU;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * bt + 4 * (lane >> 4) + i, s = 16 * bs + (lane & 15);
            dst[t * LDM + s] = (mat == 0 ? s <= t : s < t) ? y[i] : 0.f;
        }
    }
    // dO S0^T -> dq, dP S0^T -> dk, U lambda_C^T -> X3 (unscaled), [C x D]. Wave w owns the
    // channel tiles w + 4 j; its rows of S0 (then lambda_C) stay in registers over the four
    // token tiles, so each state is read from memory once per chunk.
    constexpr int NTW = D / 64;  // channel tiles per wave
    {
        f32x4_t bv[NTW][D / 16];
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int mo = 0; mo < D / 16; ++mo)
                bv[j][mo] = ld4(S0, size_t(16 * (wave + 4 * j) + rr) * D + 16 * mo + 4 * kq);
#pragma unroll 1
        for (int tt = 0; tt < kNB; ++tt) {
            f32x4_t xo[D / 16], xp[D / 16];
            rowO(16 * tt + rr, xo);
            rowP(16 * tt + rr, xp);
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int it = wave + 4 * j;
                f32x4_t y1 = zero4(), y2 = zero4();
#pragma unroll
                for (int mo = 0; mo < D / 16; ++mo)
#pragma unroll
                    for (int mi = 0; mi < 4; ++mi) {
                        y1 = __builtin_amdgcn_mfma_f32_16x16x4f32(xo[mo][mi], bv[j][mo][mi], y1, 0, 0, 0);
                        y2 = __builtin_amdgcn_mfma_f32_16x16x4f32(xp[mo][mi], bv[j][mo][mi], y2, 0, 0, 0);
                    }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * tt + 4 * kq + i;
                    if (t < nval) {
                        const size_t o = tok0 + size_t(t) * HD + 16 * it + rr;
                        dq[o] = y1[i];
                        dk[o] = y2[i];
                    }
                }
            }
        }
    }
    {
        f32x4_t bv[NTW][D / 16];
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int mo = 0; mo < D / 16; ++mo)
                bv[j][mo] = ld4(lam, size_t(16 * (wave + 4 * j) + rr) * D + 16 * mo + 4 * kq);
#pragma unroll 1
        for (int tt = 0; tt < kNB; ++tt) {
            f32x4_t xu[D / 16];
            rowU(16 * tt + rr, xu);
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int it = wave + 4 * j;
                f32x4_t y3 = zero4();
#pragma unroll
                for (int mo = 0; mo < D / 16; ++mo)
#pragma unroll
                    for (int mi = 0; mi < 4; ++mi)
                        y3 = __builtin_amdgcn_mfma_f32_16x16x4f32(xu[mo][mi], bv[j][mo][mi], y3, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * tt + 4 * kq + i;
                    if (t < nval) X3[tok0 + size_t(t) * HD + 16 * it + rr] = y3[i];
                }
            }
        }
    }
    __syncthreads();
    const float *rh = r + size_t(h) * D;
    // Decayed sums over token pairs, per 16-channel pass, on the matrix cores. With the pivots
    // of the prepare kernel, Gamma_ts = F_t * mid * R_s across 16-token blocks and
    // F4_t * mid4 * R4_s across 4-token sub-blocks of one block; pairs inside one sub-block are
    // direct products. Jobs: kind 0 (dq_hat and the read part of dk, rows = t) and kind 1 (the
    // write part of dk, rows = s), one 16-row block each; wave w takes jobs w and w + 4.
    for (int p0 = 0; p0 < D; p0 += DH) {
        if (p0 > 0) __syncthreads();
        {
            constexpr int N4 = C * DH / 4 / kBwdThreads;
            f32x4_t va[N4], vk[N4], vq[N4];
#pragma unroll
            for (int j = 0; j < N4; ++j) {
                const int e0 = 4 * (tid + kBwdThreads * j), t = e0 / DH, ii = e0 % DH;
                const size_t o = tok0 + size_t(t) * HD + p0 + ii;
                if (t < nval) {
                    va[j] = ld4(a, o);
                    vk[j] = ld4(k, o);
                    vq[j] = ld4(g, o) * ld4(q, o) * ld4(rh, p0 + ii);
                } else {
                    va[j] = f32x4_t{1.f, 1.f, 1.f, 1.f};
                    vk[j] = vq[j] = zero4();
                }
            }
#pragma unroll
            for (int j = 0; j < N4; ++j) {
                const int e0 = 4 * (tid + kBwdThreads * j), t = e0 / DH, ii = e0 % DH;
                *reinterpret_cast<f32x4_t *>(&sA[t * LDH + ii]) = va[j];
                *reinterpret_cast<f32x4_t *>(&sK[t * LDH + ii]) = vk[j];
                *reinterpret_cast<f32x4_t *>(&sQ[t * LDH + ii]) = vq[j];
            }
        }
        __syncthreads();
        if (tid < DH * kNB) {
            // Thread (channel, 16-token block): prefix and suffix products inside the block
            // and inside its four sub-blocks.
            const int ii = tid % DH, bb = tid / DH;
            float run = 1.f;
#pragma unroll
            for (int tl = 0; tl < 16; ++tl) {
                run *= sA[(16 * bb + tl) * LDH + ii];
                sF[(16 * bb + tl) * LDH + ii] = run;
            }
            run = 1.f;
#pragma unroll
            for (int tl = 15; tl >= 0; --tl) {
                sR[(16 * bb + tl) * LDH + ii] = run;
                run *= sA[(16 * bb + tl) * LDH + ii];
            }
            sBp[bb * DH + ii] = run;
#pragma unroll
            for (int u = 4 * bb; u < 4 * bb + 4; ++u) {
                float r4 = 1.f;
#pragma unroll
                for (int tl = 0; tl < 4; ++tl) {
                    r4 *= sA[(4 * u + tl) * LDH + ii];
                    sF4[(4 * u + tl) * LDH + ii] = r4;
                }
                r4 = 1.f;
#pragma unroll
                for (int tl = 3; tl >= 0; --tl) {
                    sR4[(4 * u + tl) * LDH + ii] = r4;
                    r4 *= sA[(4 * u + tl) * LDH + ii];
                }
                sB4[u * DH + ii] = r4;
            }
        }
        __syncthreads();
        if (tid < DH) {
            const int ii = tid;
            float bp[kNB];
#pragma unroll
            for (int bb = 0; bb < kNB; ++bb) bp[bb] = sBp[bb * DH + ii];
#pragma unroll
            for (int bt = 1; bt < kNB; ++bt) {
                float mid = 1.f;
#pragma unroll
                for (int bs = bt - 1; bs >= 0; --bs) {
                    sMid[(bt * (bt - 1) / 2 + bs) * DH + ii] = mid;
                    mid *= bp[bs];
                }
            }
            float before = 1.f;
#pragma unroll
            for (int bb = 0; bb < kNB; ++bb) {
                sGb[bb * DH + ii] = before;
                before *= bp[bb];
            }
            float after = 1.f;
#pragma unroll
            for (int bb = kNB - 1; bb >= 0; --bb) {
                sBa[bb * DH + ii] = after;
                after *= bp[bb];
            }
        }
        __syncthreads();
        for (int job = wave; job < 2 * kNB; job += 4) {
            const int kind = job / kNB, rb = job % kNB, it = 0;
            const int ic = 16 * it + rr;  // this lane's B / output column, within the pass
            const size_t ocol = size_t(p0 + ic);
            if (kind == 0) {
                // Rows t of block bt = rb. The rows' global operands are loaded first.
                const int bt = rb;
                float gx1[4], gx2[4], gg[4], gq[4];
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int t = 16 * bt + 4 * kq + e4;
                    const size_t o = tok0 + size_t(t) * HD + ocol;
                    const bool ok = t < nval;
                    gx1[e4] = ok ? dq[o] : 0.f;
                    gx2[e4] = ok ? dk[o] : 0.f;
                    gg[e4] = ok ? g[o] : 0.f;
                    gq[e4] = ok ? ld(q, o) : 0.f;
                }
                f32x4_t cq = zero4(), cr = zero4(), dq4 = zero4(), dr4 = zero4();
#pragma unroll
                for (int bs = 0; bs < kNB - 1; ++bs) {
                    if (bs >= bt) break;
                    f32x4_t yq = zero4(), yr = zero4();
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int kk = 4 * m + kq, sg = 16 * bs + kk;
                        const float b = sK[sg * LDH + ic] * sR[sg * LDH + ic];
                        yq = __builtin_amdgcn_mfma_f32_16x16x4f32(sOU[(16 * bt + rr) * LDM + sg], b, yq, 0, 0, 0);
                        yr = __builtin_amdgcn_mfma_f32_16x16x4f32(sPU[(16 * bt + rr) * LDM + sg], b, yr, 0, 0, 0);
                    }
                    const float md = sMid[(bt * (bt - 1) / 2 + bs) * DH + ic];
                    cq += md * yq;
                    cr += md * yr;
                }
#pragma unroll
                for (int gp = 1; gp < 4; ++gp) {
                    f32x4_t yq = zero4(), yr = zero4();
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int kk = 4 * m + kq, sg = 16 * bt + kk;
                        const int us = kk >> 2;
                        const bool on = (rr >> 2) - us == gp;
                        float mid4 = 1.f;
                        if (gp >= 2) mid4 = us + 1 < 4 ? sB4[(4 * bt + us + 1) * DH + ic] : 0.f;
                        if (gp == 3) mid4 *= us + 2 < 4 ? sB4[(4 * bt + us + 2) * DH + ic] : 0.f;
                        const float b = sK[sg * LDH + ic] * sR4[sg * LDH + ic] * mid4;
                        const float aq = on ? sOU[(16 * bt + rr) * LDM + sg] : 0.f;
                        const float ar = on ? sPU[(16 * bt + rr) * LDM + sg] : 0.f;
                        yq = __builtin_amdgcn_mfma_f32_16x16x4f32(aq, b, yq, 0, 0, 0);
                        yr = __builtin_amdgcn_mfma_f32_16x16x4f32(ar, b, yr, 0, 0, 0);
                    }
                    dq4 += yq;
                    dr4 += yr;
                }
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int t = 16 * bt + 4 * kq + e4;
                    // Pairs inside t's sub-block: s = t, t - 1, ... down to its start (a fixed
                    // four-step loop; steps below the start add nothing).
                    float sq = 0.f, sr = 0.f, run = 1.f;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int s4 = t - u;
                        const bool on = u <= (t & 3);
                        const int sc = on ? s4 : t;
                        const float ks = on ? run * sK[sc * LDH + ic] : 0.f;
                        sq = fmaf(sOU[t * LDM + sc], ks, sq);
                        sr = fmaf(sPU[t * LDM + sc], ks, sr);
                        run *= sA[sc * LDH + ic];
                    }
                    const float fb = sF[t * LDH + ic], f4 = sF4[t * LDH + ic];
                    if (t < nval) {
                        const size_t o = tok0 + size_t(t) * HD + ocol;
                        const float gam = sGb[bt * DH + ic] * fb;
                        const float dqh = gam * gx1[e4] + fb * cq[e4] + f4 * dq4[e4] + sq;
                        const float dkr = gam * gx2[e4] + fb * cr[e4] + f4 * dr4[e4] + sr;
                        const float gt = gg[e4], qt = gq[e4];
                        dq[o] = rh[ocol] * gt * dqh;
                        dg[o] = rh[ocol] * qt * dqh;
                        dk[o] = dkr;
                        dla[o] = fmaf(sQ[t * LDH + ic], dqh, sK[t * LDH + ic] * dkr);
                        atomicAdd(&sDr[ocol], gt * qt * dqh);
                    }
                }
            } else {
                // Rows s of block bs = rb.
                const int bs = rb;
                float gx3[4];
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int s4 = 16 * bs + 4 * kq + e4;
                    gx3[e4] = s4 < nval ? X3[tok0 + size_t(s4) * HD + ocol] : 0.f;
                }
                f32x4_t cw = zero4(), dw4 = zero4();
#pragma unroll
                for (int bt = 1; bt < kNB; ++bt) {
                    if (bt <= bs) continue;
                    f32x4_t y = zero4();
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int kk = 4 * m + kq, tg = 16 * bt + kk;
                        const float f = sF[tg * LDH + ic];
                        y = __builtin_amdgcn_mfma_f32_16x16x4f32(sOU[tg * LDM + 16 * bs + rr], sQ[tg * LDH + ic] * f, y, 0, 0, 0);
                        y = __builtin_amdgcn_mfma_f32_16x16x4f32(sPU[tg * LDM + 16 * bs + rr], sK[tg * LDH + ic] * f, y, 0, 0, 0);
                    }
                    cw += sMid[(bt * (bt - 1) / 2 + bs) * DH + ic] * y;
                }
#pragma unroll
                for (int gp = 1; gp < 4; ++gp) {
                    f32x4_t y = zero4();
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int kk = 4 * m + kq, tg = 16 * bs + kk;
                        const int ut = kk >> 2;
                        const bool on = ut - (rr >> 2) == gp;
                        // Products of the gp - 1 whole sub-blocks before t's.
                        float mid4 = 1.f;
                        if (gp >= 2) mid4 = ut - 1 >= 0 ? sB4[(4 * bs + ut - 1) * DH + ic] : 0.f;
                        if (gp == 3) mid4 *= ut - 2 >= 0 ? sB4[(4 * bs + ut - 2) * DH + ic] : 0.f;
                        const float f = sF4[tg * LDH + ic] * mid4;
                        const float ao = on ? sOU[tg * LDM + 16 * bs + rr] : 0.f;
                        const float ap = on ? sPU[tg * LDM + 16 * bs + rr] : 0.f;
                        y = __builtin_amdgcn_mfma_f32_16x16x4f32(ao, sQ[tg * LDH + ic] * f, y, 0, 0, 0);
                        y = __builtin_amdgcn_mfma_f32_16x16x4f32(ap, sK[tg * LDH + ic] * f, y, 0, 0, 0);
                    }
                    dw4 += y;
                }
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int s4 = 16 * bs + 4 * kq + e4;
                    // Pairs inside s's sub-block: t = s, s + 1, ... up to its end (a fixed
                    // four-step loop; steps past the end add nothing).
                    float sw = 0.f, run = 1.f;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const bool on = u <= 3 - (s4 & 3);
                        const int tc = on ? s4 + u : s4;
                        const float wq = on ? run : 0.f;
                        sw = fmaf(sOU[tc * LDM + s4], wq * sQ[tc * LDH + ic], sw);
                        sw = fmaf(sPU[tc * LDM + s4], wq * sK[tc * LDH + ic], sw);
                        run *= sA[(on && u < 3 - (s4 & 3) ? tc + 1 : tc) * LDH + ic];
                    }
                    if (s4 < nval) {
                        const size_t o = tok0 + size_t(s4) * HD + ocol;
                        const float rb_ = sR[s4 * LDH + ic], r4 = sR4[s4 * LDH + ic];
                        const float bet = rb_ * sBa[bs * DH + ic];
                        X3[o] = bet * gx3[e4] + rb_ * cw[e4] + r4 * dw4[e4] + sw;
                    }
                }
            }
        }
    }
    __syncthreads();
    {
        // Log-decay gradient: a reverse cumulative sum over the chunk per channel. Thread (part,
        // channel) takes TP consecutive tokens: suffix sums inside its part, then the totals of
        // the later parts (through LDS) and rowsum(S_C * lambda_C).
        constexpr int NP = kBwdThreads / D, TP = C / NP;
        const int i = tid % D, part = tid / D;
        if (part == 0) drp[slot * D + i] = sDr[i];
        float *sTot = un;  // [NP][D]; the pass arrays are no longer read
        float x3[TP], la[TP], dkv[TP], kv[TP];
#pragma unroll
        for (int u = 0; u < TP; ++u) {
            const int t = part * TP + u;
            const size_t o = tok0 + size_t(t) * HD + i;
            const bool ok = t < nval;
            x3[u] = ok ? X3[o] : 0.f;
            la[u] = ok ? dla[o] : 0.f;
            dkv[u] = ok ? dk[o] : 0.f;
            kv[u] = ok ? ld(k, o) : 0.f;
        }
        float cum[TP];
        float run = 0.f;
#pragma unroll
        for (int u = TP - 1; u >= 0; --u) {
            run += la[u] - kv[u] * x3[u];
            cum[u] = run;
        }
        sTot[part * D + i] = run;
        __syncthreads();
        float off = sRS[i];
        for (int p2 = part + 1; p2 < NP; ++p2) off += sTot[p2 * D + i];
#pragma unroll
        for (int u = 0; u < TP; ++u) {
            const int t = part * TP + u;
            if (t < nval) {
                const size_t o = tok0 + size_t(t) * HD + i;
                dla[o] = cum[u] + off;
                dk[o] = dkv[u] + x3[u];
            }
        }
    }
}

// dr[h] = sum over (b, chunk) of the per-chunk partials: 1024 threads, thread (group, channel)
// sums the rows equal to its group mod G, then the G partial sums are added in a fixed order.
template <int D>
__global__ __launch_bounds__(1024) void bwd_dr_kernel(const float *__restrict__ drp, float *__restrict__ dr,
                                                      int B, int H, int nchunks) {
    constexpr int G = 1024 / D;
    __shared__ float part[G][D];
    const int h = blockIdx.x, i = threadIdx.x % D, grp = threadIdx.x / D;
    const int rows = B * nchunks;
    float acc = 0.f;
#pragma unroll 4
    for (int rw = grp; rw < rows; rw += G) {
        const int b = rw / nchunks, c = rw % nchunks;
        acc += drp[((size_t(b) * H + h) * nchunks + c) * D + i];
    }
    part[grp][i] = acc;
    __syncthreads();
    if (grp == 0) {
        float sum = 0.f;
#pragma unroll
        for (int g2 = 0; g2 < G; ++g2) sum += part[g2][i];
        dr[size_t(h) * D + i] = sum;
    }
}

// Workspace regions, each 256-byte aligned.
struct BwdLayout {
    size_t fwd, o, u, states, kb, kg, qg, gC, M, P, pred, dU, lamC, X3, drp, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool bwd_layout(int B, int T, int H, int d, bool bf16, BwdLayout &L) {
    const size_t fwd = chunk_workspace_bytes(B, T, H, d, kC, bf16);
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
    L.o = take(tok * (bf16 ? 2 : 4));
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
    L.X3 = take(tok * 4);
    L.drp = take(BH * nc * d * 4);
    L.total = off;
    return true;
}

template <typename QT, int D>
hipError_t bwd_typed(const ChunkBwdArgs &x, int B, int T, int H, unsigned char *ws, const BwdLayout &L,
                     hipStream_t stream) {
    const int nchunks = (T + kC - 1) / kC;
    const int BH = B * H;
    float *u = reinterpret_cast<float *>(ws + L.u);
    float *states = reinterpret_cast<float *>(ws + L.states);
    float *kb = reinterpret_cast<float *>(ws + L.kb), *kg = reinterpret_cast<float *>(ws + L.kg);
    float *qg = reinterpret_cast<float *>(ws + L.qg), *gC = reinterpret_cast<float *>(ws + L.gC);
    float *Mw = reinterpret_cast<float *>(ws + L.M), *Pw = reinterpret_cast<float *>(ws + L.P);
    float *pred = reinterpret_cast<float *>(ws + L.pred), *dUw = reinterpret_cast<float *>(ws + L.dU);
    float *lamC = reinterpret_cast<float *>(ws + L.lamC), *X3 = reinterpret_cast<float *>(ws + L.X3);
    float *drp = reinterpret_cast<float *>(ws + L.drp);
    const bool bf16 = std::is_same_v<QT, bf16_t>;
    hipError_t err;
    if (T > 0) {
        err = launch_chunk_prepare(x.q, x.k, x.a, x.g, x.r, B, T, H, D, kC, bf16, ws + L.fwd, stream);
        if (err != hipSuccess) return err;
    }
    err = launch_chunk_scan_save(x.v, x.e, x.w, x.s0, ws + L.o, nullptr, u, states, B, T, H, D, kC, bf16,
                                 ws + L.fwd, stream);
    if (err != hipSuccess) return err;
    const QT *q = static_cast<const QT *>(x.q), *k = static_cast<const QT *>(x.k);
    const QT *v = static_cast<const QT *>(x.v), *dout = static_cast<const QT *>(x.dout);
    if (nchunks > 0) {
        auto kp = bwd_prepare_kernel<QT, D>;
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(kp), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  int(PrepBwdLds<D>::BYTES));
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(kp, dim3(nchunks, H, B), dim3(kBwdThreads), PrepBwdLds<D>::BYTES, stream, q, k,
                           x.a, x.g, x.r, states, u, kb, kg, qg, gC, Mw, Pw, pred, T, H, nchunks);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    constexpr int NVT = D / kVTS;
    auto ks = bwd_scan_kernel<QT, D>;
    err = hipFuncSetAttribute(reinterpret_cast<const void *>(ks), hipFuncAttributeMaxDynamicSharedMemorySize,
                              int(ScanBwdLds<D>::BYTES));
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(ks, dim3((BH + 7) / 8 * 8 * NVT), dim3(kBwdThreads), ScanBwdLds<D>::BYTES, stream,
                       dout, v, x.e, x.w, kb, kg, qg, gC, Mw, Pw, pred, x.dsT, dUw, lamC, x.dv, x.dw, x.de,
                       x.ds0, T, H, BH, nchunks);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (nchunks > 0) {
        auto kgk = bwd_grads_kernel<QT, D>;
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(kgk), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  int(GradLds<D>::BYTES));
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(kgk, dim3(nchunks, H, B), dim3(kBwdThreads), GradLds<D>::BYTES, stream, q, k, dout,
                           x.a, x.g, x.e, x.r, u, dUw, states, lamC, X3, x.dq, x.dk, x.dg, x.dla, drp, T, H,
                           nchunks);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL((bwd_dr_kernel<D>), dim3(H), dim3(1024), 0, stream, drp, x.dr, B, H, nchunks);
    return hipGetLastError();
}

}  // namespace

size_t chunk_bwd_workspace_bytes(int B, int T, int H, int d, bool bf16) {
    if (B < 1 || H < 1 || T < 0 || (d != 64 && d != 128)) return 0;
    BwdLayout L;
    if (!bwd_layout(B, T, H, d, bf16, L)) return 0;
    return L.total;
}

hipError_t launch_chunk_bwd(const ChunkBwdArgs &x, int B, int T, int H, int d, bool bf16, void *workspace,
                            hipStream_t stream) {
    BwdLayout L;
    if (!bwd_layout(B, T, H, d, bf16, L)) return hipErrorInvalidValue;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    if (d == 64) return bf16 ? bwd_typed<bf16_t, 64>(x, B, T, H, ws, L, stream) : bwd_typed<float, 64>(x, B, T, H, ws, L, stream);
    if (d == 128) return bf16 ? bwd_typed<bf16_t, 128>(x, B, T, H, ws, L, stream) : bwd_typed<float, 128>(x, B, T, H, ws, L, stream);
    return hipErrorInvalidValue;
}

}  // namespace muir
