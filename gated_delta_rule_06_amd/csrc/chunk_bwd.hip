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
//   bwd_products_kernel one workgroup per (b, h, chunk): O U^T, dP U^T and the state terms
//                       dO S0^T, dP S0^T, U lambda_C^T.
//   bwd_grads_kernel    one workgroup per (b, h, chunk, 64 key channels): per 16 channels the
//                       decayed pair sums for dq_hat and dk, then dq, dk, dg and a * dL/da (a
//                       reverse cumulative sum per channel).
//   bwd_dr_kernel       dr summed over batch and chunks.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "layout.hpp"
#include "mfma.hpp"

namespace muir {

namespace {

constexpr int kC = kBwdChunk;  // tokens per chunk
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

// Loads whose conversion to fp32 waits until the value is used: a prefetch of bf16 data that
// converted at once would make the wave wait for the load right there.
template <typename QT> struct Raw4 { using type = f32x4_t; };
template <> struct Raw4<bf16_t> { using type = u16x4_t; };
__device__ __forceinline__ f32x4_t raw4(const float *p, size_t i) {
    return *reinterpret_cast<const f32x4_t *>(p + i);
}
__device__ __forceinline__ u16x4_t raw4(const bf16_t *p, size_t i) {
    return *reinterpret_cast<const u16x4_t *>(p + i);
}
__device__ __forceinline__ f32x4_t cvt4(f32x4_t x) { return x; }
__device__ __forceinline__ f32x4_t cvt4(u16x4_t u) {
    return f32x4_t{bf16_to_f32(u[0]), bf16_to_f32(u[1]), bf16_to_f32(u[2]), bf16_to_f32(u[3])};
}

// Products of fp32 operands on the bf16 matrix cores (bf16 path): each fp32 value is carried as
// a bf16 pair hi + lo (hi the nearest bf16, lo the nearest bf16 to the remainder, which is exact
// in fp32), and a product takes hi*hi + hi*lo + lo*hi, leaving out only lo*lo (relative size
// about 2^-16). Per K = 32 step that is three v_mfma_f32_16x16x32_bf16 (16 cycles each) in place
// of eight v_mfma_f32_16x16x4_f32 (32 cycles each). A bf16 input (dO) needs only its hi part.
struct Split {
    Mma<bf16_t>::frag hi, lo;
};
__device__ __forceinline__ Split split8(f32x4_t a, f32x4_t b) {
    using M16 = Mma<bf16_t>;
    const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    Split sp;
    sp.hi = M16::pack(x);
    const u16x8_t hb = __builtin_bit_cast(u16x8_t, sp.hi);
    float rem[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) rem[j] = x[j] - bf16_to_f32(hb[j]);
    sp.lo = M16::pack(rem);
    return sp;
}
__device__ __forceinline__ Split split8(const float (&x)[8]) {
    return split8(f32x4_t{x[0], x[1], x[2], x[3]}, f32x4_t{x[4], x[5], x[6], x[7]});
}
__device__ __forceinline__ f32x4_t mma3(const Split &a, const Split &b, f32x4_t y) {
    using M16 = Mma<bf16_t>;
    y = M16::mma(a.hi, b.hi, y);
    y = M16::mma(a.hi, b.lo, y);
    return M16::mma(a.lo, b.hi, y);
}
__device__ __forceinline__ f32x4_t mma2(Mma<bf16_t>::frag a, const Split &b, f32x4_t y) {
    y = Mma<bf16_t>::mma(a, b.hi, y);
    return Mma<bf16_t>::mma(a, b.lo, y);
}


// ------------------------------------------------------------------------------------------
// Prepare. One workgroup per (b, h, chunk), in passes of 32 channels. LDS per pass: a, k,
// q_hat, and the prefix F and suffix R inside each 16-token block (then inside each 4-token
// sub-block) [C][33], plus per-channel products of whole blocks (then whole sub-blocks). After
// the last pass the same space holds M and P [C][C + 1]. About 44 KB, so three workgroups
// share a compute unit. The K*gamma S0 part of p accumulates in registers pass by pass.
//
// Pivots. For s < t in different 16-token blocks, Gamma_ts = F_t * (whole blocks between) *
// R_s, so each cross-block 16x16 tile of M or P is one matrix-core product over channels with
// the middle factor folded into the s side. Inside a 16-token block the same split at 4-token
// sub-blocks gives Gamma_ts = F4_t * (whole sub-blocks between) * R4_s; the middle factor
// depends only on s's sub-block and the gap (1, 2 or 3 sub-blocks), so each gap is one masked
// product. Pairs inside one sub-block split once more at its halves (three masked products).
// ------------------------------------------------------------------------------------------
template <int D> struct PrepBwdLds {
    static constexpr int DH = 32;  // channels per pass
    static constexpr int LDH = DH + 1;
    static constexpr int LDM = kC + 1;
    static constexpr int TILE = kC * LDH;  // one [C][DH] pass array
    static constexpr int PASS = 5 * TILE + 16 * DH;
    static constexpr int MP = 2 * kC * LDM;
    static constexpr int FLOATS = PASS > MP ? PASS : MP;
    static constexpr size_t BYTES = size_t(FLOATS) * 4;
};

template <typename QT, int D>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(std::is_same_v<QT, bf16_t> ? 2 : 3))) void bwd_prepare_kernel(
    const QT *__restrict__ q, const QT *__restrict__ k, const float *__restrict__ a,
    const float *__restrict__ g, const float *__restrict__ r, const float *__restrict__ states,
    const float *__restrict__ u, QT *__restrict__ kb, QT *__restrict__ kg,
    QT *__restrict__ qg, float *__restrict__ gC, float *__restrict__ Mw,
    QT *__restrict__ Pw, float *__restrict__ pred, int T, int H, int nchunks) {
    using L = PrepBwdLds<D>;
    constexpr int C = kC, LDM = L::LDM, DH = L::DH, LDH = L::LDH;
    constexpr int NJT = D / 64;  // value-column tiles of p per wavefront
    // The bf16 path multiplies on the bf16 matrix cores with split fp32 operands: one K = 32
    // step per pass, lane group kq taking channels 8 kq .. + 7. The fp32 path takes eight K = 4
    // steps, lane group kq taking channel 4 m + kq of step m.
    constexpr bool BF = std::is_same_v<QT, bf16_t>;
    static_assert(DH == 32, "one bf16 step per pass");
    static_assert(kBwdThreads == 8 * DH && kNB == 4, "thread roles assume 256 threads, 4 blocks");
    extern __shared__ float lds[];
    float *sA = lds, *sK = sA + L::TILE, *sQ = sK + L::TILE, *sF = sQ + L::TILE, *sR = sF + L::TILE;
    float *sMid = sR + L::TILE;  // [6][DH] whole blocks strictly between a block pair
    float *sBp = sMid + 6 * DH;  // [4][DH] each whole block
    float *sBef = sBp + 4 * DH;  // [4][DH] the whole blocks before each block
    float *sB4 = sMid;           // [16][DH] each whole sub-block (written after the above are read)

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int bh = b * H + h;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int cc = lane & 15, kq = lane >> 4;
    const size_t HD = size_t(H) * D;
    const int c0 = c * C;
    const int nval = min(C, T - c0);
    const size_t tok0 = (size_t(b) * T + c0) * HD + size_t(h) * D;
    const size_t slot = size_t(bh) * nchunks + c;
    const float *rh = r + size_t(h) * D;
    const float *S0 = states + (size_t(bh) * (nchunks + 1) + c) * D * D;

    // Cross-block tiles of M and P: pair p = (bt, bs), bs < bt, pair index bt (bt - 1) / 2 + bs;
    // tile job j < 12: matrix j / 6 (0: M, 1: P), pair j % 6. Wave w owns jobs w, w + 4, w + 8.
    f32x4_t acc[3] = {zero4(), zero4(), zero4()};
    // Diagonal tiles of block w, M and P, accumulated over the passes.
    f32x4_t dm = zero4(), dp = zero4();
    // p tiles: value columns 16 (w + 4 jj) .. + 15, tokens 16 tt .. + 15.
    f32x4_t pacc[NJT][kNB];
#pragma unroll
    for (int jj = 0; jj < NJT; ++jj)
#pragma unroll
        for (int tt = 0; tt < kNB; ++tt) pacc[jj][tt] = zero4();

    for (int p0 = 0; p0 < D; p0 += DH) {
        // B operands of this pass's (K*gamma) S0 steps: rows p0 .. p0 + DH - 1 of S0.
        float bS[NJT][DH / 4];
#pragma unroll
        for (int jj = 0; jj < NJT; ++jj)
#pragma unroll
            for (int m = 0; m < DH / 4; ++m)
                bS[jj][m] = S0[size_t(p0 + (BF ? 8 * kq + m : 4 * m + kq)) * D + 16 * (wave + 4 * jj) + cc];
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
        {
            // Thread (channel, 16-token block): waves 0-1 the prefix F inside the block, waves
            // 2-3 the suffix R and the whole block's product.
            const int ii = tid % DH, bb = (tid / DH) % kNB;
            float run = 1.f;
            if (tid < kBwdThreads / 2) {
#pragma unroll
                for (int tl = 0; tl < 16; ++tl) {
                    run *= sA[(16 * bb + tl) * LDH + ii];
                    sF[(16 * bb + tl) * LDH + ii] = run;
                }
            } else {
#pragma unroll
                for (int tl = 15; tl >= 0; --tl) {
                    sR[(16 * bb + tl) * LDH + ii] = run;
                    run *= sA[(16 * bb + tl) * LDH + ii];
                }
                sBp[bb * DH + ii] = run;
            }
        }
        __syncthreads();
        {
            // Thread (channel, block, half of the block): gamma and beta of its eight tokens
            // and the scaled operands K*gamma, Q_hat*gamma (channel-major, two 16-byte stores
            // each) and K*beta; the first half also the products of the whole blocks between
            // its block and each earlier one, and gamma_C.
            const int ii = tid % DH, bb = (tid / DH) % kNB, half = tid / (DH * kNB), i = p0 + ii;
            float bp[kNB];
#pragma unroll
            for (int b2 = 0; b2 < kNB; ++b2) bp[b2] = sBp[b2 * DH + ii];
            float before = 1.f, after = 1.f;
#pragma unroll
            for (int b2 = 0; b2 < kNB; ++b2) {
                if (b2 < bb) before *= bp[b2];
                if (b2 > bb) after *= bp[b2];
            }
            if (half == 0) {
                float mid = 1.f;
                for (int bs = bb - 1; bs >= 0; --bs) {
                    sMid[(bb * (bb - 1) / 2 + bs) * DH + ii] = mid;
                    mid *= bp[bs];
                }
                sBef[bb * DH + ii] = before;
                if (bb == kNB - 1) gC[slot * D + i] = before * bp[kNB - 1];
            }
            f32x4_t vkg[2], vqg[2];
#pragma unroll
            for (int tl = 0; tl < 8; ++tl) {
                const int t = 16 * bb + 8 * half + tl;
                const float gm = before * sF[t * LDH + ii];
                const float kt = sK[t * LDH + ii];
                vkg[tl >> 2][tl & 3] = kt * gm;
                vqg[tl >> 2][tl & 3] = sQ[t * LDH + ii] * gm;
                elem<QT>::store(kb, (slot * C + t) * D + i, kt * sR[t * LDH + ii] * after);
            }
            const size_t row = (slot * D + i) * C + 16 * bb + 8 * half;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                store4(kg + row + 4 * h2, vkg[h2]);
                store4(qg + row + 4 * h2, vqg[h2]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int job = wave + 4 * j;
            const int mat = job / 6, pr = job % 6;
            const int bt = pr < 1 ? 1 : (pr < 3 ? 2 : 3);
            const int bs = pr - bt * (bt - 1) / 2;
            const float *sX = mat == 0 ? sK : sQ;
            if constexpr (BF) {
                float av[8], bv[8];
#pragma unroll
                for (int j8 = 0; j8 < 8; ++j8) {
                    const int kk = 8 * kq + j8;
                    av[j8] = sX[(16 * bt + cc) * LDH + kk] * sF[(16 * bt + cc) * LDH + kk];
                    bv[j8] = sK[(16 * bs + cc) * LDH + kk] * sR[(16 * bs + cc) * LDH + kk] * sMid[pr * DH + kk];
                }
                acc[j] = mma3(split8(av), split8(bv), acc[j]);
                continue;
            }
            acc[j] = mm16<DH>(
                [&](int rr, int kk) { return sX[(16 * bt + rr) * LDH + kk] * sF[(16 * bt + rr) * LDH + kk]; },
                [&](int cc2, int kk) {
                    return sK[(16 * bs + cc2) * LDH + kk] * sR[(16 * bs + cc2) * LDH + kk] * sMid[pr * DH + kk];
                },
                acc[j]);
        }
        // (K*gamma) S0 over this pass's channels; the A operand is K*gamma as stored above.
        if constexpr (BF) {
            Split sS[NJT];
#pragma unroll
            for (int jj = 0; jj < NJT; ++jj) sS[jj] = split8(bS[jj]);
#pragma unroll
            for (int tt = 0; tt < kNB; ++tt) {
                const int t = 16 * tt + cc;
                float kv[8];
#pragma unroll
                for (int j8 = 0; j8 < 8; ++j8) {
                    const int kk = 8 * kq + j8;
                    kv[j8] = sK[t * LDH + kk] * (sBef[tt * DH + kk] * sF[t * LDH + kk]);
                }
                const Split ks = split8(kv);
#pragma unroll
                for (int jj = 0; jj < NJT; ++jj) pacc[jj][tt] = mma3(ks, sS[jj], pacc[jj][tt]);
            }
        }
#pragma unroll
        for (int tt = 0; tt < (BF ? 0 : kNB); ++tt) {
#pragma unroll
            for (int m = 0; m < DH / 4; ++m) {
                const int t = 16 * tt + cc, kk = 4 * m + kq;
                const float kgv = sK[t * LDH + kk] * (sBef[tt * DH + kk] * sF[t * LDH + kk]);
#pragma unroll
                for (int jj = 0; jj < NJT; ++jj)
                    pacc[jj][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(kgv, bS[jj][m], pacc[jj][tt], 0, 0, 0);
            }
        }
        __syncthreads();
        {
            // Thread (channel, block, half): F4, R4 and the whole-sub-block products of two of
            // the block's sub-blocks (replacing the block pivots).
            const int ii = tid % DH, bb = (tid / DH) % kNB, half = tid / (DH * kNB);
#pragma unroll
            for (int u2 = 0; u2 < 2; ++u2) {
                const int us = 4 * bb + 2 * half + u2;
                float run = 1.f;
#pragma unroll
                for (int tl = 0; tl < 4; ++tl) {
                    run *= sA[(4 * us + tl) * LDH + ii];
                    sF[(4 * us + tl) * LDH + ii] = run;
                }
                run = 1.f;
#pragma unroll
                for (int tl = 3; tl >= 0; --tl) {
                    sR[(4 * us + tl) * LDH + ii] = run;
                    run *= sA[(4 * us + tl) * LDH + ii];
                }
                sB4[us * DH + ii] = run;
            }
        }
        __syncthreads();
        {
            // Diagonal tiles of block bb = w, M (A rows from K) and P (from Q_hat). For gap g
            // (t's sub-block = s's + g) the s side carries K * R4 times the g - 1 whole
            // sub-blocks after s's. Inside one sub-block the split repeats at its halves: t in
            // the upper half, s in the lower takes (a from the half's start through t) x (a after
            // s to the half's end); t = s + 1 in one half takes a_t; t = s (P only) takes 1.
            const int bb = wave, rr = lane & 15;
            const int us = rr >> 2;  // the B row's (column s = 16 bb + rr) sub-block in the block
            const int sub = rr & 3;  // the A row's (and B column's) place in its sub-block
            const int ta = 16 * bb + rr, u0 = 4 * bb + us;
            // Partial products per sub-block gap (0-2) and half split (3-5).
            f32x4_t ym[5], yp[6];
#pragma unroll
            for (int j = 0; j < 6; ++j) {
                if (j < 5) ym[j] = zero4();
                yp[j] = zero4();
            }
            if constexpr (BF) {
                // One K = 32 step: the same factors for channels 8 kq .. + 7, split.
                float kt[8], qt[8], v1[8], v2[8], v3[8];
#pragma unroll
                for (int j8 = 0; j8 < 8; ++j8) {
                    const int kk = 8 * kq + j8;
                    kt[j8] = sK[ta * LDH + kk];
                    qt[j8] = sQ[ta * LDH + kk];
                }
                {
                    // Gaps 1-3: A = X * F4, B = K * R4 times the whole sub-blocks between.
                    float fa[8];
#pragma unroll
                    for (int j8 = 0; j8 < 8; ++j8) {
                        const int kk = 8 * kq + j8;
                        fa[j8] = sF[ta * LDH + kk];
                        v1[j8] = kt[j8] * sR[ta * LDH + kk];
                        const float m1 = us + 1 < 4 ? sB4[(u0 + 1) * DH + kk] : 0.f;
                        const float m2 = us + 2 < 4 ? sB4[(u0 + 2) * DH + kk] : 0.f;
                        v2[j8] = v1[j8] * m1;
                        v3[j8] = v2[j8] * m2;
                    }
                    const Split b1 = split8(v1), b2 = split8(v2), b3 = split8(v3);
                    float am[8], ap[8];
#pragma unroll
                    for (int j8 = 0; j8 < 8; ++j8) {
                        am[j8] = kt[j8] * fa[j8];
                        ap[j8] = qt[j8] * fa[j8];
                    }
                    const Split sm = split8(am), sp = split8(ap);
                    ym[0] = mma3(sm, b1, ym[0]);
                    ym[1] = mma3(sm, b2, ym[1]);
                    ym[2] = mma3(sm, b3, ym[2]);
                    yp[0] = mma3(sp, b1, yp[0]);
                    yp[1] = mma3(sp, b2, yp[1]);
                    yp[2] = mma3(sp, b3, yp[2]);
                }
                {
                    // Inside one sub-block: the half split, adjacent tokens, the diagonal.
                    float af[8], bf[8], at[8];
#pragma unroll
                    for (int j8 = 0; j8 < 8; ++j8) {
                        const int kk = 8 * kq + j8;
                        const float a0 = sA[ta * LDH + kk];
                        const float aprev = sA[(sub > 0 ? ta - 1 : ta) * LDH + kk];
                        const float anext = sA[(sub < 3 ? ta + 1 : ta) * LDH + kk];
                        af[j8] = sub == 2 ? a0 : (sub == 3 ? aprev * a0 : 0.f);
                        bf[j8] = kt[j8] * (sub == 0 ? anext : (sub == 1 ? 1.f : 0.f));
                        at[j8] = a0;
                    }
                    const Split bh = split8(bf), sk = split8(kt);
#pragma unroll
                    for (int j8 = 0; j8 < 8; ++j8) {
                        v1[j8] = kt[j8] * af[j8];
                        v2[j8] = qt[j8] * af[j8];
                    }
                    ym[3] = mma3(split8(v1), bh, ym[3]);
                    yp[3] = mma3(split8(v2), bh, yp[3]);
#pragma unroll
                    for (int j8 = 0; j8 < 8; ++j8) {
                        v1[j8] = kt[j8] * at[j8];
                        v2[j8] = qt[j8] * at[j8];
                    }
                    ym[4] = mma3(split8(v1), sk, ym[4]);
                    yp[4] = mma3(split8(v2), sk, yp[4]);
                    yp[5] = mma3(split8(qt), sk, yp[5]);
                }
            }
#pragma unroll 2
            for (int m = 0; m < (BF ? 0 : DH / 4); ++m) {
                const int kk = 4 * m + kq;
                const float kt = sK[ta * LDH + kk], qt = sQ[ta * LDH + kk];
                const float at = sA[ta * LDH + kk];
                const float aprev = sA[(sub > 0 ? ta - 1 : ta) * LDH + kk];
                const float anext = sA[(sub < 3 ? ta + 1 : ta) * LDH + kk];
                const float f4 = sF[ta * LDH + kk];
                const float b1 = kt * sR[ta * LDH + kk];
                const float m1 = us + 1 < 4 ? sB4[(u0 + 1) * DH + kk] : 0.f;
                const float m2 = us + 2 < 4 ? sB4[(u0 + 2) * DH + kk] : 0.f;
                const float b2 = b1 * m1, b3 = b2 * m2;
                const float f2 = sub == 2 ? at : (sub == 3 ? aprev * at : 0.f);
                const float r2 = sub == 0 ? anext : (sub == 1 ? 1.f : 0.f);
                const float avm = kt * f4, avp = qt * f4, bh2 = kt * r2;
                ym[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(avm, b1, ym[0], 0, 0, 0);
                ym[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(avm, b2, ym[1], 0, 0, 0);
                ym[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(avm, b3, ym[2], 0, 0, 0);
                ym[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(kt * f2, bh2, ym[3], 0, 0, 0);
                ym[4] = __builtin_amdgcn_mfma_f32_16x16x4f32(kt * at, kt, ym[4], 0, 0, 0);
                yp[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(avp, b1, yp[0], 0, 0, 0);
                yp[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(avp, b2, yp[1], 0, 0, 0);
                yp[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(avp, b3, yp[2], 0, 0, 0);
                yp[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(qt * f2, bh2, yp[3], 0, 0, 0);
                yp[4] = __builtin_amdgcn_mfma_f32_16x16x4f32(qt * at, kt, yp[4], 0, 0, 0);
                yp[5] = __builtin_amdgcn_mfma_f32_16x16x4f32(qt, kt, yp[5], 0, 0, 0);
            }
            // Output lane l: rows 4 (l / 16) + i (sub-block l / 16), column l % 16.
            const int ut = kq, usc = cc >> 2;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tr = 4 * ut + i;  // row within the block
                const int gap = ut - usc;
                float vm = 0.f, vp = 0.f;
                if (gap == 1) vm = ym[0][i], vp = yp[0][i];
                if (gap == 2) vm = ym[1][i], vp = yp[1][i];
                if (gap == 3) vm = ym[2][i], vp = yp[2][i];
                if (gap == 0) {
                    if ((tr & 3) >= 2 && (cc & 3) < 2) vm = ym[3][i], vp = yp[3][i];
                    else if ((tr & 1) == 1 && cc == tr - 1) vm = ym[4][i], vp = yp[4][i];
                    else if (cc == tr) vp = yp[5][i];
                }
                dm[i] += vm;
                dp[i] += vp;
            }
        }
    }
    __syncthreads();
    // M and P into LDS over the pass arrays. Only the strictly lower part of M and the lower
    // part of P (with its diagonal) are written; every read below masks the rest.
    float *sM = lds, *sP = lds + C * LDM;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int job = wave + 4 * j;
        const int mat = job / 6, pr = job % 6;
        const int bt = pr < 1 ? 1 : (pr < 3 ? 2 : 3);
        const int bs = pr - bt * (bt - 1) / 2;
        float *dst = mat == 0 ? sM : sP;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(16 * bt + 4 * kq + i) * LDM + 16 * bs + cc] = acc[j][i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tr = 4 * kq + i;  // row within the diagonal block
        if (cc <= tr) {
            sM[(16 * wave + tr) * LDM + 16 * wave + cc] = dm[i];
            sP[(16 * wave + tr) * LDM + 16 * wave + cc] = dp[i];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < C * C; idx += kBwdThreads) {
        const int t = idx / C, s = idx % C;
        Mw[slot * C * C + idx] = s < t ? sM[t * LDM + s] : 0.f;
        // P transposed: row t holds P[., t].
        elem<QT>::store(Pw, slot * C * C + idx, t <= s ? sP[s * LDM + t] : 0.f);
    }
    // p = (K*gamma) S0 + M U: the M U part, then the tokens of the chunk are stored.
    const float *Ub = u + (size_t(b) * T + c0) * HD + size_t(h) * D;
#pragma unroll
    for (int jj = 0; jj < NJT; ++jj) {
        const int jt = wave + 4 * jj;
        // B operands: token s of step m is 4 m + kq (fp32 path) or, for the two K = 32 steps
        // st of the bf16 path, 32 st + 8 kq + j.
        float bU[C / 4];
#pragma unroll
        for (int m = 0; m < C / 4; ++m) {
            const int sb = BF ? 32 * (m / 8) + 8 * kq + m % 8 : 4 * m + kq;
            bU[m] = sb < nval ? Ub[size_t(sb) * HD + 16 * jt + cc] : 0.f;
        }
        if constexpr (BF) {
            Split sU[2];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                float x8[8];
#pragma unroll
                for (int j8 = 0; j8 < 8; ++j8) x8[j8] = bU[8 * st + j8];
                sU[st] = split8(x8);
            }
#pragma unroll
            for (int tt = 0; tt < kNB; ++tt) {
                const int t = 16 * tt + cc;
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    float mv[8];
#pragma unroll
                    for (int j8 = 0; j8 < 8; ++j8) {
                        const int s2 = 32 * st + 8 * kq + j8;
                        mv[j8] = s2 < t ? sM[t * LDM + s2] : 0.f;
                    }
                    pacc[jj][tt] = mma3(split8(mv), sU[st], pacc[jj][tt]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t2 = 16 * tt + 4 * kq + i;
                    if (t2 < nval) pred[tok0 + size_t(t2) * HD + 16 * jt + cc] = pacc[jj][tt][i];
                }
            }
            continue;
        }
#pragma unroll
        for (int tt = 0; tt < kNB; ++tt) {
            const int t = 16 * tt + cc;
#pragma unroll
            for (int m = 0; m < C / 4; ++m) {
                const int s = 4 * m + kq;
                const float mv = s < t ? sM[t * LDM + s] : 0.f;
                pacc[jj][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(mv, bU[m], pacc[jj][tt], 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t2 = 16 * tt + 4 * kq + i;
                if (t2 < nval) pred[tok0 + size_t(t2) * HD + 16 * jt + cc] = pacc[jj][tt][i];
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
    const float *__restrict__ w, const QT *__restrict__ kb, const QT *__restrict__ kg,
    const QT *__restrict__ qg, const float *__restrict__ gC, const float *__restrict__ Mw,
    const QT *__restrict__ Pw, const float *__restrict__ pred, const float *__restrict__ dsT,
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
    // K*gamma (channel-major) rows of this wave's channel tiles. fp32 operands take 16-byte
    // pieces of four fp32 steps (k = 16 mo + 4 kq + mi); bf16 operands one bf16 step's
    // fragment (k = 32 s + 8 kq + j).
    using M16 = Mma<bf16_t>;
    constexpr bool BF = std::is_same_v<QT, bf16_t>;
    constexpr int KD = BF ? D / 32 : D / 16, KC = BF ? C / 32 : C / 16;
    using AF = std::conditional_t<BF, M16::frag, f32x4_t>;
    AF aKB[KD], aP[KC], aQG[NIT][KC], aKG[NIT][KC];
    auto ldA = [&](const QT *p, size_t o) {
        if constexpr (BF) return M16::load(p + o);
        else return ld4(p, o);
    };
    constexpr int KW = BF ? 32 : 16, KL = BF ? 8 : 4;  // k of step m, lane group kq: KW m + KL kq
    auto load_rhsA = [&](int c) {
        const size_t sl = slot_of(c);
#pragma unroll
        for (int m = 0; m < KD; ++m) aKB[m] = ldA(kb, (sl * C + 16 * wave + r) * D + KW * m + KL * kq);
#pragma unroll
        for (int m = 0; m < KC; ++m) aP[m] = ldA(Pw, (sl * C + 16 * wave + r) * C + KW * m + KL * kq);
    };
    auto load_lamA = [&](int c) {
        const size_t sl = slot_of(c);
#pragma unroll
        for (int n = 0; n < NIT; ++n)
#pragma unroll
            for (int m = 0; m < KC; ++m) {
                const size_t o = (sl * D + 16 * (wave + 4 * n) + r) * C + KW * m + KL * kq;
                aQG[n][m] = ldA(qg, o);
                aKG[n][m] = ldA(kg, o);
            }
    };
    // B fragment of a bf16 step: rows 32 m + 8 kq .. + 7 of an fp32 LDS array, column r;
    // ldsB2 also gives the rounding remainder as a second fragment (hi + lo carries the fp32
    // value to about 2^-17), for the operands that carry the adjoint along the sequence.
    auto ldsB = [&](const float *X, int m, int ld) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = X[(32 * m + 8 * kq + j) * ld + r];
        return M16::pack(x);
    };
    auto ldsB2 = [&](const float *X, int m, int ld, M16::frag &lo) {
        float x[8], rem[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = X[(32 * m + 8 * kq + j) * ld + r];
        const M16::frag hi = M16::pack(x);
        const u16x8_t hb = __builtin_bit_cast(u16x8_t, hi);
#pragma unroll
        for (int j = 0; j < 8; ++j) rem[j] = x[j] - bf16_to_f32(hb[j]);
        lo = M16::pack(rem);
        return hi;
    };
    // Staged through LDS: M, the per-token tiles (thread: token tid / 4, columns 4 (tid % 4)
    // .. + 3) and gamma_C. Every load is unconditional (rows past the sequence read the chunk's
    // first row and are zeroed when stored), so the next chunk's loads stay in flight.
    struct Stage {
        f32x4_t m[C * C / 4 / kBwdThreads];
        typename Raw4<QT>::type dO, v;
        f32x4_t e, w, pr;
        float gc;
    } st;
    auto load_stage = [&](int c) {
        const size_t sl = slot_of(c);
        const f32x4_t *M4 = reinterpret_cast<const f32x4_t *>(Mw + sl * C * C);
#pragma unroll
        for (int j = 0; j < C * C / 4 / kBwdThreads; ++j) st.m[j] = M4[tid + kBwdThreads * j];
        const int t = tid >> 2, c4 = 4 * (tid & 3);
        const int tc = t < T - c * C ? t : 0;
        const size_t o = tok_base(c) + size_t(tc) * HD + c4;
        st.dO = raw4(dout, o);
        st.e = ld4(e, o);
        st.w = ld4(w, o);
        st.v = raw4(v, o);
        st.pr = ld4(pred, o);
        st.gc = gC[sl * D + (tid < D ? tid : 0)];
    };
    auto store_stage = [&](int c) {
        const bool ok = (tid >> 2) < T - c * C;
#pragma unroll
        for (int j = 0; j < C * C / 4 / kBwdThreads; ++j) {
            const int e0 = 4 * (tid + kBwdThreads * j), t = e0 / C, s = e0 % C;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) sM[t * LDM + s + q4] = st.m[j][q4];
        }
        const int t = tid >> 2, c4 = 4 * (tid & 3);
        const f32x4_t dO4 = ok ? cvt4(st.dO) : zero4(), v4 = ok ? cvt4(st.v) : zero4();
        *reinterpret_cast<f32x4_t *>(&sdO[t * LDB + c4]) = dO4;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            sE[t * LDT + c4 + q4] = ok ? st.e[q4] : 0.f;
            sW[t * LDT + c4 + q4] = ok ? st.w[q4] : 0.f;
            sV[t * LDT + c4 + q4] = v4[q4];
            sPr[t * LDT + c4 + q4] = ok ? st.pr[q4] : 0.f;
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
        store_stage(c);
        for (int idx = tid; idx < D * VT; idx += kBwdThreads) {
            const int i = idx / VT, j = idx % VT;
            lamC[(slot * D + i) * D + j0 + j] = sLam[i * LDB + j];
        }
        __syncthreads();
        load_stage(c > 0 ? c - 1 : 0);
        // Right-hand side of this wave's 16 tokens.
        {
            f32x4_t y = zero4();
            if constexpr (BF) {
#pragma unroll
                for (int m = 0; m < KD; ++m) {
                    M16::frag lo;
                    const M16::frag hi = ldsB2(sLam, m, LDB, lo);
                    y = M16::mma(aKB[m], hi, y);
                    y = M16::mma(aKB[m], lo, y);
                }
#pragma unroll
                for (int m = 0; m < KC; ++m) y = M16::mma(aP[m], ldsB(sdO, m, LDB), y);
            } else {
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
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) sRhs[(16 * wave + 4 * kq + i) * LDT + r] = y[i];
        }
        load_rhsA(c > 0 ? c - 1 : 0);
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
            if constexpr (BF) {
#pragma unroll
                for (int m = 0; m < KC; ++m) {
                    M16::frag lo;
                    const M16::frag hi = ldsB2(sdP, m, LDB, lo);
                    y = M16::mma(aQG[n][m], ldsB(sdO, m, LDB), y);
                    y = M16::mma(aKG[n][m], hi, y);
                    y = M16::mma(aKG[n][m], lo, y);
                }
            } else {
#pragma unroll
                for (int mo = 0; mo < C / 16; ++mo)
#pragma unroll
                    for (int mi = 0; mi < 4; ++mi) {
                        const int tt = 16 * mo + 4 * kq + mi;
                        y = __builtin_amdgcn_mfma_f32_16x16x4f32(aQG[n][mo][mi], sdO[tt * LDB + r], y, 0, 0, 0);
                        y = __builtin_amdgcn_mfma_f32_16x16x4f32(aKG[n][mo][mi], sdP[tt * LDB + r], y, 0, 0, 0);
                    }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) sLam[(i0 + 4 * kq + i) * LDB + r] = y[i];
        }
        load_lamA(c > 0 ? c - 1 : 0);
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
// Products. One workgroup per (b, h, chunk), four wavefronts, no LDS. Wave w keeps rows
// 16 w .. 16 w + 15 of U, then of dO and dP = -e * dU, in registers as matrix-core A operands
// and streams 16-row tiles of lambda_C, U and S0 past them (the next tile loads while the
// current one is multiplied):
//   Y1 = dO S0^T, Y2 = dP S0^T, Y3 = U lambda_C^T    [C x D], stored [D/16][C][16] per chunk
//   OU = dO U^T (s <= t), PU = dP U^T (s < t)         [C x C] per chunk, upper parts zero.
// Y1 and Y2 are the state terms of dq_hat and of the read part of dk, Y3 that of the write
// part of dk; OU and PU weight the decayed pair sums. Also rowsum(S_C * lambda_C) per channel,
// the log-decay gradient's chunk-end term, [D] per chunk.
// ------------------------------------------------------------------------------------------
// rowsum(S_C * lambda_C) of rows 16 (w + 4 jj) + rr, the log-decay gradient's chunk-end term:
// lane group kq sums its 32 columns (k = 32 st + 8 kq + j) in order, and the four groups are
// added with two lane exchanges, in a fixed order.
template <int D>
__device__ __forceinline__ void rowsum_sc_lam(const float *__restrict__ SC, const float *__restrict__ lam,
                                              float *__restrict__ rs, int wave, int rr, int kq) {
#pragma unroll
    for (int jj = 0; jj < D / 64; ++jj) {
        const size_t row = size_t(16 * (wave + 4 * jj) + rr);
        f32x4_t xs[D / 16], xl[D / 16];
#pragma unroll
        for (int st = 0; st < D / 32; ++st)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                xs[2 * st + h2] = ld4(SC, row * D + 32 * st + 8 * kq + 4 * h2);
                xl[2 * st + h2] = ld4(lam, row * D + 32 * st + 8 * kq + 4 * h2);
            }
        float acc = 0.f;
#pragma unroll
        for (int x = 0; x < D / 16; ++x)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) acc = fmaf(xs[x][q4], xl[x][q4], acc);
        acc += __shfl_xor(acc, 16, 64);
        acc += __shfl_xor(acc, 32, 64);
        if (kq == 0) rs[row] = acc;
    }
}

// The products kernel's body on the bf16 path: the same three phases and outputs, contraction
// step s of lane group kq taking k = 32 s + 8 kq .. + 7 (two 16-byte loads per fp32 operand).
template <int D>
__device__ __forceinline__ void products_split(const bf16_t *__restrict__ dout, const float *__restrict__ e,
                                               const float *__restrict__ U, const float *__restrict__ dU,
                                               const float *__restrict__ S0, const float *__restrict__ lam,
                                               float *__restrict__ Y1, float *__restrict__ Y2,
                                               float *__restrict__ Y3, float *__restrict__ OU,
                                               float *__restrict__ PU, size_t tok0, size_t HD, size_t slot,
                                               int nval, int wave, int rr, int kq) {
    using M16 = Mma<bf16_t>;
    constexpr int C = kC, NT = D / 16, NS = D / 32;
    const int ta = 16 * wave + rr;  // this lane's A row
    const bool ok = ta < nval;
    auto tokrow = [&](int t) { return tok0 + size_t(t < nval ? t : 0) * HD; };
    using Raw = f32x4_t[NS][2];
    auto ld8 = [&](const float *X, size_t row0, Raw &x) {
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            x[st][0] = ld4(X, row0 + 32 * st + 8 * kq);
            x[st][1] = ld4(X, row0 + 32 * st + 8 * kq + 4);
        }
    };
    auto store_y = [&](float *Y, int it, f32x4_t y) {
        float *dst = Y + ((slot * NT + it) * C + 16 * wave + 4 * kq) * 16 + rr;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[16 * i] = y[i];
    };
    // The B operands stream through LDS, one 16-row tile at a time, double-buffered, loaded
    // once per workgroup (every wavefront multiplies every tile): the NT tiles of lambda_C
    // (phase 1), the kNB row blocks of U (phase 2), the NT tiles of S0 (phase 3). Thread tid
    // moves 16-byte pieces tid, tid + 256, ... of a tile.
    constexpr int LDT = D + 4, N4 = 16 * D / 4 / kBwdThreads, NQ = 2 * NT + kNB;
    __shared__ __align__(16) float sh_b[2][16][LDT];
    const int tid = 64 * wave + 16 * kq + rr;
    auto tile_src = [&](int q, int r) -> const float * {
        if (q < NT) return lam + size_t(16 * q + r) * D;
        if (q < NT + kNB) return U + tokrow(16 * (q - NT) + r);
        return S0 + size_t(16 * (q - NT - kNB) + r) * D;
    };
    f32x4_t nx[N4];
    auto load_tile = [&](int q) {
#pragma unroll
        for (int j = 0; j < N4; ++j) {
            const int i = tid + kBwdThreads * j, r = i / (D / 4), c4 = i % (D / 4);
            nx[j] = ld4(tile_src(q, r), 4 * c4);
        }
    };
    auto put_tile = [&](int buf) {
#pragma unroll
        for (int j = 0; j < N4; ++j) {
            const int i = tid + kBwdThreads * j, r = i / (D / 4), c4 = i % (D / 4);
            *reinterpret_cast<f32x4_t *>(&sh_b[buf][r][4 * c4]) = nx[j];
        }
    };
    // B fragment of step st: row rr of the tile, k = 32 st + 8 kq .. + 7, split.
    auto tileB = [&](int buf, int st) {
        const f32x4_t *p = reinterpret_cast<const f32x4_t *>(&sh_b[buf][rr][32 * st + 8 * kq]);
        return split8(p[0], p[1]);
    };
    load_tile(0);
    Split xu[NS];
    {
        Raw ru;
        ld8(U, tokrow(ta), ru);
#pragma unroll
        for (int st = 0; st < NS; ++st) xu[st] = split8(ru[st][0], ru[st][1]);
    }
    put_tile(0);
    // The wave's rows of dO (exact in bf16) and dP = -e * dU (split), zero past the sequence.
    M16::frag xo[NS];
    Split xp[NS];
    {
        Raw re, rd;
        ld8(e, tokrow(ta), re);
        ld8(dU, tokrow(ta), rd);
#pragma unroll
        for (int st = 0; st < NS; ++st) xo[st] = M16::load(dout + tokrow(ta) + 32 * st + 8 * kq);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            xp[st] = split8(-re[st][0] * rd[st][0], -re[st][1] * rd[st][1]);
            if (!ok) {
                xo[st] = M16::zero();
                xp[st].hi = xp[st].lo = M16::zero();
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int buf = q & 1;
        if (q + 1 < NQ) load_tile(q + 1);
        if (q < NT) {
            // 1. Y3 = U lambda_C^T.
            f32x4_t y3 = zero4();
#pragma unroll
            for (int st = 0; st < NS; ++st) y3 = mma3(xu[st], tileB(buf, st), y3);
            store_y(Y3, q, y3);
        } else if (q < NT + kNB) {
            // 2. O U^T and dP U^T against column block bs <= w; blocks after w are zero.
            const int bs = q - NT;
            f32x4_t yo = zero4(), yp = zero4();
            if (bs <= wave) {
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    const Split b = tileB(buf, st);
                    yo = mma2(xo[st], b, yo);
                    yp = mma3(xp[st], b, yp);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * wave + 4 * kq + i, sc = 16 * bs + rr;
                OU[(slot * C + t) * C + sc] = sc <= t ? yo[i] : 0.f;
                PU[(slot * C + t) * C + sc] = sc < t ? yp[i] : 0.f;
            }
        } else {
            // 3. Y1 = dO S0^T and Y2 = dP S0^T.
            const int it = q - NT - kNB;
            f32x4_t y1 = zero4(), y2 = zero4();
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const Split b = tileB(buf, st);
                y1 = mma2(xo[st], b, y1);
                y2 = mma3(xp[st], b, y2);
            }
            store_y(Y1, it, y1);
            store_y(Y2, it, y2);
        }
        if (q + 1 < NQ) put_tile(buf ^ 1);
        __syncthreads();
    }
}

template <typename QT, int D>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(3))) void bwd_products_kernel(
    const QT *__restrict__ dout, const float *__restrict__ e, const float *__restrict__ U,
    const float *__restrict__ dU, const float *__restrict__ states, const float *__restrict__ lamC,
    float *__restrict__ Y1, float *__restrict__ Y2, float *__restrict__ Y3, float *__restrict__ OU,
    float *__restrict__ PU, float *__restrict__ rs, int T, int H, int nchunks) {
    constexpr int C = kC, NT = D / 16;
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int bh = b * H + h;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rr = lane & 15, kq = lane >> 4;
    const size_t HD = size_t(H) * D;
    const int c0 = c * C;
    const int nval = min(C, T - c0);
    const size_t tok0 = (size_t(b) * T + c0) * HD + size_t(h) * D;
    const size_t slot = size_t(bh) * nchunks + c;
    const float *S0 = states + (size_t(bh) * (nchunks + 1) + c) * D * D;
    const float *lam = lamC + slot * D * D;
    // The chunk-end state is the next 64-token block's start state.
    rowsum_sc_lam<D>(S0 + size_t(D) * D, lam, rs + slot * D, wave, lane & 15, lane >> 4);
    if constexpr (std::is_same_v<QT, bf16_t>) {
        products_split<D>(dout, e, U, dU, S0, lam, Y1, Y2, Y3, OU, PU, tok0, HD, slot, nval, wave, lane & 15,
                          lane >> 4);
        return;
    }

    // Contraction step (mo, mi) of lane group kq takes k = 16 mo + 4 kq + mi: a lane's four
    // values of one mo are one 16-byte load. Token rows past the sequence load the chunk's first
    // row (every load unconditional, so none waits on another). Only the dO and dP rows are
    // zeroed there: that makes every O U^T, dP U^T, Y1 and Y2 entry of such a row zero, and the
    // U rows past the sequence meet only rows whose results are not used.
    auto load_tok = [&](const float *X, int t, f32x4_t (&x)[NT]) {
#pragma unroll
        for (int mo = 0; mo < NT; ++mo) x[mo] = ld4(X, tok0 + size_t(t < nval ? t : 0) * HD + 16 * mo + 4 * kq);
    };
    auto zero_past = [&](int t, f32x4_t (&x)[NT]) {
#pragma unroll
        for (int mo = 0; mo < NT; ++mo) x[mo] = t < nval ? x[mo] : zero4();
    };
    auto load_rows = [&](const float *S, int row, f32x4_t (&x)[NT]) {
#pragma unroll
        for (int mo = 0; mo < NT; ++mo) x[mo] = ld4(S, size_t(row) * D + 16 * mo + 4 * kq);
    };
    // Output lane l: rows 4 (l / 16) + i of the wave's block, column l % 16 of the tile.
    auto store_y = [&](float *Y, int it, f32x4_t y) {
        float *dst = Y + ((slot * NT + it) * C + 16 * wave + 4 * kq) * 16 + rr;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[16 * i] = y[i];
    };
    const int ta = 16 * wave + rr;  // this lane's A row
    // 1. Y3 = U lambda_C^T, the tiles of lambda_C streaming past the wave's U rows.
    {
        f32x4_t xu[NT], bL[2][NT];
        load_tok(U, ta, xu);
        load_rows(lam, rr, bL[0]);
#pragma unroll
        for (int it = 0; it < NT; ++it) {
            const int cur = it & 1;
            if (it + 1 < NT) load_rows(lam, 16 * (it + 1) + rr, bL[cur ^ 1]);
            f32x4_t y3 = zero4();
#pragma unroll
            for (int mo = 0; mo < NT; ++mo)
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
                    y3 = __builtin_amdgcn_mfma_f32_16x16x4f32(xu[mo][mi], bL[cur][mo][mi], y3, 0, 0, 0);
            store_y(Y3, it, y3);
        }
    }
    // 2. O U^T and dP U^T: the wave's row block against each column block bs <= w (U rows of
    // block bs, the next loading while the current is multiplied); blocks after w are zero.
    f32x4_t xo[NT], xp[NT];
    {
        f32x4_t bu[2][NT];
        load_tok(U, rr, bu[0]);
#pragma unroll
        for (int mo = 0; mo < NT; ++mo) {
            const size_t o = tok0 + size_t(ta < nval ? ta : 0) * HD + 16 * mo + 4 * kq;
            xo[mo] = ld4(dout, o);
            xp[mo] = -ld4(e, o) * ld4(dU, o);
        }
        zero_past(ta, xo);
        zero_past(ta, xp);
#pragma unroll
        for (int bs = 0; bs < kNB; ++bs) {
            const int cur = bs & 1;
            f32x4_t yo = zero4(), yp = zero4();
            if (bs <= wave) {
                if (bs + 1 <= wave) load_tok(U, 16 * (bs + 1) + rr, bu[cur ^ 1]);
#pragma unroll
                for (int mo = 0; mo < NT; ++mo)
#pragma unroll
                    for (int mi = 0; mi < 4; ++mi) {
                        yo = __builtin_amdgcn_mfma_f32_16x16x4f32(xo[mo][mi], bu[cur][mo][mi], yo, 0, 0, 0);
                        yp = __builtin_amdgcn_mfma_f32_16x16x4f32(xp[mo][mi], bu[cur][mo][mi], yp, 0, 0, 0);
                    }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * wave + 4 * kq + i, s = 16 * bs + rr;
                OU[(slot * C + t) * C + s] = s <= t ? yo[i] : 0.f;
                PU[(slot * C + t) * C + s] = s < t ? yp[i] : 0.f;
            }
        }
    }
    // 3. Y1 = dO S0^T and Y2 = dP S0^T, the tiles of S0 streaming past the wave's rows.
    {
        f32x4_t bS[2][NT];
        load_rows(S0, rr, bS[0]);
#pragma unroll
        for (int it = 0; it < NT; ++it) {
            const int cur = it & 1;
            if (it + 1 < NT) load_rows(S0, 16 * (it + 1) + rr, bS[cur ^ 1]);
            f32x4_t y1 = zero4(), y2 = zero4();
#pragma unroll
            for (int mo = 0; mo < NT; ++mo)
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    y1 = __builtin_amdgcn_mfma_f32_16x16x4f32(xo[mo][mi], bS[cur][mo][mi], y1, 0, 0, 0);
                    y2 = __builtin_amdgcn_mfma_f32_16x16x4f32(xp[mo][mi], bS[cur][mo][mi], y2, 0, 0, 0);
                }
            store_y(Y1, it, y1);
            store_y(Y2, it, y2);
        }
    }
}

// ------------------------------------------------------------------------------------------
// Chunk-parallel gradients. One workgroup per (b, h, chunk, group of 64 key channels); the
// groups of one chunk take consecutive dispatch slots of one XCD, so they share its L2.
//   1. O U^T and dP U^T into LDS, with rowsum(S_C * lambda_C) of the group's channels (both from
//      the products kernel).
//   2. Per 16-channel pass, after the pivots: wave w takes the rows t of block w (dq_hat and the
//      read part of dk) and the rows s of block w (the write part of dk), each its state term
//      from the products kernel plus the decayed pair sums on the matrix cores. dq and dg are
//      stored; the two parts of dk and the log-decay terms meet in LDS.
//   3. Per pass: dk, and a * dL/da as a reverse cumulative sum over the chunk per channel.
// The next pass's operands load while the current pass runs.
// LDS: O U^T and dP U^T [C][C + 1]; per pass a, k, q_hat, F, R (16-token blocks), F4, R4
// (4-token sub-blocks) [C][16] and the per-channel products of whole blocks and sub-blocks;
// the read and write parts of dk and the log-decay terms [C][17]. About 78 KB, so two
// workgroups share a compute unit.
// ------------------------------------------------------------------------------------------
template <int D> struct GradLds {
    static constexpr int DG = 64;     // key channels per workgroup
    static constexpr int G = D / DG;  // workgroups per chunk
    static constexpr int LDM = kC + 1, DH = 16, LDH = DH, LDO = DH + 1;
    static constexpr int OUPU = 2 * kC * LDM;
    static constexpr int PASS = 7 * kC * LDH + (6 + 16 + 4 + 4) * DH;
    static constexpr int OUTS = 3 * kC * LDO;
    static constexpr int SMALL = 2 * DG + kNB * 4 * DH + kNB * DH + 16 * DH;
    static constexpr int FLOATS = OUPU + PASS + OUTS + SMALL;
    static constexpr size_t BYTES = size_t(FLOATS) * 4;
};

template <typename QT, int D>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2))) void bwd_grads_kernel(
    const QT *__restrict__ q, const QT *__restrict__ k, const float *__restrict__ a,
    const float *__restrict__ g, const float *__restrict__ r, const float *__restrict__ states,
    const float *__restrict__ lamC, const float *__restrict__ Y1, const float *__restrict__ Y2,
    const float *__restrict__ Y3, const float *__restrict__ OU, const float *__restrict__ PU,
    const float *__restrict__ rs, float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dg,
    float *__restrict__ dla, float *__restrict__ drp, int T, int H, int nchunks, int nwork) {
    using L = GradLds<D>;
    constexpr int C = kC, LDM = L::LDM, LDH = L::LDH, DH = L::DH, LDO = L::LDO, G = L::G, DG = L::DG;
    constexpr int NT = D / 16;
    static_assert(kBwdThreads == 16 * DH && kNB == 4, "thread roles assume 256 threads, 4 blocks");
    extern __shared__ float lds[];
    float *sOU = lds, *sPU = lds + C * LDM;
    float *pass = lds + L::OUPU;
    float *sA = pass, *sK = sA + C * LDH, *sQ = sK + C * LDH, *sF = sQ + C * LDH, *sR = sF + C * LDH,
          *sF4 = sR + C * LDH, *sR4 = sF4 + C * LDH, *sMid = sR4 + C * LDH, *sB4 = sMid + 6 * DH,
          *sGb = sB4 + 16 * DH, *sBa = sGb + 4 * DH;
    float *sDkr = pass + L::PASS, *sDkw = sDkr + C * LDO, *sLa = sDkw + C * LDO;
    float *sRS = sLa + C * LDO;        // rowsum(S_C * lambda_C) per channel of the group
    float *sDr = sRS + DG;             // sum over tokens of g * q * dq_hat per channel
    float *sDrP = sDr + DG;            // dr partials of one pass: [block][lane group][channel]
    float *sBp = sDrP + kNB * 4 * DH;  // whole-block decay products per channel
    float *sTot = sBp + kNB * DH;      // per-part sums of the reverse cumulative sum

    // Workgroups are dealt to the eight XCDs in turn: slot pos of XCD x is workgroup 8 pos + x.
    const int wid = blockIdx.x, xcd = wid & 7, pos = wid >> 3;
    const int work = 8 * (pos / G) + xcd, grp = pos % G;
    if (work >= nwork) return;
    const int c = work % nchunks, bh = work / nchunks;
    const int h = bh % H, b = bh / H;
    const int gc0 = grp * DG;  // the group's first channel
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rr = lane & 15, kq = lane >> 4;
    const size_t HD = size_t(H) * D;
    const int c0 = c * C;
    const int nval = min(C, T - c0);
    const size_t tok0 = (size_t(b) * T + c0) * HD + size_t(h) * D;
    const size_t slot = size_t(bh) * nchunks + c;
    const float *rh = r + size_t(h) * D;

    // A pass's operands from memory: the [C][16] slab of a, k, g, q, r (thread: token tid / 4,
    // channels 4 (tid % 4) .. + 3) and, for this lane's four rows 16 w + 4 kq + e4 and channel
    // rr, the state terms and g, q. Every load is unconditional (rows past the sequence read the
    // chunk's first row and are masked where used) and k, q stay in their stored precision until
    // used, so the next pass's loads stay in flight while the current pass runs.
    struct PassIn {
        f32x4_t a, g, r;
        typename Raw4<QT>::type k, q;
        float y1[4], y2[4], y3[4], gg[4];
        QT gq[4];
    };
    auto load_pass = [&](int p0, PassIn &x) {
        const int t = tid >> 2, ii = 4 * (tid & 3);
        const size_t o = tok0 + size_t(t < nval ? t : 0) * HD + p0 + ii;
        x.a = ld4(a, o);
        x.k = raw4(k, o);
        x.g = ld4(g, o);
        x.q = raw4(q, o);
        x.r = ld4(rh, p0 + ii);
        const size_t yo = ((slot * NT + p0 / 16) * C + 16 * wave + 4 * kq) * 16 + rr;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            x.y1[e4] = Y1[yo + 16 * e4];
            x.y2[e4] = Y2[yo + 16 * e4];
            x.y3[e4] = Y3[yo + 16 * e4];
            const int t2 = 16 * wave + 4 * kq + e4;
            const size_t o2 = tok0 + size_t(t2 < nval ? t2 : 0) * HD + p0 + rr;
            x.gg[e4] = g[o2];
            x.gq[e4] = q[o2];
        }
    };
    PassIn cur;
    load_pass(gc0, cur);
    {
        // O U^T and dP U^T into LDS: thread tid takes 16-byte pieces tid, tid + 256, ...
        constexpr int N4 = C * C / 4 / kBwdThreads;
        f32x4_t vo[N4], vp[N4];
        const f32x4_t *OU4 = reinterpret_cast<const f32x4_t *>(OU + slot * C * C);
        const f32x4_t *PU4 = reinterpret_cast<const f32x4_t *>(PU + slot * C * C);
#pragma unroll
        for (int j = 0; j < N4; ++j) {
            vo[j] = OU4[tid + kBwdThreads * j];
            vp[j] = PU4[tid + kBwdThreads * j];
        }
#pragma unroll
        for (int j = 0; j < N4; ++j) {
            const int e0 = 4 * (tid + kBwdThreads * j), t = e0 / C, s = e0 % C;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                sOU[t * LDM + s + q4] = vo[j][q4];
                sPU[t * LDM + s + q4] = vp[j][q4];
            }
        }
        if (tid < DG) sRS[tid] = rs[slot * D + gc0 + tid];
    }
    for (int i = tid; i < DG; i += kBwdThreads) sDr[i] = 0.f;
    // Decayed sums over token pairs, per 16-channel pass, on the matrix cores. With the pivots
    // of the prepare kernel, Gamma_ts = F_t * mid * R_s across 16-token blocks and
    // F4_t * mid4 * R4_s across 4-token sub-blocks of one block; pairs inside one sub-block are
    // direct products.
    for (int pp = 0; pp < DG / DH; ++pp) {
        const int p0 = gc0 + pp * DH;  // the pass's first channel
        const int ic = rr;             // this lane's B / output column, within the pass
        const size_t ocol = size_t(p0 + ic);
        __syncthreads();  // the previous pass is finished with the pass arrays
        {
            const int t = tid >> 2, ii = 4 * (tid & 3);
            const bool ok = t < nval;
            *reinterpret_cast<f32x4_t *>(&sA[t * LDH + ii]) = ok ? cur.a : f32x4_t{1.f, 1.f, 1.f, 1.f};
            *reinterpret_cast<f32x4_t *>(&sK[t * LDH + ii]) = ok ? cvt4(cur.k) : zero4();
            *reinterpret_cast<f32x4_t *>(&sQ[t * LDH + ii]) = ok ? cur.g * cvt4(cur.q) * cur.r : zero4();
        }
        // The next pass's operands (the last pass reloads its own, unused).
        PassIn nxt;
        load_pass(pp + 1 < DG / DH ? p0 + DH : p0, nxt);
        __syncthreads();
        {
            // Pivots, thread (channel, 16-token block, role = wave): 0 the prefix F inside the
            // block, 1 the suffix R and the block's product, 2 and 3 the prefix F4, suffix R4
            // and product of two sub-blocks each.
            const int ii = tid % DH, bb = (tid / DH) % kNB;
            if (wave == 0) {
                float run = 1.f;
#pragma unroll
                for (int tl = 0; tl < 16; ++tl) {
                    run *= sA[(16 * bb + tl) * LDH + ii];
                    sF[(16 * bb + tl) * LDH + ii] = run;
                }
            } else if (wave == 1) {
                float run = 1.f;
#pragma unroll
                for (int tl = 15; tl >= 0; --tl) {
                    sR[(16 * bb + tl) * LDH + ii] = run;
                    run *= sA[(16 * bb + tl) * LDH + ii];
                }
                sBp[bb * DH + ii] = run;
            } else {
#pragma unroll
                for (int u2 = 0; u2 < 2; ++u2) {
                    const int u = 4 * bb + 2 * (wave - 2) + u2;
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
        {
            // Rows t of block bt = w: dq_hat and the read part of dk.
            const int bt = wave;
            f32x4_t cq = zero4(), cr = zero4(), dq4 = zero4(), dr4 = zero4();
            float drl = 0.f;  // this lane's share of dr: its four tokens, in order
#pragma unroll
            for (int bs = 0; bs < kNB - 1; ++bs) {
                if (bs >= bt) break;
                f32x4_t yq = zero4(), yr = zero4();
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int kk = 4 * m + kq, sg = 16 * bs + kk;
                    const float bv = sK[sg * LDH + ic] * sR[sg * LDH + ic];
                    yq = __builtin_amdgcn_mfma_f32_16x16x4f32(sOU[(16 * bt + rr) * LDM + sg], bv, yq, 0, 0, 0);
                    yr = __builtin_amdgcn_mfma_f32_16x16x4f32(sPU[(16 * bt + rr) * LDM + sg], bv, yr, 0, 0, 0);
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
                    const float bv = sK[sg * LDH + ic] * sR4[sg * LDH + ic] * mid4;
                    const float aq = on ? sOU[(16 * bt + rr) * LDM + sg] : 0.f;
                    const float ar = on ? sPU[(16 * bt + rr) * LDM + sg] : 0.f;
                    yq = __builtin_amdgcn_mfma_f32_16x16x4f32(aq, bv, yq, 0, 0, 0);
                    yr = __builtin_amdgcn_mfma_f32_16x16x4f32(ar, bv, yr, 0, 0, 0);
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
                const float gam = sGb[bt * DH + ic] * fb;
                const float dqh = gam * cur.y1[e4] + fb * cq[e4] + f4 * dq4[e4] + sq;
                const float dkr = gam * cur.y2[e4] + fb * cr[e4] + f4 * dr4[e4] + sr;
                sDkr[t * LDO + ic] = dkr;
                sLa[t * LDO + ic] = fmaf(sQ[t * LDH + ic], dqh, sK[t * LDH + ic] * dkr);
                if (t < nval) {
                    const size_t o = tok0 + size_t(t) * HD + ocol;
                    const float gt = cur.gg[e4], qt = to_f32(cur.gq[e4]);
                    dq[o] = rh[ocol] * gt * dqh;
                    dg[o] = rh[ocol] * qt * dqh;
                    drl += gt * qt * dqh;
                }
            }
            sDrP[(bt * 4 + kq) * DH + ic] = drl;
        }
        {
            // Rows s of block bs = w: the write part of dk.
            const int bs = wave;
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
                const float rb_ = sR[s4 * LDH + ic], r4 = sR4[s4 * LDH + ic];
                const float bet = rb_ * sBa[bs * DH + ic];
                sDkw[s4 * LDO + ic] = bet * cur.y3[e4] + rb_ * cw[e4] + r4 * dw4[e4] + sw;
            }
        }
        __syncthreads();
        {
            // dk = read part + write part, and the log-decay gradient: a reverse cumulative sum
            // over the chunk per channel of q_hat dq_hat + k dk_read - k dk_write, plus
            // rowsum(S_C * lambda_C). Thread (channel, part) takes four consecutive tokens.
            const int ii = tid % DH, part = tid / DH;
            float cum[4], run = 0.f;
#pragma unroll
            for (int u = 3; u >= 0; --u) {
                const int t = 4 * part + u;
                run += sLa[t * LDO + ii] - sK[t * LDH + ii] * sDkw[t * LDO + ii];
                cum[u] = run;
            }
            sTot[part * DH + ii] = run;
            if (tid < DH) {
                // The dr partials of the pass, added in a fixed order (block, then lane group).
                float sum = 0.f;
#pragma unroll
                for (int x = 0; x < kNB * 4; ++x) sum += sDrP[x * DH + tid];
                sDr[pp * DH + tid] = sum;
            }
            __syncthreads();
            float off = sRS[pp * DH + ii];
            for (int p2 = part + 1; p2 < C / 4; ++p2) off += sTot[p2 * DH + ii];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = 4 * part + u;
                if (t < nval) {
                    const size_t o = tok0 + size_t(t) * HD + p0 + ii;
                    dla[o] = cum[u] + off;
                    dk[o] = sDkr[t * LDO + ii] + sDkw[t * LDO + ii];
                }
            }
        }
        cur = nxt;
    }
    __syncthreads();
    for (int i = tid; i < DG; i += kBwdThreads) drp[slot * D + gc0 + i] = sDr[i];
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

template <typename QT, int D>
hipError_t bwd_typed(const ChunkBwdArgs &x, int B, int T, int H, unsigned char *ws, const BwdLayout &L,
                     hipStream_t stream) {
    const int nchunks = (T + kC - 1) / kC;
    const int BH = B * H;
    float *u = reinterpret_cast<float *>(ws + L.u);
    float *states = reinterpret_cast<float *>(ws + L.states);
    // The scan's operands K*beta, K*gamma, Q_hat*gamma and P^T are stored in the operand
    // precision (bf16 on the bf16 path); their regions are sized for fp32 because the products
    // kernel reuses them afterwards.
    QT *kb = reinterpret_cast<QT *>(ws + L.kb), *kg = reinterpret_cast<QT *>(ws + L.kg);
    QT *qg = reinterpret_cast<QT *>(ws + L.qg), *Pw = reinterpret_cast<QT *>(ws + L.P);
    float *gC = reinterpret_cast<float *>(ws + L.gC), *Mw = reinterpret_cast<float *>(ws + L.M);
    float *pred = reinterpret_cast<float *>(ws + L.pred), *dUw = reinterpret_cast<float *>(ws + L.dU);
    float *lamC = reinterpret_cast<float *>(ws + L.lamC);
    float *drp = reinterpret_cast<float *>(ws + L.drp);
    const bool bf16 = std::is_same_v<QT, bf16_t>;
    hipError_t err;
    // The forward rerun, at its own chunk size, keeping u and the state every 64 tokens.
    const int cf = bwd_fwd_chunk(B, T, H, D);
    if (T > 0) {
        err = bf16 ? launch_chunk_prepare_state(x.k, x.a, x.g, x.r, B, T, H, D, cf, ws + L.fwd, stream)
                   : launch_chunk_prepare(x.q, x.k, x.a, x.g, x.r, B, T, H, D, cf, bf16, ws + L.fwd, stream);
        if (err != hipSuccess) return err;
    }
    err = launch_chunk_scan_save(x.v, x.e, x.w, x.s0, nullptr, nullptr, u, states, B, T, H, D, cf, bf16,
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
        // The products go where the scan's operands were (K*beta, K*gamma, Q_hat*gamma, M, P and
        // gamma_C are not read again): Y1, Y2, Y3 over kb, kg, qg, OU, PU over M, P, and the
        // rowsums over gamma_C.
        float *Y1 = reinterpret_cast<float *>(ws + L.kb), *Y2 = reinterpret_cast<float *>(ws + L.kg);
        float *Y3 = reinterpret_cast<float *>(ws + L.qg), *OU = Mw, *PU = reinterpret_cast<float *>(ws + L.P);
        hipLaunchKernelGGL((bwd_products_kernel<QT, D>), dim3(nchunks, H, B), dim3(kBwdThreads), 0, stream, dout,
                           x.e, u, dUw, states, lamC, Y1, Y2, Y3, OU, PU, gC, T, H, nchunks);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
        auto kgk = bwd_grads_kernel<QT, D>;
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(kgk), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  int(GradLds<D>::BYTES));
        if (err != hipSuccess) return err;
        const int nwork = BH * nchunks;
        const int nwg = (nwork + 7) / 8 * 8 * GradLds<D>::G;
        hipLaunchKernelGGL(kgk, dim3(nwg), dim3(kBwdThreads), GradLds<D>::BYTES, stream, q, k, x.a, x.g, x.r,
                           states, lamC, Y1, Y2, Y3, OU, PU, gC, x.dq, x.dk, x.dg, x.dla, drp, T, H, nchunks, nwork);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL((bwd_dr_kernel<D>), dim3(H), dim3(1024), 0, stream, drp, x.dr, B, H, nchunks);
    return hipGetLastError();
}

}  // namespace

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
