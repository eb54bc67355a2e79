// Fused single-token recurrent step (decode), one workgroup per (batch, head).
//
// Constant-memory inference against a fixed per-head state (Muir abstract, "Full
// text" on the Astral Feed page; openai-hub news page, opening section). For one token:
//   p_j  = sum_i a_i k_i S_ij            prediction of the decayed state for k
//   y_j  = sum_i a_i qh_i S_ij           readout of the decayed state, qh = r*g*q
//   u_j  = w_j v_j - e_j p_j             erase (value-channel gate) then write
//   S_ij <- a_i S_ij + k_i u_j
//   o_j  = sum_i qh_i S_ij(new) = y_j + (qh . k) u_j
// Both reductions need only the OLD state, so S is read once into registers, reduced
// over rows, updated and written once: 2 * dk * dv * 4 bytes of state traffic per
// head-step, which is the whole cost (the step is HBM-bound, about 1 flop/byte).
//
// Layout: state [B,H,dk,dv] fp32 with dv contiguous. A thread owns 4 consecutive
// columns (one float4) of ROWS rows strided by ROW_GROUPS, so each wave reads whole
// contiguous rows (coalesced 16-byte loads) and all loads are issued up front. The new
// state is written with non-temporal stores: it is not read again in this step.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace muir {

namespace {

constexpr int kDecodeThreads = 512;

template <typename QT, int D>
__global__ __launch_bounds__(kDecodeThreads) void decode_step_kernel(
    const QT *__restrict__ q, const QT *__restrict__ k, const QT *__restrict__ v,
    const float *__restrict__ a, const float *__restrict__ g,
    const float *__restrict__ e, const float *__restrict__ w,
    const float *__restrict__ r, float *__restrict__ state, QT *__restrict__ o, int H) {
    constexpr int TPR = D / 4;                       // threads per row (float4 each)
    constexpr int ROW_GROUPS = kDecodeThreads / TPR;  // rows handled in parallel
    constexpr int ROWS = D / ROW_GROUPS;              // rows per thread
    static_assert(D % 4 == 0 && kDecodeThreads % TPR == 0 && D % ROW_GROUPS == 0, "shape");

    __shared__ float sh_ak[D], sh_aq[D], sh_k[D], sh_a[D];
    __shared__ float sh_b[D], sh_e[D], sh_u[D];
    __shared__ float sh_part[2][ROW_GROUPS][D];
    __shared__ float sh_qk;

    const int bh = blockIdx.x;              // b * H + h
    const int h = bh % H;
    const int tid = threadIdx.x;
    const int c4 = tid % TPR;               // column quad
    const int rg = tid / TPR;               // row group

    float4 *S4 = reinterpret_cast<float4 *>(state + static_cast<size_t>(bh) * D * D);
    float4 s[ROWS];
#pragma unroll
    for (int m = 0; m < ROWS; ++m) s[m] = S4[(rg + m * ROW_GROUPS) * TPR + c4];

    const size_t vo = static_cast<size_t>(bh) * D;
    if (tid < D) {
        const float ai = a[vo + tid];
        const float ki = elem<QT>::load(k, vo + tid);
        const float qh = r[static_cast<size_t>(h) * D + tid] * g[vo + tid] *
                         elem<QT>::load(q, vo + tid);
        sh_a[tid] = ai;
        sh_k[tid] = ki;
        sh_ak[tid] = ai * ki;
        sh_aq[tid] = ai * qh;
        sh_b[tid] = w[vo + tid] * elem<QT>::load(v, vo + tid);
        sh_e[tid] = e[vo + tid];
        // q_hat . k over the D rows: the first D threads are whole waves (D >= 64).
        float part = wave_sum(qh * ki);
        if (D == 64) {
            if (tid == 0) sh_qk = part;
        } else {
            if ((tid & 63) == 0) sh_part[0][0][tid >> 6] = part;
        }
    }
    __syncthreads();
    if (D != 64 && tid == 0) {
        float t = 0.f;
        for (int i = 0; i < D / 64; ++i) t += sh_part[0][0][i];
        sh_qk = t;
    }
    __syncthreads();

    float4 p = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < ROWS; ++m) {
        const int i = rg + m * ROW_GROUPS;
        const float ak = sh_ak[i], aq = sh_aq[i];
        p.x += ak * s[m].x; p.y += ak * s[m].y; p.z += ak * s[m].z; p.w += ak * s[m].w;
        y.x += aq * s[m].x; y.y += aq * s[m].y; y.z += aq * s[m].z; y.w += aq * s[m].w;
    }
    reinterpret_cast<float4 *>(sh_part[0][rg])[c4] = p;
    reinterpret_cast<float4 *>(sh_part[1][rg])[c4] = y;
    __syncthreads();

    if (tid < D) {
        float pj = 0.f, yj = 0.f;
#pragma unroll
        for (int i = 0; i < ROW_GROUPS; ++i) {
            pj += sh_part[0][i][tid];
            yj += sh_part[1][i][tid];
        }
        const float uj = sh_b[tid] - sh_e[tid] * pj;
        sh_u[tid] = uj;
        elem<QT>::store(o, vo + tid, yj + sh_qk * uj);
    }
    __syncthreads();

    const float4 u = reinterpret_cast<const float4 *>(sh_u)[c4];
#pragma unroll
    for (int m = 0; m < ROWS; ++m) {
        const int i = rg + m * ROW_GROUPS;
        const float ai = sh_a[i], ki = sh_k[i];
        const f32x4_t t = {ai * s[m].x + ki * u.x, ai * s[m].y + ki * u.y,
                           ai * s[m].z + ki * u.z, ai * s[m].w + ki * u.w};
        __builtin_nontemporal_store(t, reinterpret_cast<f32x4_t *>(&S4[i * TPR + c4]));
    }
}

}  // namespace

hipError_t launch_decode_step(const void *q, const void *k, const void *v, const float *a,
                              const float *g, const float *e, const float *w, const float *r,
                              float *state, void *o, int B, int H, int d, bool bf16,
                              hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(B) * static_cast<unsigned>(H));
    const dim3 block(kDecodeThreads);
#define MUIR_DECODE(QT, D)                                                              \
    hipLaunchKernelGGL((decode_step_kernel<QT, D>), grid, block, 0, stream,             \
                       static_cast<const QT *>(q), static_cast<const QT *>(k),          \
                       static_cast<const QT *>(v), a, g, e, w, r, state,                \
                       static_cast<QT *>(o), H)
    if (bf16) {
        if (d == 64) MUIR_DECODE(bf16_t, 64); else MUIR_DECODE(bf16_t, 128);
    } else {
        if (d == 64) MUIR_DECODE(float, 64); else MUIR_DECODE(float, 128);
    }
#undef MUIR_DECODE
    return hipGetLastError();
}

}  // namespace muir
