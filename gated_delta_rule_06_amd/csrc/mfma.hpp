// gfx950 matrix-core (MFMA) helpers for the chunk kernels.
//
// Every contraction in the chunk forward is D[16x16] += A[16xK] * B[Kx16] with the
// operands held as "row x contraction" matrices on both sides: A rows are output rows,
// B "rows" are output columns. Both operands therefore use the same fragment layout.
//
//   bf16 operands: v_mfma_f32_16x16x32_bf16. Per instruction K = 32; lane l holds
//                  row (l % 16) and contraction indices 8*(l / 16) + [0, 8).
//   fp32 operands: v_mfma_f32_16x16x4_f32.   Per instruction K = 4; lane l holds
//                  row (l % 16) and contraction index (l / 16).
//   Accumulator (both): 16x16 fp32, lane l holds column (l % 16), rows 4*(l/16)+[0,4).
//
// Accumulation is always fp32.
#pragma once

#include "common.hpp"

namespace muir {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

template <typename OpT> struct Mma;

template <> struct Mma<bf16_t> {
    static constexpr int KSTEP = 32;  // contraction length per instruction
    static constexpr int VALS = 8;    // contraction values per lane
    using frag = bf16x8_t;

    // Contraction index (within one KSTEP block) of element j held by lane l.
    static __device__ __forceinline__ int kidx(int lane, int j) { return (lane >> 4) * 8 + j; }

    static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // Round 8 floats to bf16 (nearest even) into one fragment.
    static __device__ __forceinline__ frag pack(const float (&x)[8]) {
        u16x8_t u;
#pragma unroll
        for (int j = 0; j < 8; ++j) u[j] = f32_to_bf16(x[j]);
        return __builtin_bit_cast(frag, u);
    }
    // Fragment from 8 consecutive stored operands (16-byte aligned).
    static __device__ __forceinline__ frag load(const bf16_t *p) {
        return __builtin_bit_cast(frag, *reinterpret_cast<const u16x8_t *>(p));
    }
    static __device__ __forceinline__ frag zero() {
        u16x8_t u = {0, 0, 0, 0, 0, 0, 0, 0};
        return __builtin_bit_cast(frag, u);
    }
    static __device__ __forceinline__ void store(bf16_t *p, const float (&x)[8]) {
        u16x8_t u;
#pragma unroll
        for (int j = 0; j < 8; ++j) u[j] = f32_to_bf16(x[j]);
        *reinterpret_cast<u16x8_t *>(p) = u;
    }
    static __device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x.bits); }
    static __device__ __forceinline__ bf16_t from_f32(float x) { return bf16_t{f32_to_bf16(x)}; }
};

template <> struct Mma<float> {
    static constexpr int KSTEP = 4;
    static constexpr int VALS = 1;
    using frag = float;

    static __device__ __forceinline__ int kidx(int lane, int) { return lane >> 4; }

    static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ frag pack(const float (&x)[1]) { return x[0]; }
    static __device__ __forceinline__ frag load(const float *p) { return *p; }
    static __device__ __forceinline__ frag zero() { return 0.f; }
    static __device__ __forceinline__ void store(float *p, const float (&x)[1]) { *p = x[0]; }
    static __device__ __forceinline__ float to_f32(float x) { return x; }
    static __device__ __forceinline__ float from_f32(float x) { return x; }
};

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// N consecutive elements (16-byte aligned for N >= 4) as floats.
template <int N> __device__ __forceinline__ void load_vec(const float *p, float (&x)[N]) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const float4 t = reinterpret_cast<const float4 *>(p)[i];
            x[4 * i] = t.x; x[4 * i + 1] = t.y; x[4 * i + 2] = t.z; x[4 * i + 3] = t.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = p[i];
    }
}
template <int N> __device__ __forceinline__ void load_vec(const bf16_t *p, float (&x)[N]) {
    if constexpr (N == 8) {
        const u16x8_t u = *reinterpret_cast<const u16x8_t *>(p);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = bf16_to_f32(u[i]);
    } else if constexpr (N == 4) {
        const u16x4_t u = *reinterpret_cast<const u16x4_t *>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = bf16_to_f32(u[i]);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = bf16_to_f32(p[i].bits);
    }
}
// Four consecutive elements from an fp32 accumulator.
__device__ __forceinline__ void store4(float *p, f32x4_t v) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(bf16_t *p, f32x4_t v) {
    u16x4_t u;
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = f32_to_bf16(v[i]);
    *reinterpret_cast<u16x4_t *>(p) = u;
}

// Workgroup barrier that orders LDS only. Waves of one workgroup never exchange data
// through global memory inside these kernels, so global loads issued as prefetches
// stay in flight across the barrier (a full __syncthreads() would wait for them).
// The scheduling barriers keep every instruction on its side of the barrier: without
// them the machine scheduler, which sees one region across many unrolled phases, sinks
// prefetch loads down to their uses to save registers and so undoes the prefetch.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    __builtin_amdgcn_sched_barrier(0);
}

// Order this wave's LDS writes before its following LDS reads from other lanes.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace muir
