// Shared device helpers for libmuir's gfx950 kernels: element types, bf16
// conversion, wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muir {

// Raw bfloat16 storage (upper 16 bits of an IEEE float32).
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float32 -> bfloat16 bits. The __bf16 conversion lowers to
// gfx950's v_cvt_pk_bf16_f32 (nearest-even, NaN stays NaN), with no branches.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x.bits); }

// Element access for the two q/k/v/o types.
template <typename T> struct elem;

template <> struct elem<float> {
    static __device__ __forceinline__ float load(const float *p, size_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float *p, size_t i, float x) { p[i] = x; }
};

template <> struct elem<bf16_t> {
    static __device__ __forceinline__ float load(const bf16_t *p, size_t i) {
        return bf16_to_f32(p[i].bits);
    }
    static __device__ __forceinline__ void store(bf16_t *p, size_t i, float x) {
        p[i].bits = f32_to_bf16(x);
    }
};

// Activations of the low-rank gate projection: the decay from its log rate y, in (0, 1],
// and the logistic function for the other gates.
__device__ __forceinline__ float gate_decay(float y) { return __expf(-__expf(y)); }
__device__ __forceinline__ float gate_sigmoid(float y) { return 1.f / (1.f + __expf(-y)); }

// Sum over the 64 lanes of a wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

}  // namespace muir
