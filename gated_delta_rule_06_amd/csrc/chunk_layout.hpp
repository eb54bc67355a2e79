// Layout of the chunk-forward workspace and the matrix-core operand helpers shared by the
// chunk kernels (the channel-wise scan and the shared-erase variant).
#pragma once

#include <stddef.h>
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "layout.hpp"
#include "mfma.hpp"

namespace muir {

// Slot<OpT, D, C>: the workspace slot of one (batch, head, chunk) (layout.hpp), for operands of
// type OpT.
template <typename OpT, int D, int C> using Slot = SlotLayout<int(sizeof(OpT)), D, C>;

// Storage position of index x under the 32-group permutation described above.
__host__ __device__ constexpr int pair_perm(int x) {
    return (x & ~31) | (((x >> 2) & 3) << 3) | (((x >> 4) & 1) << 2) | (x & 3);
}

// Fragment order of the operands Kg, Qg ([C rows][D positions]) and KbT ([D][C]): the
// operand a lane group needs for one 16-row group and one 32-position group is 64
// lanes x 8 values, stored contiguously with lane 16G + r holding row r and positions
// 8G .. 8G + 7 of the group. The scan then reads a whole fragment as one contiguous
// 16-byte (bf16) load per lane, eight full cache lines per load. Element (row, pos) of
// an operand with npos positions per row:
__host__ __device__ constexpr size_t frag_idx(int row, int pos, int npos) {
    return ((size_t(row >> 4) * (npos >> 5) + (pos >> 5)) * 64 + 16 * ((pos & 31) >> 3) + (row & 15)) * 8 +
           (pos & 7);
}


// Every product of the scan is D[16x16] += A[16xK] B[16xK]^T on the matrix cores with
// K = 16 (mma4, four values per lane) or K = 32 (mma8, eight values per lane). Lane l
// holds row l%16 of each operand; which contraction index its j-th value stands for is
// chosen by the caller, the same on both sides, so the hardware's own k order never
// matters. Accumulator: lane l holds column l%16, rows 4(l/16) + i.
// Buffer resources: every load and store of the scan goes through a descriptor whose
// base is wave-uniform, with a 32-bit per-lane byte offset and a uniform byte offset.
// Reads past num_records return zero and writes past it are dropped, which is how the
// tokens past the end of the sequence are handled.
using rsrc_t = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, int(bytes), 0x00020000);
}
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2_t buf_load8(rsrc_t r, unsigned voff, unsigned soff) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, int(voff), int(soff), 0);
}
__device__ __forceinline__ u32x4_t buf_load16(rsrc_t r, unsigned voff, unsigned soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, int(voff), int(soff), 0);
}
__device__ __forceinline__ f32x4_t buf_load_f4(rsrc_t r, unsigned voff, unsigned soff) {
    return __builtin_bit_cast(f32x4_t, buf_load16(r, voff, soff));
}

template <typename OpT> struct Frag;
template <> struct Frag<bf16_t> {
    using f4 = u16x4_t;
    using f8 = u16x8_t;
    static __device__ __forceinline__ f4 bload4(rsrc_t r, unsigned voff, unsigned soff) {
        return __builtin_bit_cast(u16x4_t, buf_load8(r, voff, soff));
    }
    static __device__ __forceinline__ f8 bload8(rsrc_t r, unsigned voff, unsigned soff) {
        return __builtin_bit_cast(u16x8_t, buf_load16(r, voff, soff));
    }
    static __device__ __forceinline__ f4 load4(const bf16_t *p) {
        return *reinterpret_cast<const u16x4_t *>(p);
    }
    static __device__ __forceinline__ f8 load8(const bf16_t *p) {
        return *reinterpret_cast<const u16x8_t *>(p);
    }
    static __device__ __forceinline__ f8 cat(f4 a, f4 b) {
        return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    static __device__ __forceinline__ f4 lo(f8 v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3); }
    static __device__ __forceinline__ f4 hi(f8 v) { return __builtin_shufflevector(v, v, 4, 5, 6, 7); }
    static __device__ __forceinline__ f4 pack(f32x4_t v) {
        u16x4_t u;
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = f32_to_bf16(v[i]);
        return u;
    }
    // Lane (n, g) of the 16x16 identity as an mma4 operand: value j is I[n][4g + j].
    static __device__ __forceinline__ f4 unit(int n, int g) {
        u16x4_t u;
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] = n == 4 * g + j ? 0x3f80 : 0;
        return u;
    }
    // K = 16 products run as the K = 32 instruction with a zero upper half: an
    // accumulation chain that alternates the 16x16x16 and 16x16x32 bf16 instructions
    // needs more wait states between them than the compiler inserts on gfx950, so only
    // one instruction kind is ever used.
    static __device__ __forceinline__ f32x4_t mma4(f4 a, f4 b, f32x4_t c) {
        const f4 z = {0, 0, 0, 0};
        return mma8(cat(a, z), cat(b, z), c);
    }
    static __device__ __forceinline__ f32x4_t mma8(f8 a, f8 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
    // The 16x16x16 instruction itself, with no accumulator input: nothing to chain with.
    static __device__ __forceinline__ f32x4_t mma16_fresh(f4 a, f4 b) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                         __builtin_bit_cast(s16x4_t, b), zero4(), 0, 0, 0);
    }
};
template <> struct Frag<float> {
    using f4 = f32x4_t;
    struct f8 {
        f32x4_t lo, hi;
    };
    static __device__ __forceinline__ f4 load4(const float *p) {
        const float4 t = *reinterpret_cast<const float4 *>(p);
        return f32x4_t{t.x, t.y, t.z, t.w};
    }
    static __device__ __forceinline__ f8 load8(const float *p) { return {load4(p), load4(p + 4)}; }
    static __device__ __forceinline__ f4 bload4(rsrc_t r, unsigned voff, unsigned soff) {
        return buf_load_f4(r, voff, soff);
    }
    static __device__ __forceinline__ f8 bload8(rsrc_t r, unsigned voff, unsigned soff) {
        return {buf_load_f4(r, voff, soff), buf_load_f4(r, voff + 16, soff)};
    }
    static __device__ __forceinline__ f8 cat(f4 a, f4 b) { return {a, b}; }
    static __device__ __forceinline__ f4 lo(f8 v) { return v.lo; }
    static __device__ __forceinline__ f4 hi(f8 v) { return v.hi; }
    static __device__ __forceinline__ f4 pack(f32x4_t v) { return v; }
    static __device__ __forceinline__ f4 unit(int n, int g) {
        f32x4_t u;
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] = n == 4 * g + j ? 1.f : 0.f;
        return u;
    }
    static __device__ __forceinline__ f32x4_t mma4(f4 a, f4 b, f32x4_t c) {
#pragma unroll
        for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ f32x4_t mma8(f8 a, f8 b, f32x4_t c) {
        return mma4(a.hi, b.hi, mma4(a.lo, b.lo, c));
    }
    static __device__ __forceinline__ f32x4_t mma16_fresh(f4 a, f4 b) { return mma4(a, b, zero4()); }
};

// Calls fn(std::integral_constant<int, 0>{}) ... fn(std::integral_constant<int, N-1>{}) in
// order, so that indices into register arrays are compile-time constants.
template <typename Fn, int... Is>
__device__ __forceinline__ void static_for_impl(Fn &&fn, std::integer_sequence<int, Is...>) {
    (fn(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename Fn> __device__ __forceinline__ void static_for(Fn &&fn) {
    static_for_impl(fn, std::make_integer_sequence<int, N>{});
}

// VC (4, 2 or 1) consecutive q/k/v-typed elements through a buffer resource, held as the
// first VC values of a four-vector; the other values are zero.
template <int VC> __device__ __forceinline__ f32x4_t buf_load_fn(rsrc_t r, unsigned voff, unsigned soff) {
    static_assert(VC == 4 || VC == 2 || VC == 1, "VC is 4, 2 or 1");
    if constexpr (VC == 4) {
        return buf_load_f4(r, voff, soff);
    } else if constexpr (VC == 2) {
        // Whole-vector casts only: this compiler lowers __builtin_bit_cast of a subscripted
        // vector element as a read of element 0.
        const f32x2_t f = __builtin_bit_cast(f32x2_t, buf_load8(r, voff, soff));
        return f32x4_t{f[0], f[1], 0.f, 0.f};
    } else {
        const unsigned u = __builtin_amdgcn_raw_buffer_load_b32(r, int(voff), int(soff), 0);
        return f32x4_t{__builtin_bit_cast(float, u), 0.f, 0.f, 0.f};
    }
}
template <typename QT, int VC> struct RowV;
template <int VC> struct RowV<bf16_t, VC> {
    static_assert(VC == 4 || VC == 2 || VC == 1, "VC is 4, 2 or 1");
    using raw = u16x4_t;
    static __device__ __forceinline__ raw load(rsrc_t r, unsigned voff, unsigned soff) {
        if constexpr (VC == 4) {
            return __builtin_bit_cast(u16x4_t, buf_load8(r, voff, soff));
        } else if constexpr (VC == 2) {
            const unsigned u = __builtin_amdgcn_raw_buffer_load_b32(r, int(voff), int(soff), 0);
            return u16x4_t{uint16_t(u & 0xffffu), uint16_t(u >> 16), 0, 0};
        } else {
            const uint16_t u = __builtin_amdgcn_raw_buffer_load_b16(r, int(voff), int(soff), 0);
            return u16x4_t{u, 0, 0, 0};
        }
    }
    static __device__ __forceinline__ float get(raw v, int i) { return bf16_to_f32(v[i]); }
    static __device__ __forceinline__ void store(rsrc_t r, unsigned voff, unsigned soff, f32x4_t v) {
        if constexpr (VC == 4) {
            u16x4_t u;
#pragma unroll
            for (int i = 0; i < 4; ++i) u[i] = f32_to_bf16(v[i]);
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, u), r, int(voff), int(soff), 0);
        } else if constexpr (VC == 2) {
            const unsigned u = unsigned(f32_to_bf16(v[0])) | (unsigned(f32_to_bf16(v[1])) << 16);
            __builtin_amdgcn_raw_buffer_store_b32(u, r, int(voff), int(soff), 0);
        } else {
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v[0]), r, int(voff), int(soff), 0);
        }
    }
};
template <int VC> struct RowV<float, VC> {
    static_assert(VC == 4 || VC == 2 || VC == 1, "VC is 4, 2 or 1");
    using raw = f32x4_t;
    static __device__ __forceinline__ raw load(rsrc_t r, unsigned voff, unsigned soff) {
        return buf_load_fn<VC>(r, voff, soff);
    }
    static __device__ __forceinline__ float get(raw v, int i) { return v[i]; }
    static __device__ __forceinline__ void store(rsrc_t r, unsigned voff, unsigned soff, f32x4_t v) {
        if constexpr (VC == 4) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, int(voff), int(soff), 0);
        } else if constexpr (VC == 2) {
            const f32x2_t f = {v[0], v[1]};
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, f), r, int(voff), int(soff), 0);
        } else {
            const float f = v[0];
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, f), r, int(voff), int(soff), 0);
        }
    }
};
// Four consecutive elements.
template <typename QT> using Row4 = RowV<QT, 4>;

}  // namespace muir
