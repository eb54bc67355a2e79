// Gates of the recurrence from the fused low-rank gate projection.
//
// The pages fuse all five gates into one projection of total rank 512: one shared
// down-projection, then a separate up-projection per gate with its own rank, decay 64,
// erase 64, output 128, write 128 and dynamic read 128 (openai-hub news page, section on
// sensitivity-allocated gating, gate table; liuch.name summary, second bullet). The
// down-projection's output z [B, T, 512] (rank slices in the table's order) is the input;
// per gate n, with U_n [H, d, r_n] and an offset c_n [H, d]:
//   y_n = z[..., slice_n] U_n^T + c_n,   a = exp(-exp(y_decay)),   e, w, g = sigmoid(y)
// (y_decay is a log decay rate, so a lies in (0, 1]). The output gate's slice feeds none of
// the four.
//
// Each product is a 16-token x 16-channel tile with the rank as the contraction, on the
// matrix cores: the up-projection's rows (channels) are the A operand and z's rows
// (tokens) the B operand, so lane (t, G) of the accumulator holds token t and channels
// 4G .. 4G + 3 of the tile: one 16-byte store of four gate values per lane.
#include "chunk_layout.hpp"
#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace muir {

namespace {

// Rank offsets of the four gates' slices of z, and their ranks.
constexpr int kZRank = 512;
constexpr int kOffDecay = 0, kOffErase = 64, kOffWrite = 256, kOffRead = 384;
constexpr int kRankDecay = 64, kRankErase = 64, kRankWrite = 128, kRankRead = 128;

__device__ __forceinline__ float decay_of(float y) { return __expf(-__expf(y)); }
__device__ __forceinline__ float sigmoid_of(float y) { return 1.f / (1.f + __expf(-y)); }

// One gate's up-projection rows for one 16-channel tile, held as A operands: lane (x, G)
// holds channel 16c + x, ranks 32s + 8G .. + 7 of K-step s.
template <int R> struct UpRows {
    Frag<bf16_t>::f8 f[R / 32];
    f32x4_t off;  // c_n at channels 16c + 4G + r (the accumulator's rows of lane (t, G))
};

template <int R>
__device__ __forceinline__ void load_up(UpRows<R> &u, const bf16_t *U, const float *c, int h,
                                        int D, int ch0, int lane) {
    const int x = lane & 15, G = lane >> 4;
#pragma unroll
    for (int s = 0; s < R / 32; ++s)
        u.f[s] = Frag<bf16_t>::load8(U + (size_t(h) * D + ch0 + x) * R + 32 * s + 8 * G);
    u.off = *reinterpret_cast<const f32x4_t *>(c + size_t(h) * D + ch0 + 4 * G);
}

// y (pre-activation) of one gate for the token block whose z rows this lane group loaded.
template <int R>
__device__ __forceinline__ f32x4_t preact(const UpRows<R> &u, const Frag<bf16_t>::f8 *zr) {
    f32x4_t acc = u.off;
#pragma unroll
    for (int s = 0; s < R / 32; ++s) acc = Frag<bf16_t>::mma8(u.f[s], zr[s], acc);
    return acc;
}

// One wavefront per (head, 16-channel tile, batch, token-block group): the up-projection
// rows stay in registers while the wavefront walks its token blocks. Gates whose output
// pointer is null are skipped.
template <int D>
__global__ __launch_bounds__(256) void lowrank_gates_kernel(
    const bf16_t *__restrict__ z, const bf16_t *__restrict__ Ua, const bf16_t *__restrict__ Ue,
    const bf16_t *__restrict__ Uw, const bf16_t *__restrict__ Ug, const float *__restrict__ ca,
    const float *__restrict__ ce, const float *__restrict__ cw, const float *__restrict__ cg,
    float *__restrict__ a, float *__restrict__ e, float *__restrict__ w, float *__restrict__ g,
    int T, int H, int nwaves_t) {
    using F = Frag<bf16_t>;
    using f8 = F::f8;
    constexpr int NCT = D / 16;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63, x = lane & 15, G = lane >> 4;
    const int h = blockIdx.x / NCT, c = blockIdx.x % NCT, b = blockIdx.y;
    const int tw = blockIdx.z * 4 + wave;  // this wavefront's index along the token blocks
    const int ch0 = 16 * c;
    const int nblk = (T + 15) / 16;

    UpRows<kRankDecay> ua;
    UpRows<kRankErase> ue;
    UpRows<kRankWrite> uw;
    UpRows<kRankRead> ug;
    if (a) load_up(ua, Ua, ca, h, D, ch0, lane);
    if (e) load_up(ue, Ue, ce, h, D, ch0, lane);
    if (w) load_up(uw, Uw, cw, h, D, ch0, lane);
    if (g) load_up(ug, Ug, cg, h, D, ch0, lane);

    // z rows of this batch through a descriptor: tokens at or past T read zero. Gate
    // stores likewise: tokens at or past T are dropped.
    const rsrc_t rz = make_rsrc(z + size_t(b) * T * kZRank, unsigned(size_t(T) * kZRank * 2));
    const size_t HD = size_t(H) * D;
    const size_t gbase = size_t(b) * T * HD + size_t(h) * D + ch0;  // uniform
    const unsigned gbytes = unsigned((size_t(T) * HD - size_t(h) * D - ch0) * 4);
    auto store = [&](float *p, int t, f32x4_t v) {
        const rsrc_t r = make_rsrc(p + gbase, gbytes);
        const unsigned off = (unsigned(min(t, T)) * unsigned(HD) + unsigned(4 * G)) * 4u;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, int(off), 0, 0);
    };
    for (int tb = tw; tb < nblk; tb += nwaves_t) {
        const int t = 16 * tb + x;
        const unsigned zoff = unsigned(min(t, T)) * unsigned(kZRank) * 2u + unsigned(8 * G) * 2u;
        auto zrow = [&](int off, f8 *dst, int nsteps) {
#pragma unroll
            for (int s = 0; s < nsteps; ++s)
                dst[s] = F::bload8(rz, zoff + unsigned(off + 32 * s) * 2u, 0u);
        };
        if (a) {
            f8 zr[kRankDecay / 32];
            zrow(kOffDecay, zr, kRankDecay / 32);
            f32x4_t y = preact(ua, zr);
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = decay_of(y[r]);
            store(a, t, y);
        }
        if (e) {
            f8 zr[kRankErase / 32];
            zrow(kOffErase, zr, kRankErase / 32);
            f32x4_t y = preact(ue, zr);
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = sigmoid_of(y[r]);
            store(e, t, y);
        }
        if (w) {
            f8 zr[kRankWrite / 32];
            zrow(kOffWrite, zr, kRankWrite / 32);
            f32x4_t y = preact(uw, zr);
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = sigmoid_of(y[r]);
            store(w, t, y);
        }
        if (g) {
            f8 zr[kRankRead / 32];
            zrow(kOffRead, zr, kRankRead / 32);
            f32x4_t y = preact(ug, zr);
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = sigmoid_of(y[r]);
            store(g, t, y);
        }
    }
}

template <int D>
hipError_t gates_typed(const void *z, const void *Ua, const void *Ue, const void *Uw,
                       const void *Ug, const float *ca, const float *ce, const float *cw,
                       const float *cg, float *a, float *e, float *w, float *g, int B, int T,
                       int H, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int nblk = (T + 15) / 16;
    // Enough wavefronts along the tokens to fill the machine about four times over, each
    // walking at least a few token blocks with its up-projection rows resident.
    const int tiles = H * (D / 16) * B;
    int groups = (4 * 256 * 4 + tiles * 4 - 1) / (tiles * 4);
    groups = max(1, min(groups, (nblk + 3) / 4));
    hipLaunchKernelGGL((lowrank_gates_kernel<D>), dim3(H * (D / 16), B, groups), dim3(256), 0,
                       stream, static_cast<const bf16_t *>(z), static_cast<const bf16_t *>(Ua),
                       static_cast<const bf16_t *>(Ue), static_cast<const bf16_t *>(Uw),
                       static_cast<const bf16_t *>(Ug), ca, ce, cw, cg, a, e, w, g, T, H,
                       groups * 4);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lowrank_gates(const void *z, const void *Ua, const void *Ue, const void *Uw,
                                const void *Ug, const float *ca, const float *ce, const float *cw,
                                const float *cg, float *a, float *e, float *w, float *g, int B,
                                int T, int H, int d, hipStream_t stream) {
    if (d == 64) return gates_typed<64>(z, Ua, Ue, Uw, Ug, ca, ce, cw, cg, a, e, w, g, B, T, H, stream);
    if (d == 128) return gates_typed<128>(z, Ua, Ue, Uw, Ug, ca, ce, cw, cg, a, e, w, g, B, T, H, stream);
    return hipErrorInvalidValue;
}

}  // namespace muir
