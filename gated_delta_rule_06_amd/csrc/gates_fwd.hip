// Gates of the recurrence from the fused low-rank gate projection.
//
// The pages fuse all five gates into one projection of total rank 512: one shared
// down-projection, then a separate up-projection per gate with its own rank, decay 64,
// erase 64, output 128, write 128 and dynamic read 128 (openai-hub news page, section on
// sensitivity-allocated gating, gate table; liuch.name summary, second bullet). The
// down-projection's output z [B, T, 512] (rank slices in the table's order) is the input;
// per gate n, with U_n [H, d, r_n] and an offset c_n [H, d]:
//   y_n = z[..., slice_n] U_n^T + c_n,   a = exp(-exp(y_decay)),   e, w, g, og = sigmoid(y)
// (y_decay is a log decay rate, so a lies in (0, 1]). The output gate og multiplies the
// readout; its slice feeds none of the recurrence's four gates.
//
// Each product is a 16-token x 16-channel tile with the rank as the contraction, on the
// matrix cores: the up-projection's rows (channels) are the A operand and z's rows
// (tokens) the B operand, so lane (t, G) of the accumulator holds token t and channels
// 4G .. 4G + 3 of the tile: one 16-byte store of four gate values per lane. The offset
// c_n is the accumulator's initial value.
#include "chunk_layout.hpp"
#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace muir {

namespace {

// Rank offsets of the gates' slices of z (their ranks: gate_rank below), in the order the
// kernel takes them: decay, erase, write, read, output.
constexpr int kZRank = 512;
constexpr int kOffDecay = 0, kOffErase = 64, kOffWrite = 256, kOffRead = 384, kOffOutput = 128;
constexpr int kGates = 5;

// LDS of the gate kernel: the head's up-projection rows of the requested gates (row pitch
// padded by 8 elements against bank conflicts) and their offsets; gate n's region starts at
// the byte offset the host computes (unrequested gates take no room).
constexpr int kPad = 8;
struct GateLds {
    int u_off[kGates];   // byte offsets of U_n rows, [D][r_n + kPad] bf16
    int c_off[kGates];   // byte offsets of c_n, [D] fp32
    int bytes;
};
__host__ __device__ constexpr int gate_rank(int n) { return n < 2 ? 64 : 128; }
__host__ __device__ constexpr int gate_zoff(int n) {
    return n == 0 ? kOffDecay : n == 1 ? kOffErase : n == 2 ? kOffWrite : n == 3 ? kOffRead : kOffOutput;
}

// PK: e and w are stored tile-packed for the split scan, [B*H][D/8][T][8] fp32 (eight value
// columns of one token contiguous, a tile's tokens consecutive), the other gates as [B, T, H, D].
// One workgroup of four wavefronts per (head, batch, token-block group). The head's
// up-projection rows sit in LDS, so each z row a wavefront loads serves every channel tile
// of the head: per token block, z's four slices are loaded once (the next block's while the
// current one computes), then for each 16-channel tile every requested gate is one short
// chain of K = 32 products. Gates whose output pointer is null are skipped.
template <int D, bool PK>
__global__ __launch_bounds__(256) void lowrank_gates_kernel(
    const bf16_t *__restrict__ z, const bf16_t *__restrict__ Ua, const bf16_t *__restrict__ Ue,
    const bf16_t *__restrict__ Uw, const bf16_t *__restrict__ Ug, const bf16_t *__restrict__ Uo,
    const float *__restrict__ ca, const float *__restrict__ ce, const float *__restrict__ cw,
    const float *__restrict__ cg, const float *__restrict__ co, float *__restrict__ a,
    float *__restrict__ e, float *__restrict__ w, float *__restrict__ g, float *__restrict__ og,
    int T, int H, GateLds lay) {
    using F = Frag<bf16_t>;
    using f8 = F::f8;
    constexpr int NCT = D / 16;
    extern __shared__ __align__(16) unsigned char smem[];
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int tid = threadIdx.x, lane = tid & 63, x = lane & 15, G = lane >> 4;
    const int h = blockIdx.x, b = blockIdx.y;
    const int tw = blockIdx.z * 4 + wave, nw = gridDim.z * 4;
    const int nblk = (T + 15) / 16;
    const bf16_t *U[kGates] = {Ua, Ue, Uw, Ug, Uo};
    const float *cc[kGates] = {ca, ce, cw, cg, co};
    float *out[kGates] = {a, e, w, g, og};

    // The head's rows of every requested gate into LDS.
#pragma unroll
    for (int n = 0; n < kGates; ++n) {
        if (!out[n]) continue;
        const int R = gate_rank(n), pitch = R + kPad, per_row = R / 8;
        bf16_t *su = reinterpret_cast<bf16_t *>(smem + lay.u_off[n]);
        for (int i = tid; i < D * per_row; i += 256) {
            const int row = i / per_row, c8 = i % per_row;
            *reinterpret_cast<f8 *>(su + row * pitch + 8 * c8) =
                F::load8(U[n] + (size_t(h) * D + row) * R + 8 * c8);
        }
        float *sc = reinterpret_cast<float *>(smem + lay.c_off[n]);
        for (int i = tid; i < D; i += 256) sc[i] = cc[n][size_t(h) * D + i];
    }
    lds_barrier();

    const rsrc_t rz = make_rsrc(z + size_t(b) * T * kZRank, unsigned(size_t(T) * kZRank * 2));
    const size_t HD = size_t(H) * D;
    const size_t gbase = size_t(b) * T * HD + size_t(h) * D;  // uniform
    const unsigned gbytes = unsigned((size_t(T) * HD - size_t(h) * D) * 4);
    const size_t pbase = (size_t(b) * H + h) * D * T;  // packed e, w of this head (PK)
    const unsigned pbytes = unsigned(size_t(D) * T * 4);

    struct ZRows {
        f8 r[16];  // decay 2, erase 2, write 4, read 4, output 4 K-steps
    };
    constexpr int kStep0[kGates] = {0, 2, 4, 8, 12};
    auto load_z = [&](int tb, ZRows &zr) {
        const unsigned t = unsigned(min(16 * tb + x, T));
        const unsigned zoff = t * unsigned(kZRank) * 2u + unsigned(8 * G) * 2u;
#pragma unroll
        for (int n = 0; n < kGates; ++n) {
            if (!out[n]) continue;
#pragma unroll
            for (int s = 0; s < gate_rank(n) / 32; ++s)
                zr.r[kStep0[n] + s] = F::bload8(rz, zoff + unsigned(gate_zoff(n) + 32 * s) * 2u, 0u);
        }
    };
    auto compute = [&](int tb, const ZRows &zr) {
        const unsigned t = unsigned(min(16 * tb + x, T));
#pragma unroll
        for (int n = 0; n < kGates; ++n) {
            if (!out[n]) continue;
            const int R = gate_rank(n), pitch = R + kPad;
            const bf16_t *su = reinterpret_cast<const bf16_t *>(smem + lay.u_off[n]);
            const float *sc = reinterpret_cast<const float *>(smem + lay.c_off[n]);
            const bool pk = PK && (n == 1 || n == 2);
            const rsrc_t ro = pk ? make_rsrc(out[n] + pbase, pbytes) : make_rsrc(out[n] + gbase, gbytes);
#pragma unroll 2
            for (int c = 0; c < NCT; ++c) {
                f32x4_t y = *reinterpret_cast<const f32x4_t *>(sc + 16 * c + 4 * G);
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    if (s < R / 32)
                        y = F::mma8(*reinterpret_cast<const f8 *>(su + (16 * c + x) * pitch + 32 * s + 8 * G),
                                    zr.r[kStep0[n] + s], y);
#pragma unroll
                for (int r = 0; r < 4; ++r) y[r] = n == 0 ? gate_decay(y[r]) : gate_sigmoid(y[r]);
                // Tokens past T (t == T here) are dropped: [B, T, H, D] offsets lie past the
                // buffer's end, packed ones are moved there.
                const unsigned off = pk ? (t < unsigned(T) ? ((unsigned(2 * c + (G >> 1)) * unsigned(T) + t) * 8u +
                                                              4u * unsigned(G & 1)) * 4u
                                                           : 0xfffffff0u)
                                        : (t * unsigned(HD) + unsigned(16 * c + 4 * G)) * 4u;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, y), ro, int(off), 0, 0);
            }
        }
    };
    // Two z buffers, alternate token blocks (two blocks per iteration keep register indices
    // static).
    ZRows z0, z1;
    if (tw < nblk) load_z(tw, z0);
    for (int tb = tw; tb < nblk; tb += 2 * nw) {
        const int tb1 = tb + nw;
        if (tb1 < nblk) load_z(tb1, z1);
        compute(tb, z0);
        if (tb1 < nblk) {
            if (tb1 + nw < nblk) load_z(tb1 + nw, z0);
            compute(tb1, z1);
        }
    }
}

template <int D>
hipError_t gates_typed(const void *z, const void *Ua, const void *Ue, const void *Uw,
                       const void *Ug, const void *Uo, const float *ca, const float *ce,
                       const float *cw, const float *cg, const float *co, float *a, float *e,
                       float *w, float *g, float *og, int B, int T, int H, bool packed_ew,
                       hipStream_t stream) {
    if (T == 0) return hipSuccess;
    GateLds lay{};
    const float *outs[kGates] = {a, e, w, g, og};
    int off = 0;
    for (int n = 0; n < kGates; ++n) {
        lay.u_off[n] = lay.c_off[n] = 0;
        if (!outs[n]) continue;
        lay.u_off[n] = off;
        off += D * (gate_rank(n) + kPad) * 2;
        lay.c_off[n] = off;
        off += D * 4;
    }
    lay.bytes = off;
    if (off == 0) return hipSuccess;
    auto kern = packed_ew ? lowrank_gates_kernel<D, true> : lowrank_gates_kernel<D, false>;
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, off);
    if (err != hipSuccess) return err;
    // Enough workgroups along the tokens to fill the machine, each walking several token
    // blocks so that loading the head's rows into LDS is amortised.
    const int nblk = (T + 15) / 16;
    int groups = (2 * 256 + H * B - 1) / (H * B);
    groups = max(1, min(groups, (nblk + 15) / 16));
    hipLaunchKernelGGL(kern, dim3(H, B, groups), dim3(256), off, stream,
                       static_cast<const bf16_t *>(z), static_cast<const bf16_t *>(Ua),
                       static_cast<const bf16_t *>(Ue), static_cast<const bf16_t *>(Uw),
                       static_cast<const bf16_t *>(Ug), static_cast<const bf16_t *>(Uo), ca, ce, cw,
                       cg, co, a, e, w, g, og, T, H, lay);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lowrank_gates(const void *z, const void *Ua, const void *Ue, const void *Uw,
                                const void *Ug, const void *Uo, const float *ca, const float *ce,
                                const float *cw, const float *cg, const float *co, float *a,
                                float *e, float *w, float *g, float *og, int B, int T, int H, int d,
                                hipStream_t stream, bool packed_ew) {
    if (d == 64)
        return gates_typed<64>(z, Ua, Ue, Uw, Ug, Uo, ca, ce, cw, cg, co, a, e, w, g, og, B, T, H,
                               packed_ew, stream);
    if (d == 128)
        return gates_typed<128>(z, Ua, Ue, Uw, Ug, Uo, ca, ce, cw, cg, co, a, e, w, g, og, B, T, H,
                                packed_ew, stream);
    return hipErrorInvalidValue;
}

}  // namespace muir
