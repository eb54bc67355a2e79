// The 16-token leaf of the sequential scan, shared by the scan kernels: the per-leaf inputs
// of the serial chain and one step of the leaf's forward substitution.
#pragma once

#include "chunk_layout.hpp"

namespace muir {

// One step of the leaf's forward substitution for the VC value columns a lane holds (4 or
// 2): x_c += n_c * x_c(lane S of the 16-lane row), the broadcast done by the DPP row
// broadcast inside the FMA. A DPP read needs two wait states after a VALU write of its
// register. With four columns the other columns' instructions provide them (every
// register is read three instructions after it was written) and only the first step
// waits; with two columns one more state is waited each step.
template <int S, int VC>
__device__ __forceinline__ void subst_step(float &x0, float &x1, float &x2, float &x3, float n0,
                                           float n1, float n2, float n3) {
#define MUIR_BCAST_FMA(R, N) \
    "v_fmac_f32_dpp " R ", " R ", " N " row_newbcast:%8 row_mask:0xf bank_mask:0xf\n\t"
    if constexpr (VC == 4) {
        if constexpr (S == 0) {
            asm("s_nop 1\n\t" MUIR_BCAST_FMA("%0", "%4") MUIR_BCAST_FMA("%1", "%5")
                    MUIR_BCAST_FMA("%2", "%6") MUIR_BCAST_FMA("%3", "%7")
                : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3)
                : "v"(n0), "v"(n1), "v"(n2), "v"(n3), "i"(S));
        } else {
            asm(MUIR_BCAST_FMA("%0", "%4") MUIR_BCAST_FMA("%1", "%5") MUIR_BCAST_FMA("%2", "%6")
                    MUIR_BCAST_FMA("%3", "%7")
                : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3)
                : "v"(n0), "v"(n1), "v"(n2), "v"(n3), "i"(S));
        }
    } else {
        static_assert(VC == 2, "VC is 4 or 2");
        asm("s_nop %5\n\t"
            "v_fmac_f32_dpp %0, %0, %2 row_newbcast:%4 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %1, %1, %3 row_newbcast:%4 row_mask:0xf bank_mask:0xf"
            : "+v"(x0), "+v"(x1)
            : "v"(n0), "v"(n1), "i"(S), "i"(S == 0 ? 1 : 0));
    }
#undef MUIR_BCAST_FMA
}

// Per-leaf inputs of the serial chain, row layout: lane (t, g) holds token t of the
// leaf and the tile's value columns of lane group g (the first VC values).
template <typename QT, int VC> struct LeafIn {
    f32x4_t ev, wv;
    typename RowV<QT, VC>::raw vv;
};

}  // namespace muir
