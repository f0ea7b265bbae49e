// gemm_tile_nt.hip -- GEMM 1's 256x256 tile kernel (tile_gemm.h) with its
// weight DMA marked nontemporal, for batches where each expert holds about
// one row tile, so each weight panel is read once.  A translation unit of its
// own: built beside the plain GEMM 1 kernel in gemm_tile.hip, each spilled a
// register.
#include "tile_gemm.h"

namespace moe {

hipError_t launch_gemm1_swiglu_tile_nt(const void* x_perm, const void* w1, const void* w3,
                                       const int32_t* offsets, int R, int E, int d, int f, int kb,
                                       float* partials, void* h, hipStream_t stream) {
    return launch_tile<true, true>(x_perm, w1, w3, h, partials, offsets, R, E, d, f, kb, stream);
}

}  // namespace moe
