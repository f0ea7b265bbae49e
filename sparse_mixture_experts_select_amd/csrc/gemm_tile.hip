// gemm_tile.hip -- launchers of the 256x256 tile GEMMs (tile_gemm.h): GEMM 1
// with its weight DMA not marked (several row tiles of an expert share each
// weight panel through L2), GEMM 2 with it marked nontemporal, and the size of
// GEMM 2's partial-sum buffer.  GEMM 1 with nontemporal weight DMA is built in
// gemm_tile_nt.hip: with both GEMM 1 kernels in one translation unit, each
// spilled a register.
#include "tile_gemm.h"

namespace moe {

size_t tile_partials_bytes(int R, int E, int d, int f) {
    // Only GEMM 2 (K = f, N = d, 256-column tiles) cuts tiles.  Per XCD at
    // most its share of the tiles, each cut into at most
    // min(kMaxPieces, K steps / 8) pieces, and at most 2 cpx pieces in all
    // (the schedule's limits); with fewer than 2 pieces possible nothing is
    // cut and only the header is needed.
    const long long mtiles = (R + kBM - 1) / kBM + E;
    const long long nt2 = (d + 255) / 256;
    const long long per_xcd = (mtiles * nt2 + 7) / 8;
    long long pmax = (f / kBK) / 8;
    if (pmax > kMaxPieces) pmax = kMaxPieces;
    long long slots = 0;
    if (pmax >= 2) {
        long long per = per_xcd * pmax;
        if (per > 2 * kMaxCpx) per = 2 * kMaxCpx;
        slots = 8 * per;
    }
    return ((size_t)slots * kSlotFloats + kHeaderFloats) * sizeof(float);
}

hipError_t launch_gemm1_swiglu_tile(const void* x_perm, const void* w1, const void* w3,
                                    const int32_t* offsets, int R, int E, int d, int f, int kb,
                                    float* partials, bool nt_weights, void* h,
                                    hipStream_t stream) {
    if (nt_weights)
        return launch_gemm1_swiglu_tile_nt(x_perm, w1, w3, offsets, R, E, d, f, kb, partials, h,
                                           stream);
    return launch_tile<true, false>(x_perm, w1, w3, h, partials, offsets, R, E, d, f, kb, stream);
}

hipError_t launch_gemm2_tile(const void* h, const void* w2, const int32_t* offsets, int R, int E,
                             int f, int d, int kb, float* partials, float* y, hipStream_t stream) {
    return launch_tile<false, true>(h, w2, nullptr, y, partials, offsets, R, E, f, d, kb, stream);
}

}  // namespace moe
