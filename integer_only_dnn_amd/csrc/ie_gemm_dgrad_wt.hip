// Contraction kernels of the convolution input gradient that read a
// whole-tensor-exponent weight in its stored layout (no transposed copy).
#include "ie_gemm_impl.h"

namespace ie {

hipError_t launch_gemm_dgrad_wt(const Operand &A, const Operand &B, int M, int N, int K, Tile t, int splits,
                                int k_chunk, bool partial, const Epi &ep, hipStream_t st) {
#define IE_CASE(a, b) IE_TILE_CASE(LD_DGRAD, LD_WT, a, b)
    IE_TILES_CONV(IE_CASE)
#undef IE_CASE
    return hipErrorInvalidValue;
}

}  // namespace ie
