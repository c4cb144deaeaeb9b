// Contraction kernels of the convolution input gradient (gather of the
// output gradient through the stride, weights pre-transposed to [C x R*S*K]).
#include "ie_gemm_impl.h"

namespace ie {

hipError_t launch_gemm_dgrad(const Operand &A, const Operand &B, int M, int N, int K, Tile t, int splits,
                             int k_chunk, bool partial, const Epi &ep, hipStream_t st) {
    if (B.kind == LD_WT) return launch_gemm_dgrad_wt(A, B, M, N, K, t, splits, k_chunk, partial, ep, st);
#define IE_CASE(a, b) IE_TILE_CASE(LD_DGRAD, LD_K, a, b)
    IE_TILES_CONV(IE_CASE)
#undef IE_CASE
    return hipErrorInvalidValue;
}

}  // namespace ie
