// Contraction kernels of the forward convolution (implicit GEMM over the
// im2col view of an NHWC activation, weights [K x R*S*C]).
#include "ie_gemm_impl.h"

namespace ie {

hipError_t launch_gemm_im2col(const Operand &A, const Operand &B, int M, int N, int K, Tile t, int splits,
                              int k_chunk, bool partial, const Epi &ep, hipStream_t st) {
#define IE_CASE(a, b) IE_TILE_CASE(LD_IM2COL, LD_K, a, b)
    IE_TILES_CONV(IE_CASE)
#undef IE_CASE
    return hipErrorInvalidValue;
}

}  // namespace ie
