// Contraction kernels over K-contiguous dense operands: the linear layer's
// forward product (X . W^T) and input gradient (dY . W, with W pre-transposed).
#include "ie_gemm_impl.h"

namespace ie {

hipError_t launch_gemm_kk(const Operand &A, const Operand &B, int M, int N, int K, Tile t, int splits,
                          int k_chunk, bool partial, const Epi &ep, hipStream_t st) {
#define IE_CASE(a, b) IE_TILE_CASE(LD_K, LD_K, a, b)
    IE_TILES_DENSE(IE_CASE)
#undef IE_CASE
    return hipErrorInvalidValue;
}

}  // namespace ie
