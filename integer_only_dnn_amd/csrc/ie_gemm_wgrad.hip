// Contraction kernels of weight gradients: both operands are contiguous
// along the output dimension and contracted over the batch (linear: dY^T . X;
// convolution: dY^T . im2col(X)).  Always split over the contraction, with
// exact int32 partial sums.
#include "ie_gemm_impl.h"

namespace ie {

#define IE_WG_CASE(KB, MI_, NI_) \
    if (t.mi == MI_ && t.ni == NI_) return launch_one<LD_T, KB, MI_, NI_, true>(A, B, M, N, K, splits, k_chunk, ep, st);

hipError_t launch_gemm_wgrad(const Operand &A, const Operand &B, int M, int N, int K, Tile t, int splits,
                             int k_chunk, bool partial, const Epi &ep, hipStream_t st) {
    if (!partial) return hipErrorInvalidValue;
#define IE_CASE_T(a, b) IE_WG_CASE(LD_T, a, b)
#define IE_CASE_I(a, b) IE_WG_CASE(LD_IM2COL_T, a, b)
    if (B.kind == LD_T) {
        IE_TILES_WGRAD(IE_CASE_T)
    } else {
        IE_TILES_WGRAD(IE_CASE_I)
    }
#undef IE_CASE_T
#undef IE_CASE_I
    return hipErrorInvalidValue;
}

}  // namespace ie
