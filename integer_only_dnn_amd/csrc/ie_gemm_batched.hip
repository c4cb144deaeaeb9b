// Batched products over stacks of slices: A . B^T (both K-contiguous), A . B
// (B row-contiguous) and A^T . B (both row-contiguous): a ViT's attention
// products per (image, head).
#include "ie_gemm_impl.h"

namespace ie {

#define IE_BATCHED_CASE(KA, KB, MI_, NI_) \
    if (t.mi == MI_ && t.ni == NI_) return launch_batched_one<KA, KB, MI_, NI_>(A, B, M, N, K, ep, ba, st);

hipError_t launch_gemm_batched(const Operand &A, const Operand &B, int M, int N, int K, Tile t, const Epi &ep,
                               const BatchArgs &ba, hipStream_t st) {
    if (M <= 0 || N <= 0 || ba.Z <= 0) return hipSuccess;
    if (ep.mode != EPI_DIRECT && ep.mode != EPI_RTO) return hipErrorInvalidValue;
    if (!ep.row_group) return hipErrorInvalidValue;  // one exponent per row of every slice
    if (ep.mode == EPI_DIRECT && N > t.bn()) return hipErrorInvalidValue;
    if (A.kind == LD_K && B.kind == LD_K) {
        // one contraction step (attention scores at head size 64)
        if (K <= BK && t.mi == 1 && t.ni == 4) return launch_batched_one<LD_K, LD_K, 1, 4, true>(A, B, M, N, K, ep, ba, st);
        IE_BATCHED_CASE(LD_K, LD_K, 2, 2)
        IE_BATCHED_CASE(LD_K, LD_K, 1, 4)
        IE_BATCHED_CASE(LD_K, LD_K, 2, 1)
        IE_BATCHED_CASE(LD_K, LD_K, 1, 1)
    } else if (A.kind == LD_K && B.kind == LD_T) {
        IE_BATCHED_CASE(LD_K, LD_T, 2, 2)
        IE_BATCHED_CASE(LD_K, LD_T, 2, 1)
        IE_BATCHED_CASE(LD_K, LD_T, 1, 1)
    } else if (A.kind == LD_T && B.kind == LD_T) {
        IE_BATCHED_CASE(LD_T, LD_T, 2, 2)
        IE_BATCHED_CASE(LD_T, LD_T, 2, 1)
        IE_BATCHED_CASE(LD_T, LD_T, 1, 1)
    }
    return hipErrorInvalidValue;
}

}  // namespace ie
