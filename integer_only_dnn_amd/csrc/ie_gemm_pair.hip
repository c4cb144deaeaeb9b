// The input gradient (round-to-odd product) and the weight gradient (split
// contraction) of a convolution in one launch: the grid holds both products'
// workgroups, so they run side by side without a second stream and the
// events that would join it.  The input gradient reads the weight in place
// (whole-tensor exponent, LD_WT) or its aligned transposed copy (per-channel
// exponents, LD_K; that form's kernels are built in ie_gemm_pair_al.hip).
#include "ie_gemm_impl.h"

namespace ie {

hipError_t launch_gemm_pair_al(const PairPart &p1, Tile t1, const PairPart &p2, Tile t2, hipStream_t st);

bool gemm_pair_supported(const Operand &A1, const Operand &B1, Tile t1, const Operand &A2, const Operand &B2,
                         Tile t2) {
    if (A1.kind != LD_DGRAD || (B1.kind != LD_WT && B1.kind != LD_K) || A2.kind != LD_T ||
        B2.kind != LD_IM2COL_T)
        return false;
    return pair_tiles_built(t1, t2);
}

hipError_t launch_gemm_pair(const Operand &A1, const Operand &B1, int M1, int N1, int K1, Tile t1, int k_chunk1,
                            const Epi &ep1, const Operand &A2, const Operand &B2, int M2, int N2, int K2, Tile t2,
                            int splits2, int k_chunk2, const Epi &ep2, hipStream_t st) {
    if (!gemm_pair_supported(A1, B1, t1, A2, B2, t2) || M1 <= 0 || N1 <= 0 || M2 <= 0 || N2 <= 0)
        return hipErrorInvalidValue;
    const PairPart p1 = pair_part(A1, B1, M1, N1, K1, t1.mi, t1.ni, 1, k_chunk1, ep1);
    const PairPart p2 = pair_part(A2, B2, M2, N2, K2, t2.mi, t2.ni, splits2, k_chunk2, ep2);
    if (B1.kind == LD_K) return launch_gemm_pair_al(p1, t1, p2, t2, st);
#define IE_PAIR_CASE(a, b, c, d)                                       \
    if (t1.mi == a && t1.ni == b && t2.mi == c && t2.ni == d)          \
        return launch_pair<LD_DGRAD, LD_WT, a, b, LD_T, LD_IM2COL_T, c, d>(p1, p2, st);
    IE_TILES_PAIR(IE_PAIR_CASE)
#undef IE_PAIR_CASE
    return hipErrorInvalidValue;
}

}  // namespace ie
