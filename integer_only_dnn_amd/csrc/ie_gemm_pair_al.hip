// Paired convolution backward (see ie_gemm_pair.hip) whose input gradient
// reads the aligned, transposed copy of a weight with per-channel exponents.
#include "ie_gemm_impl.h"

namespace ie {

hipError_t launch_gemm_pair_al(const PairPart &p1, Tile t1, const PairPart &p2, Tile t2, hipStream_t st) {
#define IE_PAIR_CASE(a, b, c, d)                                       \
    if (t1.mi == a && t1.ni == b && t2.mi == c && t2.ni == d)          \
        return launch_pair<LD_DGRAD, LD_K, a, b, LD_T, LD_IM2COL_T, c, d>(p1, p2, st);
    IE_TILES_PAIR(IE_PAIR_CASE)
#undef IE_PAIR_CASE
    return hipErrorInvalidValue;
}

}  // namespace ie
