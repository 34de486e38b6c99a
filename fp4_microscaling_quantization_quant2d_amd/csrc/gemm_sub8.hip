// Dense products of FP4 operands in 8x8 scale blocks (one of the block
// sides compared in Table 4 of "Stable FP4 Training via Transposition-
// Invariant Block Quantization"): each 32-K MFMA split into 4 MFMAs, one per
// 8-wide sub-block, with that sub-block's scales.
#include "gemm_kernel.hpp"

namespace fp4q {

hipError_t launch_gemm_sub8(const GemmArgs& g, bool a_st, bool b_st, bool accumulate, hipStream_t s)
{
    return launch_sub_any<4>(g, a_st, b_st, accumulate, s);
}

} // namespace fp4q
