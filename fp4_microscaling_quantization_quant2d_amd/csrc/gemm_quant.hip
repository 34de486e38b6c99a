// Dense FP4 products whose epilogue quantizes the fp32 result into the 2D
// 32x32 FP4 planes of the next operand (row plane, transposed plane, scale
// grid) instead of writing it ("Stable FP4 Training via Transposition-
// Invariant Block Quantization", Sec. 3 "Application to linear layers": the
// output of one product is an operand of the next, quantized once).
#include "gemm_kernel.hpp"

namespace fp4q {

hipError_t launch_gemm_quant(const GemmArgs& g, bool a_st, bool b_st, hipStream_t s)
{
    const bool kt = g.K % 256 != 0;
    if (!a_st && !b_st)
        return kt ? launch_quant_k<false, false, true>(g, s) : launch_quant_k<false, false, false>(g, s);
    if (!a_st && b_st)
        return kt ? launch_quant_k<false, true, true>(g, s) : launch_quant_k<false, true, false>(g, s);
    if (a_st && b_st)
        return kt ? launch_quant_k<true, true, true>(g, s) : launch_quant_k<true, true, false>(g, s);
    return kt ? launch_quant_k<true, false, true>(g, s) : launch_quant_k<true, false, false>(g, s);
}

} // namespace fp4q
