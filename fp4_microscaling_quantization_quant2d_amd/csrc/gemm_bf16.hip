// bf16-output epilogue variants of the dense and batched products.
#include "gemm_kernel.hpp"

namespace fp4q {

// bf16 C for FP4 operands with square-block grids, and for MXFP8 S = Q K^T.
hipError_t launch_gemm_obf(const GemmArgs& g, int fmt, bool a_st, bool b_st, int batch, hipStream_t s)
{
    if (fmt == 2)
        return launch_dense<2, false, false, 0, false, true>(g, batch, s);
    if (!a_st && !b_st)
        return launch_dense<1, false, false, 0, false, true>(g, batch, s);
    if (!a_st && b_st)
        return launch_dense<1, false, true, 0, false, true>(g, batch, s);
    if (a_st && b_st)
        return launch_dense<1, true, true, 0, false, true>(g, batch, s);
    return launch_dense<1, true, false, 0, false, true>(g, batch, s);
}

} // namespace fp4q
