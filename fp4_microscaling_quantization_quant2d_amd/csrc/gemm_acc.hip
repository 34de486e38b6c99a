// Accumulating epilogue variants (C += A B^T) of the dense products.
#include "gemm_kernel.hpp"

namespace fp4q {

// C += A B^T for FP4 operands with 32x32 or 64x64 blocks, or a 1D-layout B
// (the weight gradient of a 1D activation).
hipError_t launch_gemm_acc(const GemmArgs& g, bool a_st, bool b_st, int oned, int batch, hipStream_t s, bool force_kt)
{
    if (oned == 2)
        return a_st ? launch_dense<1, true, false, 2, true>(g, batch, s, force_kt)
                    : launch_dense<1, false, false, 2, true>(g, batch, s, force_kt);
    if (!a_st && !b_st)
        return launch_dense<1, false, false, 0, true>(g, batch, s, force_kt);
    if (!a_st && b_st)
        return launch_dense<1, false, true, 0, true>(g, batch, s, force_kt);
    if (a_st && b_st)
        return launch_dense<1, true, true, 0, true>(g, batch, s, force_kt);
    return launch_dense<1, true, false, 0, true>(g, batch, s, force_kt);
}

} // namespace fp4q
