// Dense products with operands in the 1D activation layout.
#include "gemm_kernel.hpp"

namespace fp4q {

// 1D-layout operands (FP4, dense): the grid orientation of such an operand
// does not apply.
hipError_t launch_gemm_1d(const GemmArgs& g, bool a_st, bool b_st, int oned, int batch, hipStream_t s, bool force_kt)
{
    if (oned == 3)
        return launch_dense<1, false, false, 3>(g, batch, s, force_kt);
    if (oned == 1)
        return b_st ? launch_dense<1, false, true, 1>(g, batch, s, force_kt)
                    : launch_dense<1, false, false, 1>(g, batch, s, force_kt);
    return a_st ? launch_dense<1, true, false, 2>(g, batch, s, force_kt)
                : launch_dense<1, false, false, 2>(g, batch, s, force_kt);
}

} // namespace fp4q
