// Dense and batched products C = A B^T (FWD, DGRAD, WGRAD orientations of the
// scale grids; MXFP8 S = Q K^T): the kernels of the benchmarked step.
#include "gemm_kernel.hpp"

namespace fp4q {

hipError_t launch_gemm_plain(const GemmArgs& g, int fmt, bool a_st, bool b_st, int batch, hipStream_t s, bool force_kt)
{
    if (fmt == 2)
        return launch_dense<2, false, false>(g, batch, s);
    if (!a_st && !b_st)
        return launch_dense<1, false, false>(g, batch, s, force_kt);
    if (!a_st && b_st)
        return launch_dense<1, false, true>(g, batch, s, force_kt);
    if (a_st && b_st)
        return launch_dense<1, true, true>(g, batch, s, force_kt);
    return launch_dense<1, true, false>(g, batch, s, force_kt);
}

} // namespace fp4q
