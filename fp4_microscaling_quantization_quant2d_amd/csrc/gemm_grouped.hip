// Grouped (expert) products, host or device group offsets, fp32 or bf16 C.
#include "gemm_kernel.hpp"

namespace fp4q {

hipError_t launch_gemm_grouped(const GemmArgs& g, int op, bool out_bf16, hipStream_t s)
{
    const bool dev = g.row_off_dev != nullptr;
    if (out_bf16) {
        if (op == kGemmFwd)
            return dev ? launch_grouped<kGemmFwd, false, false, true, true>(g, s)
                       : launch_grouped<kGemmFwd, false, false, false, true>(g, s);
        if (op == kGemmDgrad)
            return dev ? launch_grouped<kGemmDgrad, false, true, true, true>(g, s)
                       : launch_grouped<kGemmDgrad, false, true, false, true>(g, s);
        return dev ? launch_grouped<kGemmWgrad, true, true, true, true>(g, s)
                   : launch_grouped<kGemmWgrad, true, true, false, true>(g, s);
    }
    if (op == kGemmFwd)
        return dev ? launch_grouped<kGemmFwd, false, false, true>(g, s) : launch_grouped<kGemmFwd, false, false, false>(g, s);
    if (op == kGemmDgrad)
        return dev ? launch_grouped<kGemmDgrad, false, true, true>(g, s)
                   : launch_grouped<kGemmDgrad, false, true, false>(g, s);
    return dev ? launch_grouped<kGemmWgrad, true, true, true>(g, s) : launch_grouped<kGemmWgrad, true, true, false>(g, s);
}

} // namespace fp4q
