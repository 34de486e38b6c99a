// Entry of the GEMM kernels: picks the kernel family for a validated request.
// The kernels themselves are in gemm_kernel.hpp; each family is compiled in
// its own translation unit.
#include "gemm_kernel.hpp"

namespace fp4q {

hipError_t launch_gemm(const GemmArgs& g, int fmt, bool a_st, bool b_st, int oned, int grouped_op, int batch,
                       bool accumulate, bool out_bf16, hipStream_t s)
{
    if (grouped_op >= 0)
        return launch_gemm_grouped(g, grouped_op, out_bf16, s);
    if (out_bf16)
        return launch_gemm_obf(g, fmt, a_st, b_st, batch, s);
    if (accumulate)
        return launch_gemm_acc(g, a_st, b_st, oned, batch, s);
    if (fmt == 1 && oned != 0)
        return launch_gemm_1d(g, a_st, b_st, oned, batch, s);
    return launch_gemm_plain(g, fmt, a_st, b_st, batch, s);
}

hipError_t launch_gemm_subblock(const GemmArgs& g, int block, bool a_st, bool b_st, bool accumulate, hipStream_t s)
{
    return block == 16 ? launch_gemm_sub16(g, a_st, b_st, accumulate, s) : launch_gemm_sub8(g, a_st, b_st, accumulate, s);
}

int gemm_tile_m() { return kBM; }
int gemm_tile_n() { return kBN; }
size_t gemm_lds_bytes(int fmt, int K) { return lds_bytes(fmt, K, 0); }

} // namespace fp4q
