// Entry of the GEMM kernels: picks the kernel family for a validated request.
// The kernels themselves are in gemm_kernel.hpp; each family is compiled in
// its own translation unit.
#include "gemm_kernel.hpp"

namespace fp4q {

namespace {

// Dense FP4 products whose contraction is longer than one tile stages scale
// bytes for: chunks of kDenseKChunk contraction values (a multiple of 256),
// every chunk after the first adding into C.  The operand bases move k0/2
// bytes into each row and the scale grids k0/b blocks along K (for a 1D
// tiled grid, k0/128 chunks of 512 bytes); the operand rows, the grids'
// other dimension and C are unchanged.
hipError_t launch_gemm_chunked(const GemmArgs& g, bool a_st, bool b_st, int oned, int batch, bool accumulate,
                               hipStream_t s)
{
    for (int k0 = 0; k0 < g.K; k0 += kDenseKChunk) {
        GemmArgs c = g;
        c.K = min(kDenseKChunk, g.K - k0);
        c.a = g.a + k0 / 2;
        c.b = g.b + k0 / 2;
        c.sa = g.sa + (a_st ? (int64_t)(k0 >> g.sh_a) * g.lds_a : (int64_t)(k0 >> g.sh_a));
        if (oned & 2)
            c.sb = g.sb + (int64_t)(k0 / 128) * 512;
        else
            c.sb = g.sb + (b_st ? (int64_t)(k0 >> g.sh_b) * g.lds_b : (int64_t)(k0 >> g.sh_b));
        // chunks after the first start inside the planes: the K-checked
        // variant keeps their loads past the chunk from reaching beyond the
        // planes' end
        const bool kt = k0 > 0;
        hipError_t e;
        if (accumulate || k0 > 0)
            e = launch_gemm_acc(c, a_st, b_st, oned, batch, s, kt);
        else if (oned != 0)
            e = launch_gemm_1d(c, a_st, b_st, oned, batch, s, kt);
        else
            e = launch_gemm_plain(c, 1, a_st, b_st, batch, s, kt);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

} // namespace

hipError_t launch_gemm(const GemmArgs& g, int fmt, bool a_st, bool b_st, int oned, int grouped_op, int batch,
                       bool accumulate, bool out_bf16, hipStream_t s)
{
    if (fmt == 1 && grouped_op < 0 && !out_bf16 && (oned & 1) == 0 && g.K > kDenseKChunk)
        return launch_gemm_chunked(g, a_st, b_st, oned, batch, accumulate, s);
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
