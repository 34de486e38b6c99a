// 2D-block FP4 quantizer for gfx950.
//
// "Stable FP4 Training via Transposition-Invariant Block Quantization":
//   Sec. 3    square 32x32 blocks share one scale, S(B) = S(B^T)
//   Sec. 3.1  truncation-free S = 2^ceil(log2(2M/(Qp-Qn))), stochastic rounding
//   Sec. 2.1  P = round_FP4(X/S)
//   appendix  "Boundary blocks": the amax covers valid entries only
//
// Work decomposition (bandwidth-bound kernel, one read of x):
//   workgroup = 256 threads = 4 waves, covering a 128x128 region (2x2 waves);
//   wave      = 64x64 region = 2x2 tiles of 32x32;
//   lane      = one 8x8 block: lane = bc + 8*br, rows 8br.., cols 8bc..
// A lane loads its block with 16-byte loads (a wave's load instruction reads
// 8 rows x 128 contiguous bytes), reduces |x| to a tile amax over the 16
// lanes of its tile with cross-lane xor shuffles, derives the E8M0 byte,
// draws 8 Philox blocks, rounds its 64 elements and packs them into 8 row
// words; an in-register nibble transpose gives the 8 column words of the
// transposed plane, so both planes and the scale grid come from one read.
//
// Random bits: element (r, c) uses the Philox block keyed by the unordered
// pair (a, b) = (min, max) and its 16-bit half b%8.  For a block strictly
// above the diagonal (block row < block col) the 8 elements of one row share
// a Philox block; below the diagonal the 8 elements of one column do; on a
// diagonal block element (i, j) uses block min(i, j), half max(i, j).  Waves
// entirely above or below the diagonal take a uniform branch; only waves on
// the diagonal select per lane.
#include "fp4q_device.hpp"
#include "fp4q_launch.hpp"

namespace fp4q {

namespace {

constexpr int kThreads = 256;
constexpr int kRegion = 128;

template <bool F32>
struct Block8x8;

// bf16: 8 rows x 4 dwords, dword d of row i holds columns 2d (low) and 2d+1.
template <>
struct Block8x8<false> {
    uint32_t v[8][4];
    __device__ __forceinline__ uint32_t x32(int i, int j) const
    {
        const uint32_t d = v[i][j >> 1];
        return (j & 1) ? (d & 0xFFFF0000u) : (d << 16);
    }
};

// fp32: 8 rows x 8 words.
template <>
struct Block8x8<true> {
    uint32_t v[8][8];
    __device__ __forceinline__ uint32_t x32(int i, int j) const { return v[i][j]; }
};

template <bool F32, bool ALIGNED>
__device__ __forceinline__ void load_block(Block8x8<F32>& blk, const Quant2dArgs& p, int R0, int C0)
{
    const int esz = F32 ? 4 : 2;
    const char* base = static_cast<const char*>(p.x);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = R0 + i;
        const char* row = base + ((int64_t)r * p.ldx) * esz;
        if (r < p.rows && ALIGNED && C0 + 8 <= p.cols) {
            if (F32) {
                const uint4 a = *reinterpret_cast<const uint4*>(row + (int64_t)C0 * 4);
                const uint4 b = *reinterpret_cast<const uint4*>(row + (int64_t)C0 * 4 + 16);
                uint32_t* dst = &blk.v[i][0];
                dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
                dst[4] = b.x; dst[5] = b.y; dst[6] = b.z; dst[7] = b.w;
            } else {
                const uint4 a = *reinterpret_cast<const uint4*>(row + (int64_t)C0 * 2);
                uint32_t* dst = &blk.v[i][0];
                dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = C0 + j;
                uint32_t val = 0;
                if (r < p.rows && c < p.cols) {
                    if (F32)
                        val = reinterpret_cast<const uint32_t*>(row)[c];
                    else
                        val = reinterpret_cast<const uint16_t*>(row)[c];
                }
                if (F32) {
                    blk.v[i][j] = val;
                } else {
                    uint32_t* dst = &blk.v[i][0];
                    if (j & 1)
                        dst[j >> 1] |= val << 16;
                    else
                        dst[j >> 1] = val;
                }
            }
        }
    }
}

template <bool F32, int RNE, bool EXACT_SUB>
__device__ __forceinline__ void round_block(const Block8x8<F32>& blk, const uint32_t rnd[8][4],
                                            int c133k, int c127k, uint32_t rw[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t rd = rnd[i][j >> 1];
            const uint32_t r16 = (j & 1) ? (rd >> 16) : (rd & 0xFFFFu);
            w |= e2m1_nibble<RNE, EXACT_SUB>(blk.x32(i, j), r16, c133k, c127k) << (4 * j);
        }
        rw[i] = w;
    }
}

template <bool F32, int RNE, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void quant2d_kernel(Quant2dArgs p)
{
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int nbx = (p.cols_pad + kRegion - 1) / kRegion;
    const int by = blockIdx.x / nbx;
    const int bx = blockIdx.x - by * nbx;
    const int r0w = by * kRegion + (wave >> 1) * 64;
    const int c0w = bx * kRegion + (wave & 1) * 64;
    const int br = lane >> 3, bc = lane & 7;
    const int R0 = r0w + 8 * br;
    const int C0 = c0w + 8 * bc;
    const bool active = R0 < p.rows_pad && C0 < p.cols_pad;

    Block8x8<F32> blk;
    uint32_t mx = 0;
    if (active) {
        load_block<F32, ALIGNED>(blk, p, R0, C0);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                mx = max(mx, blk.x32(i, j) & 0x7FFFFFFFu);
    }
    // Tile amax: the 16 lanes of a 32x32 tile differ in lane bits 0,1,3,4.
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 1));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 2));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 8));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16));
    if (!active)
        return;

    const int k = truncfree_exp_e2m1(mx);

    // Philox blocks: canonical orientation (P0, Q0) with P0 <= Q0 in block units.
    const int BR = R0 >> 3, BC = C0 >> 3;
    const int P0 = BR <= BC ? R0 : C0;
    const int Q0 = BR <= BC ? C0 : R0;
    uint32_t w[8][4];
    if (RNE == 0) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            U4 c;
            c.x = (uint32_t)(((P0 & 31) + t) * 4 + ((Q0 & 31) >> 3));
            c.y = (uint32_t)(P0 >> 5);
            c.z = (uint32_t)(Q0 >> 5);
            c.w = p.stream;
            const U4 o = philox10(c, p.key0, p.key1);
            w[t][0] = o.x; w[t][1] = o.y; w[t][2] = o.z; w[t][3] = o.w;
        }
        const int WR = r0w >> 6, WC = c0w >> 6;
        if (WR > WC) {
            uint32_t t2[8][4];
            half_transpose8(w, t2);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    w[i][d] = t2[i][d];
        } else if (WR == WC) {
            uint32_t t2[8][4];
            half_transpose8(w, t2);
            const bool lower = BR > BC, diag = BR == BC;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    // diagonal block: (i, j) takes row-block min(i,j), half max(i,j)
                    uint32_t dv;
                    if (i <= 2 * d)
                        dv = w[i][d];
                    else if (i >= 2 * d + 2)
                        dv = t2[i][d];
                    else // i == 2d+1: j = 2d from the transpose, j = 2d+1 = i from w
                        dv = perm_b32(w[i][d], t2[i][d], 0x07060100u);
                    w[i][d] = lower ? t2[i][d] : (diag ? dv : w[i][d]);
                }
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int d = 0; d < 4; ++d)
                w[t][d] = 0;
    }

    uint32_t rw[8];
    const int c133k = 133 + k, c127k = 127 + k;
    if (k >= -109)
        round_block<F32, RNE, false>(blk, w, c133k, c127k, rw);
    else
        round_block<F32, RNE, true>(blk, w, c133k, c127k, rw);

#pragma unroll
    for (int i = 0; i < 8; ++i)
        *reinterpret_cast<uint32_t*>(p.codes + (int64_t)(R0 + i) * p.ld + (C0 >> 1)) = rw[i];
    if (p.codes_t) {
        nibble_transpose8(rw);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *reinterpret_cast<uint32_t*>(p.codes_t + (int64_t)(C0 + j) * p.ld_t + (R0 >> 1)) = rw[j];
    }
    if (((br | bc) & 3) == 0)
        p.scales[(int64_t)(R0 >> 5) * p.ld_s + (C0 >> 5)] = (uint8_t)(k + 127);
}

template <bool F32, int RNE, bool ALIGNED>
hipError_t launch_t(const Quant2dArgs& p, hipStream_t s)
{
    const int nbx = (p.cols_pad + kRegion - 1) / kRegion;
    const int nby = (p.rows_pad + kRegion - 1) / kRegion;
    hipLaunchKernelGGL((quant2d_kernel<F32, RNE, ALIGNED>), dim3(nbx * nby), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <bool F32, int RNE>
hipError_t launch_a(const Quant2dArgs& p, bool aligned, hipStream_t s)
{
    return aligned ? launch_t<F32, RNE, true>(p, s) : launch_t<F32, RNE, false>(p, s);
}

} // namespace

hipError_t launch_quant2d(const Quant2dArgs& p, bool f32, bool rne, bool aligned, hipStream_t s)
{
    if (f32)
        return rne ? launch_a<true, 1>(p, aligned, s) : launch_a<true, 0>(p, aligned, s);
    return rne ? launch_a<false, 1>(p, aligned, s) : launch_a<false, 0>(p, aligned, s);
}

} // namespace fp4q
