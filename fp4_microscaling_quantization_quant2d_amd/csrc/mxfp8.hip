// MXFP8 quantizer for the query/key projections ("Stable FP4 Training via
// Transposition-Invariant Block Quantization", Sec. 3.2): E4M3FN elements,
// one E8M0 scale per 1x32 group along each row, truncation-free (the Sec. 3.1
// rule with Qp = 448, Qn = -448), round-to-nearest-even.
//
// A 1x32 group is spread over consecutive lanes that each read 16 contiguous
// bytes (4 lanes of 8 bf16 values, or 8 lanes of 4 fp32 values), so every
// load instruction of a wave reads 1 KB of whole cache lines.  The group
// amax is a max over those lanes (DPP and ds_swizzle exchanges).  Each lane
// converts its own values on the gfx950 FP8 converters (two values per
// instruction, the block scale as their divisor) and writes their code
// bytes; the group's first lane writes the scale byte.
#include "fp4q_cvt.hpp"
#include "fp4q_device.hpp"
#include "fp4q_launch.hpp"
#include "lane_ops.hpp"

namespace fp4q {

namespace {

constexpr int kThreads = 256;

// E4M3FN (OCP FP8) conversions: v_cvt_scalef32_pk_fp8_{bf16,f32} divide two
// values by the float scale, round them to nearest (ties to even) and write
// the two code bytes (first value in the low byte) into word HI of the
// destination, keeping the other word, which the wrappers tie.  The
// quantizer only converts values whose magnitude after scaling is at most
// 448, so saturation never applies.  Checked on MI355X against the oracle's
// round-to-nearest-even for every finite bf16 pattern at every block exponent.

// Word HI of acc <- E4M3 codes of the two bf16 halves of d (low half -> low byte).
template <int HI>
__device__ __forceinline__ void cvt8_rne_bf16_word(uint32_t& acc, uint32_t d, float scale)
{
    if constexpr (HI == 0)
        asm("v_cvt_scalef32_pk_fp8_bf16 %0, %1, %2" : "+v"(acc) : "v"(d), "v"(scale));
    else
        asm("v_cvt_scalef32_pk_fp8_bf16 %0, %1, %2 op_sel:[0,0,1]" : "+v"(acc) : "v"(d), "v"(scale));
}

// Word HI of acc <- E4M3 codes of x0 (low byte) and x1 (high byte).
template <int HI>
__device__ __forceinline__ void cvt8_rne_f32_word(uint32_t& acc, float x0, float x1, float scale)
{
    if constexpr (HI == 0)
        asm("v_cvt_scalef32_pk_fp8_f32 %0, %1, %2, %3" : "+v"(acc) : "v"(x0), "v"(x1), "v"(scale));
    else
        asm("v_cvt_scalef32_pk_fp8_f32 %0, %1, %2, %3 op_sel:[0,0,0,1]"
            : "+v"(acc) : "v"(x0), "v"(x1), "v"(scale));
}

// Lanes per 1x32 group: 16 bytes of input each.
template <bool F32>
constexpr int lanes_per_group() { return F32 ? 8 : 4; }

template <bool F32, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void mxfp8_kernel(Mxfp8Args p)
{
    constexpr int LPG = lanes_per_group<F32>();
    constexpr int esz = F32 ? 4 : 2;
    const uint32_t groups = (uint32_t)(p.cols_pad >> 5);
    // fewer than 2^32 work-items per launch (checked by the caller)
    const uint32_t t = blockIdx.x * (uint32_t)kThreads + threadIdx.x;
    const uint32_t gid = t / LPG;
    const int sub = (int)(t % LPG);
    const bool live = (int64_t)gid < p.rows * groups;
    const uint32_t r = live ? gid / groups : 0u;
    const int g = live ? (int)(gid - r * groups) : 0;
    const int c0 = g * 32 + sub * (32 / LPG);

    // the lane's 16 input bytes: 8 bf16 (two per word) or 4 fp32
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (live) {
        const char* row = static_cast<const char*>(p.x) + (int64_t)r * p.ldx * esz;
        if (ALIGNED && c0 + 32 / LPG <= p.cols) {
            const uint4 v = *reinterpret_cast<const uint4*>(row + (int64_t)c0 * esz);
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else {
#pragma unroll
            for (int j = 0; j < 32 / LPG; ++j) {
                const int c = c0 + j;
                if (c >= p.cols)
                    continue;
                if (F32)
                    w[j] = reinterpret_cast<const uint32_t*>(row)[c];
                else
                    w[j >> 1] |= (uint32_t)reinterpret_cast<const uint16_t*>(row)[c] << (16 * (j & 1));
            }
        }
    }
    // |x| as fp32 bits (bf16: the high half of the fp32 pattern)
    uint32_t mx = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        if (F32)
            mx = max(mx, w[d] & 0x7FFFFFFFu);
        else
            mx = max(mx, max((w[d] << 16) & 0x7FFFFFFFu, w[d] & 0x7FFF0000u));
    }
    // Every lane takes part in the shuffles; the group's lanes are
    // consecutive within the wave.
    mx = max_xor<1>(mx);
    mx = max_xor<2>(mx);
    if constexpr (LPG == 8)
        mx = max_xor<4>(mx);
    if (!live)
        return;
    const int k = truncfree_exp_e4m3(mx);
    const float scale = e8m0_scale(k);
    uint8_t* dst = p.codes + (int64_t)r * p.ld + c0;
    if constexpr (F32) {
        uint32_t o = 0;
        cvt8_rne_f32_word<0>(o, __uint_as_float(w[0]), __uint_as_float(w[1]), scale);
        cvt8_rne_f32_word<1>(o, __uint_as_float(w[2]), __uint_as_float(w[3]), scale);
        *reinterpret_cast<uint32_t*>(dst) = o;
    } else {
        uint32_t o0 = 0, o1 = 0;
        cvt8_rne_bf16_word<0>(o0, w[0], scale);
        cvt8_rne_bf16_word<1>(o0, w[1], scale);
        cvt8_rne_bf16_word<0>(o1, w[2], scale);
        cvt8_rne_bf16_word<1>(o1, w[3], scale);
        *reinterpret_cast<uint2*>(dst) = uint2{o0, o1};
    }
    if (sub == 0)
        p.scales[(int64_t)r * p.ld_s + g] = (uint8_t)(k + 127);
}

template <bool F32>
hipError_t launch_f(const Mxfp8Args& p, bool aligned, hipStream_t s)
{
    const int64_t n = p.rows * (p.cols_pad >> 5) * lanes_per_group<F32>();
    const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
    if (aligned)
        hipLaunchKernelGGL((mxfp8_kernel<F32, true>), grid, dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((mxfp8_kernel<F32, false>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

} // namespace

hipError_t launch_quant1d_mxfp8(const Mxfp8Args& p, bool f32, bool aligned, hipStream_t s)
{
    return f32 ? launch_f<true>(p, aligned, s) : launch_f<false>(p, aligned, s);
}

} // namespace fp4q
