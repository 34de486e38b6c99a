// Dequantization X ~ P * S ("Stable FP4 Training via Transposition-Invariant
// Block Quantization", Sec. 2.1) of a FP4 2D-block plane (row or transposed),
// a plane of the 1D activation layout, or a MXFP8 1x32 plane, to fp32 or bf16.  One lane per 8 output elements.
// Every E2M1 or E4M3 value times a power of two is exact in fp32, and the
// FP4 products (at most 2 significant bits) are exact in bf16 as well.
#include "fp4q_device.hpp"
#include "fp4q_launch.hpp"

namespace fp4q {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float pow2_e8m0(uint32_t b)
{
    // 2^(b-127): normal for b >= 1; b = 0 is the subnormal 2^-127
    return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

__device__ __forceinline__ float e2m1_val(uint32_t nib)
{
    const uint32_t code = nib & 7u;
    const uint32_t e = code >> 1, m = code & 1u;
    const float mag = e == 0 ? 0.5f * (float)m : (float)(2u + m) * (float)(1u << e) * 0.25f;
    return (nib & 8u) ? -mag : mag;
}

__device__ __forceinline__ float e4m3_val(uint32_t byte)
{
    const uint32_t e = (byte >> 3) & 15u, m = byte & 7u;
    float mag;
    if (e == 0)
        mag = (float)m * 0.001953125f;  // 2^-9
    else
        mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (byte & 0x80u) ? -mag : mag;
}

template <int FMT, bool BF16>
__global__ __launch_bounds__(kThreads) void dequant_kernel(DequantArgs p)
{
    const int per_row = (p.cols + 7) >> 3;
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= (int64_t)p.rows * per_row)
        return;
    const int r = (int)(gid / per_row);
    const int c0 = (int)(gid - (int64_t)r * per_row) * 8;
    float out[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int c = c0 + j;
        float val = 0.0f;
        if (c < p.cols) {
            if (FMT == 1) {
                const uint32_t byte = p.codes[(int64_t)r * p.ld + (c >> 1)];
                const uint32_t nib = (byte >> (4 * (c & 1))) & 15u;
                const int bs = p.block_shift;
                uint32_t sb;
                if (p.scale_transposed == 2)  // 1D layout: tiled grid of this plane
                    sb = p.scales[(int64_t)(r >> 7) * p.ld_s + (c >> 7) * 512 + ((c >> 5) & 1) * 256 + (r & 31) * 8 +
                                  ((r >> 5) & 3) * 2 + ((c >> 6) & 1)];
                else
                    sb = p.scale_transposed ? p.scales[(int64_t)(c >> bs) * p.ld_s + (r >> bs)]
                                            : p.scales[(int64_t)(r >> bs) * p.ld_s + (c >> bs)];
                val = e2m1_val(nib) * pow2_e8m0(sb);
            } else {
                const uint32_t byte = p.codes[(int64_t)r * p.ld + c];
                val = e4m3_val(byte) * pow2_e8m0(p.scales[(int64_t)r * p.ld_s + (c >> 5)]);
            }
        }
        out[j] = val;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int c = c0 + j;
        if (c >= p.cols)
            break;
        if (BF16)
            reinterpret_cast<uint16_t*>(p.y)[(int64_t)r * p.ldy + c] = (uint16_t)(__float_as_uint(out[j]) >> 16);
        else
            reinterpret_cast<float*>(p.y)[(int64_t)r * p.ldy + c] = out[j];
    }
}

template <int FMT>
hipError_t launch_f(const DequantArgs& p, bool bf16, hipStream_t s)
{
    const int64_t n = (int64_t)p.rows * ((p.cols + 7) >> 3);
    const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
    if (bf16)
        hipLaunchKernelGGL((dequant_kernel<FMT, true>), grid, dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((dequant_kernel<FMT, false>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

} // namespace

hipError_t launch_dequant(const DequantArgs& p, int fmt, bool out_bf16, hipStream_t s)
{
    return fmt == 1 ? launch_f<1>(p, out_bf16, s) : launch_f<2>(p, out_bf16, s);
}

} // namespace fp4q
