// MXFP8 quantizer for the query/key projections ("Stable FP4 Training via
// Transposition-Invariant Block Quantization", Sec. 3.2): E4M3FN elements,
// one E8M0 scale per 1x32 group along each row, truncation-free (the Sec. 3.1
// rule with Qp = 448, Qn = -448), round-to-nearest-even.
//
// One lane per 1x32 group: it reads 64 contiguous bytes (bf16) with four
// 16-byte loads, so a wave streams 4 KB; the group amax, the exponent and the
// 32 conversions stay in registers; 32 code bytes and one scale byte go out.
#include "fp4q_device.hpp"
#include "fp4q_launch.hpp"

namespace fp4q {

namespace {

constexpr int kThreads = 256;

// |x| * 2^-k rounded to nearest-even E4M3FN, magnitude code 0..126.
// x32: fp32 bits of x; the scaled value is at most 448 by construction.
__device__ __forceinline__ uint32_t e4m3_code(uint32_t x32, int k)
{
    const uint32_t a = x32 & 0x7FFFFFFFu;
    int E = (int)(a >> 23);
    uint32_t m24 = (a & 0x7FFFFFu) | 0x800000u;
    if (E == 0) {
        if (a == 0)
            return 0;
        const int lz = __builtin_clz(a) - 8;   // normalize a subnormal input
        m24 = a << lz;
        E = 1 - lz;
    }
    const int Ev = E - k;                      // biased exponent of v = |x| * 2^-k
    if (Ev >= 121) {                           // v >= 2^-6: normal E4M3, 3 mantissa bits
        uint32_t T = m24 >> 20;
        const uint32_t rem = m24 & 0xFFFFFu;
        T += (rem > 0x80000u || (rem == 0x80000u && (T & 1u))) ? 1u : 0u;
        int e = Ev - 120;
        if (T == 16u) {
            T = 8u;
            ++e;
        }
        return ((uint32_t)e << 3) | (T & 7u);
    }
    // subnormal E4M3: multiples of 2^-9, code = RNE(v * 2^9)
    const int s = imin(141 - Ev, 31);
    const uint32_t T = m24 >> s;
    const uint32_t rem = m24 & ((1u << s) - 1u);
    const uint32_t half = 1u << (s - 1);
    return T + ((rem > half || (rem == half && (T & 1u))) ? 1u : 0u);
}

template <bool F32, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void mxfp8_kernel(Mxfp8Args p)
{
    const int groups = p.cols_pad >> 5;
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= p.rows * groups)
        return;
    const int64_t r = gid / groups;
    const int g = (int)(gid - r * groups);
    const int c0 = g * 32;
    const int esz = F32 ? 4 : 2;
    const char* row = static_cast<const char*>(p.x) + r * p.ldx * esz;

    uint32_t v[32];
    if (ALIGNED && c0 + 32 <= p.cols) {
        const uint4* src = reinterpret_cast<const uint4*>(row + (int64_t)c0 * esz);
        if (F32) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint4 t = src[q];
                v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 t = src[q];
                const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    v[8 * q + 2 * d] = w[d] << 16;
                    v[8 * q + 2 * d + 1] = w[d] & 0xFFFF0000u;
                }
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const int c = c0 + j;
            uint32_t x = 0;
            if (c < p.cols)
                x = F32 ? reinterpret_cast<const uint32_t*>(row)[c]
                        : (uint32_t)reinterpret_cast<const uint16_t*>(row)[c] << 16;
            v[j] = x;
        }
    }
    uint32_t mx = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j)
        mx = max(mx, v[j] & 0x7FFFFFFFu);
    const int k = truncfree_exp_e4m3(mx);
    uint32_t out[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        uint32_t w = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t x = v[4 * q + b];
            const uint32_t byte = e4m3_code(x, k) | ((x >> 24) & 0x80u);
            w |= byte << (8 * b);
        }
        out[q] = w;
    }
    uint4* dst = reinterpret_cast<uint4*>(p.codes + r * p.ld + c0);
    dst[0] = uint4{out[0], out[1], out[2], out[3]};
    dst[1] = uint4{out[4], out[5], out[6], out[7]};
    p.scales[r * p.ld_s + g] = (uint8_t)(k + 127);
}

template <bool F32>
hipError_t launch_f(const Mxfp8Args& p, bool aligned, hipStream_t s)
{
    const int64_t n = p.rows * (p.cols_pad >> 5);
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
