// Measured-peak probes.  (1) A sustained loop of block-scaled FP4 MFMAs, the
// instruction every FP4 product of this library runs on
// (v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands).  Its rate is the
// practical ceiling of the GEMMs on the chip at hand -- the clock the chip
// holds under matrix-core load, and the data-dependent issue rate -- and is
// reported next to the nominal dense FP4 peak.
//
// Each wave keeps 8 independent 32x32 accumulators (128 accumulation
// registers), so the matrix core never waits on a dependency, and multiplies
// operand words drawn from a per-lane hash: quantized Gaussian data, like
// the GEMMs' operands, has varied codes, and the MFMA rate measured on the box
// depends on the codes (structured codes run faster than random ones) -- or
// from a caller's code planes, so the loop multiplies a workload's own codes.
// (2) A streaming device copy with 16-byte accesses: the HBM rate a plain
// read-once / write-once kernel reaches.
#include "fp4q_launch.hpp"

#include <hip/hip_runtime.h>

namespace fp4q {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t mix32(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352dU;
    x ^= x >> 15;
    x *= 0x846ca68bU;
    x ^= x >> 16;
    return x;
}

// codes: NULL (operand words hashed per lane) or n_words >= 8 words of real
// FP4 code planes, of which each lane takes 8 consecutive words.
__global__ __launch_bounds__(256) void mfma_probe_kernel(int64_t iters, float* sink, const uint32_t* codes,
                                                         int64_t n_words)
{
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    v8i a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = i < 4 ? (int)mix32(2 * t + 17u * i + 1u) : 0;
        b[i] = i < 4 ? (int)mix32(2 * t + 17u * i + 2u) : 0;
    }
    if (codes) {
        const int64_t base = ((int64_t)t * 8) % (n_words - 7);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i] = (int)codes[base + i];
            b[i] = (int)codes[base + 4 + i];
        }
    }
    const int sa = 127 + (int)(mix32(t) & 3u), sb = 127 - (int)(mix32(t + 5u) & 3u);
    v16f acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[k][r] = 0.0f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            acc[k] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[k], 4, 4, 0, sa, 0, sb);
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            s += acc[k][r];
    sink[t] = s;
}

} // namespace

hipError_t launch_mfma_probe(int64_t iters, int workgroups, float* sink, const uint32_t* codes, int64_t n_words,
                             hipStream_t s)
{
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(256), 0, s, iters, sink, codes, n_words);
    return hipGetLastError();
}

namespace {

// Streaming copy: every thread moves 4 x 16 bytes per step of a grid-stride
// loop (16-byte loads and stores, 4 loads in flight before the stores).
__global__ __launch_bounds__(256) void copy_probe_kernel(const uint4* src, uint4* dst, int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * 256 * 4;
    int64_t i = ((int64_t)blockIdx.x * 256 * 4) + threadIdx.x;
    for (; i + 3 * 256 < n16; i += stride) {
        const uint4 v0 = src[i], v1 = src[i + 256], v2 = src[i + 512], v3 = src[i + 768];
        dst[i] = v0;
        dst[i + 256] = v1;
        dst[i + 512] = v2;
        dst[i + 768] = v3;
    }
    for (; i < n16; i += 256)
        dst[i] = src[i];
}

} // namespace

hipError_t launch_copy_probe(const void* src, void* dst, int64_t bytes, int workgroups, hipStream_t s)
{
    hipLaunchKernelGGL(copy_probe_kernel, dim3(workgroups), dim3(256), 0, s, static_cast<const uint4*>(src),
                       static_cast<uint4*>(dst), bytes / 16);
    return hipGetLastError();
}

namespace {

// A stream with a given read:write mix: every 16-byte word of dst is the
// xor of the words at the same index in `nread` consecutive source streams
// of n16 words each (a grid-stride loop, one word per thread per step).
// nread = 2 is the quantizer's mix (2 bytes of bf16 read per byte of codes
// written).
__global__ __launch_bounds__(256) void stream_probe_kernel(const uint4* src, uint4* dst, int64_t n16, int nread)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
        uint4 x = src[i];
        for (int r = 1; r < nread; ++r) {
            const uint4 y = src[i + r * n16];
            x.x ^= y.x;
            x.y ^= y.y;
            x.z ^= y.z;
            x.w ^= y.w;
        }
        dst[i] = x;
    }
}

} // namespace

hipError_t launch_stream_probe(const void* src, void* dst, int64_t bytes, int nread, int workgroups, hipStream_t s)
{
    hipLaunchKernelGGL(stream_probe_kernel, dim3(workgroups), dim3(256), 0, s, static_cast<const uint4*>(src),
                       static_cast<uint4*>(dst), bytes / 16, nread);
    return hipGetLastError();
}

namespace {

// One block-scaled FP8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 A and B)
// on a 32x64 A, a 32x64 B and their E8M0 scales (one per row and 32 K
// values): C[32 x 32] = A B^T.  One wave; lane l holds row (column) l % 32
// of A (B): registers 0-3 K values 16 (l / 32) .. +16 and registers 4-7 K
// values 32 + 16 (l / 32) .. +16, so K-block j (K 32 j .. +32) is registers
// 4j .. 4j+3 of both lane halves, and lane half j supplies K-block j's scale
// byte.  Accumulator register r of lane l is C[8 (r / 4) + 4 (l / 32) + r % 4]
// [l % 32].
__global__ __launch_bounds__(64) void mfma_fp8_block_kernel(const uint8_t* a, const uint8_t* b, const uint8_t* sa,
                                                            const uint8_t* sb, float* c)
{
    const int l = threadIdx.x, row = l & 31, kh = l >> 5;
    v8i va, vb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int k = (i >> 2) * 32 + kh * 16 + 4 * (i & 3);
        va[i] = *reinterpret_cast<const int*>(a + row * 64 + k);
        vb[i] = *reinterpret_cast<const int*>(b + row * 64 + k);
    }
    v16f acc;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        acc[r] = 0.0f;
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, 0, 0, 0, (int)sa[row * 2 + kh], 0,
                                                          (int)sb[row * 2 + kh]);
#pragma unroll
    for (int r = 0; r < 16; ++r)
        c[(8 * (r >> 2) + 4 * kh + (r & 3)) * 32 + row] = acc[r];
}

} // namespace

hipError_t launch_mfma_fp8_block(const uint8_t* a, const uint8_t* b, const uint8_t* sa, const uint8_t* sb, float* c,
                                 hipStream_t s)
{
    hipLaunchKernelGGL(mfma_fp8_block_kernel, dim3(1), dim3(64), 0, s, a, b, sa, sb, c);
    return hipGetLastError();
}

} // namespace fp4q
