// Device-side building blocks shared by the fp4q kernels (gfx950).
//
// Number formats ("Stable FP4 Training via Transposition-Invariant Block
// Quantization", Sec. 2 / 2.1): E2M1 elements (magnitudes 0, .5, 1, 1.5, 2,
// 3, 4, 6), E8M0 power-of-two scales, and for the query/key path of Sec. 3.2
// E4M3FN elements.  These helpers are written for the CDNA4 execution model:
// 64-wide waves, integer-only scale selection, register-level transposes.
// Element rounding to E2M1 is done by the hardware converters (fp4q_cvt.hpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define FP4Q_HD __host__ __device__ __forceinline__

namespace fp4q {

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw: "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11).  Ten rounds; each multiplies counter words 0 and
// 2 by the published 32-bit constants, xors the high halves into the other
// words with the round key, and advances the key by the Weyl increments.
// The key is wave-uniform, so its schedule lives in scalar registers.
// ---------------------------------------------------------------------------
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

struct U4 {
    uint32_t x, y, z, w;
};

// a ^ b ^ k with k wave-uniform: one gfx950 three-input bit operation
// (truth table 0x96 = xor of all three) with a scalar operand.
FP4Q_HD uint32_t xor3_uniform(uint32_t a, uint32_t b, uint32_t k)
{
#if defined(__HIP_DEVICE_COMPILE__)
    uint32_t r;
    asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
    return r;
#else
    return a ^ b ^ k;
#endif
}

FP4Q_HD U4 philox10(U4 c, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)kPhiloxM0 * c.x;
        const uint64_t p1 = (uint64_t)kPhiloxM1 * c.z;
        U4 n;
        n.x = xor3_uniform((uint32_t)(p1 >> 32), c.y, k0);
        n.y = (uint32_t)p1;
        n.z = xor3_uniform((uint32_t)(p0 >> 32), c.w, k1);
        n.w = (uint32_t)p0;
        c = n;
        k0 += kPhiloxW0;
        k1 += kPhiloxW1;
    }
    return c;
}

// ---------------------------------------------------------------------------
// Truncation-free E8M0 exponent (Sec. 3.1, S = 2^ceil(log2(M/6)) for E2M1,
// the same rule with 448 for E4M3), computed exactly from the fp32 bits of
// the block amax M (an unsigned magnitude bit pattern).
//   M = 1.m * 2^(E-127):  M/6 = (1.m/1.5) * 2^(E-129) and 1.m/1.5 is in
//   [2/3, 4/3), so ceil(log2(M/6)) = E - 129 + [1.m > 1.5].
//   For 448 = 1.75 * 2^8: ceil(log2(M/448)) = E - 135 + [1.m > 1.75].
// Zero or subnormal M (E = 0) and anything below 2^-127 clamp to -127.
// ---------------------------------------------------------------------------
FP4Q_HD int truncfree_exp_e2m1(uint32_t amax_bits)
{
    const int E = (int)(amax_bits >> 23);
    if (E == 0)
        return -127;
    const int k = E - 129 + ((amax_bits & 0x7FFFFFu) > 0x400000u ? 1 : 0);
    return k < -127 ? -127 : k;
}

FP4Q_HD int imin(int a, int b) { return a < b ? a : b; }
FP4Q_HD int imax(int a, int b) { return a > b ? a : b; }

FP4Q_HD int truncfree_exp_e4m3(uint32_t amax_bits)
{
    const int E = (int)(amax_bits >> 23);
    if (E == 0)
        return -127;
    const int k = E - 135 + ((amax_bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    return k < -127 ? -127 : k;
}

// ---------------------------------------------------------------------------
// 8x8 nibble transpose in registers: w[i] holds row i (nibble j = column j)
// on entry and column i (nibble j = row j) on exit.  Three levels: swap the
// off-diagonal 4x4 blocks (16-bit halves), then the 2x2 blocks of each 4x4
// (bytes), then single nibbles.  32 VALU ops for 64 elements.
// ---------------------------------------------------------------------------
FP4Q_HD uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_perm(hi, lo, sel);
#else
    const uint64_t v = ((uint64_t)hi << 32) | lo;
    uint32_t r = 0;
    for (int b = 0; b < 4; ++b) {
        const uint32_t s = (sel >> (8 * b)) & 0xFFu;
        r |= (uint32_t)((v >> (8 * (s & 7))) & 0xFFu) << (8 * b);
    }
    return r;
#endif
}

FP4Q_HD uint32_t bfi_b32(uint32_t mask, uint32_t a, uint32_t b) { return (mask & a) | (~mask & b); }

FP4Q_HD void nibble_transpose8(uint32_t w[8])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t a = w[i], b = w[i + 4];
        w[i] = perm_b32(b, a, 0x05040100u);     // lo16(a) | lo16(b) << 16
        w[i + 4] = perm_b32(b, a, 0x07060302u); // hi16(a) | hi16(b) << 16
    }
#pragma unroll
    for (int h = 0; h < 8; h += 4) {
#pragma unroll
        for (int i = h; i < h + 2; ++i) {
            const uint32_t a = w[i], b = w[i + 2];
            w[i] = perm_b32(b, a, 0x06020400u);
            w[i + 2] = perm_b32(b, a, 0x07030501u);
        }
    }
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        const uint32_t a = w[i], b = w[i + 1];
        w[i] = bfi_b32(0x0F0F0F0Fu, a, b << 4);
        w[i + 1] = bfi_b32(0x0F0F0F0Fu, a >> 4, b);
    }
}

} // namespace fp4q
