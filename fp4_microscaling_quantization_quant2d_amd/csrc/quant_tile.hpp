// Per-lane quantization of an 8x8 block, shared by the 2D quantizer
// (quant2d.hip) and the GEMM epilogue that quantizes its own output
// (gemm_quant.hip), so both produce the same codes for the same values.
//
// "Stable FP4 Training via Transposition-Invariant Block Quantization":
//   Sec. 3    square blocks share one scale, S(B) = S(B^T)
//   Sec. 3.1  truncation-free S = 2^ceil(log2(M/6)), stochastic rounding
//   Sec. 2.1  P = round_FP4(X/S)
//
// A lane owns one 8x8 block; 64 lanes of a wave cover a 64-aligned 64x64
// square (lane = bc + 8*br: rows 8br.., cols 8bc..).  The square block of
// side BLK (8, 16, 32 or 64) of an element is therefore held by 1, 4, 16 or
// 64 lanes of one wave, and its amax is a cross-lane max over exactly those.
//
// Random bits: element (r, c) uses the Philox block keyed by the unordered
// pair (a, b) = (min, max) and its 16-bit half b%8.  For a block strictly
// above the diagonal (block row < block col) the 8 elements of one row share
// a Philox block; below the diagonal the 8 elements of one column do; on a
// diagonal block element (i, j) uses block min(i, j), half max(i, j).  Waves
// entirely above or below the diagonal take a uniform branch and index the
// words directly; only waves on the diagonal rearrange them per lane.
#pragma once

#include "fp4q_cvt.hpp"
#include "fp4q_device.hpp"
#include "lane_ops.hpp"

#include <type_traits>

namespace fp4q {
namespace qtile {

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

// Stochastic rounding of the lane's 8x8 block to nibbles, one converter per
// element (seed = its 16 random bits << 16).  The random bits of element
// (i, j) are half h of word w[a][b] of the lane's 8 Philox blocks:
//   ROWS   (block above the diagonal):  (a, b, h) = (i, j/2, j%2)
//   COLS   (block below the diagonal):  (a, b, h) = (j, i/2, i%2)
//   on the diagonal block:              a = min(i, j), half max(i, j)
// MIXED waves (those crossing the diagonal) pick among the three per lane.
// Even columns fill the bytes of a, odd columns those of b, so row word i is
// a | b << 4.
enum { kRows = 0, kCols = 1, kMixed = 2 };

// f(std::integral_constant<int, e>) for e = 0..3 (converter byte selects).
template <typename F>
__device__ __forceinline__ void static_for_sel(F&& f)
{
    f(std::integral_constant<int, 0>());
    f(std::integral_constant<int, 1>());
    f(std::integral_constant<int, 2>());
    f(std::integral_constant<int, 3>());
}

__device__ __forceinline__ uint32_t half_seed(uint32_t rd, int h) { return h ? (rd & 0xFFFF0000u) : (rd << 16); }

template <int MODE>
__device__ __forceinline__ uint32_t seed_of(const uint32_t w[8][4], int i, int j, bool lower, bool diag)
{
    const uint32_t up = half_seed(w[i][j >> 1], j & 1);
    const uint32_t lo = half_seed(w[j][i >> 1], i & 1);
    if (MODE == kRows)
        return up;
    if (MODE == kCols)
        return lo;
    const int a = i < j ? i : j, m = i < j ? j : i;
    const uint32_t dg = half_seed(w[a][m >> 1], m & 1);
    return diag ? dg : (lower ? lo : up);
}

template <int SEL, bool F32>
__device__ __forceinline__ void sr_pair(uint32_t& a, uint32_t& b, const Block8x8<F32>& blk, int i,
                                        uint32_t seed_even, uint32_t seed_odd, float scale)
{
    cvt_sr_byte<SEL>(a, __uint_as_float(blk.x32(i, 2 * SEL)), seed_even, scale);
    cvt_sr_byte<SEL>(b, __uint_as_float(blk.x32(i, 2 * SEL + 1)), seed_odd, scale);
}

template <bool F32, int MODE>
__device__ __forceinline__ void round_sr(const Block8x8<F32>& blk, const uint32_t w[8][4], float scale,
                                         bool lower, bool diag, uint32_t rw[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t a = 0, b = 0;
        sr_pair<0>(a, b, blk, i, seed_of<MODE>(w, i, 0, lower, diag), seed_of<MODE>(w, i, 1, lower, diag), scale);
        sr_pair<1>(a, b, blk, i, seed_of<MODE>(w, i, 2, lower, diag), seed_of<MODE>(w, i, 3, lower, diag), scale);
        sr_pair<2>(a, b, blk, i, seed_of<MODE>(w, i, 4, lower, diag), seed_of<MODE>(w, i, 5, lower, diag), scale);
        sr_pair<3>(a, b, blk, i, seed_of<MODE>(w, i, 6, lower, diag), seed_of<MODE>(w, i, 7, lower, diag), scale);
        rw[i] = a | (b << 4);
    }
}

// Round-to-nearest-even: one converter per pair of elements.
template <bool F32>
__device__ __forceinline__ void round_rne(const Block8x8<F32>& blk, float scale, uint32_t rw[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t a = 0;
        if (F32) {
            cvt_rne_f32_byte<0>(a, __uint_as_float(blk.x32(i, 0)), __uint_as_float(blk.x32(i, 1)), scale);
            cvt_rne_f32_byte<1>(a, __uint_as_float(blk.x32(i, 2)), __uint_as_float(blk.x32(i, 3)), scale);
            cvt_rne_f32_byte<2>(a, __uint_as_float(blk.x32(i, 4)), __uint_as_float(blk.x32(i, 5)), scale);
            cvt_rne_f32_byte<3>(a, __uint_as_float(blk.x32(i, 6)), __uint_as_float(blk.x32(i, 7)), scale);
        } else {
            cvt_rne_bf16_byte<0>(a, blk.v[i][0], scale);
            cvt_rne_bf16_byte<1>(a, blk.v[i][1], scale);
            cvt_rne_bf16_byte<2>(a, blk.v[i][2], scale);
            cvt_rne_bf16_byte<3>(a, blk.v[i][3], scale);
        }
        rw[i] = a;
    }
}

// Largest |x| bit pattern of the lane's block (fp32 bits).
template <bool F32>
__device__ __forceinline__ uint32_t block_amax(const Block8x8<F32>& blk)
{
    if (F32) {
        uint32_t mx = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                mx = max(mx, blk.x32(i, j) & 0x7FFFFFFFu);
        return mx;
    }
    // bf16: both halves at once with packed 16-bit max over the magnitudes
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    u16x2 m = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int d = 0; d < 4; ++d)
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, blk.v[i][d] & 0x7FFF7FFFu));
    return (uint32_t)max(m.x, m.y) << 16;
}

// Square-block amax: the lanes holding one BLK x BLK block differ in lane
// bits {0, 3} (16), {0, 1, 3, 4} (32) or all six (64); an 8x8 block is one
// lane.
template <int BLK>
__device__ __forceinline__ uint32_t square_amax(uint32_t mx)
{
    static_assert(BLK == 8 || BLK == 16 || BLK == 32 || BLK == 64, "block side");
    if constexpr (BLK >= 16)
        mx = max_xor<1>(mx);
    if constexpr (BLK >= 32)
        mx = max_xor<2>(mx);
    if constexpr (BLK >= 16)
        mx = max_xor<8>(mx);
    if constexpr (BLK >= 32)
        mx = max_xor<16>(mx);
    if constexpr (BLK == 64) {
        mx = max_xor<4>(mx);
        mx = max_xor<32>(mx);
    }
    return mx;
}

// Does this lane write its block's scale byte (the block's first lane)?
template <int BLK>
__device__ __forceinline__ bool block_leader(int lane)
{
    return BLK == 8 ? true : BLK == 16 ? (lane & 0x09) == 0 : BLK == 32 ? (lane & 0x1B) == 0 : lane == 0;
}

// The lane's 8 Philox blocks for its 8x8 block at (R0, C0): canonical
// orientation (P0, Q0) with P0 <= Q0 in 8-element units; block t covers row
// P0 + t and the eight values Q0 .. Q0 + 7 of its pair partner.
__device__ __forceinline__ void philox_words(uint32_t w[8][4], int R0, int C0, uint32_t stream, uint32_t key0,
                                             uint32_t key1)
{
    const int BR = R0 >> 3, BC = C0 >> 3;
    const int P0 = BR <= BC ? R0 : C0;
    const int Q0 = BR <= BC ? C0 : R0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        U4 c;
        c.x = (uint32_t)(((P0 & 31) + t) * 4 + ((Q0 & 31) >> 3));
        c.y = (uint32_t)(P0 >> 5);
        c.z = (uint32_t)(Q0 >> 5);
        c.w = stream;
        const U4 o = philox10(c, key0, key1);
        w[t][0] = o.x; w[t][1] = o.y; w[t][2] = o.z; w[t][3] = o.w;
    }
}

// Rounds the lane's block with block exponent k into 8 row words (nibble j
// of word i = element (i, j)).  (r0w, c0w): origin of the wave's 64-aligned
// 64x64 square, which decides the wave-uniform draw orientation.
template <bool F32, int RNE>
__device__ __forceinline__ void round_lane_block(const Block8x8<F32>& blk, int k, int R0, int C0, int r0w, int c0w,
                                                 uint32_t stream, uint32_t key0, uint32_t key1, uint32_t rw[8])
{
    const float scale = e8m0_scale(k);
    if (RNE) {
        round_rne<F32>(blk, scale, rw);
        return;
    }
    uint32_t w[8][4];
    philox_words(w, R0, C0, stream, key0, key1);
    // Waves strictly above the diagonal draw along rows, strictly below
    // along columns; a wave crossing the diagonal selects per lane.
    const int WR = r0w >> 6, WC = c0w >> 6;
    const int BR = R0 >> 3, BC = C0 >> 3;
    if (WR < WC)
        round_sr<F32, kRows>(blk, w, scale, false, false, rw);
    else if (WR > WC)
        round_sr<F32, kCols>(blk, w, scale, true, false, rw);
    else
        round_sr<F32, kMixed>(blk, w, scale, BR > BC, BR == BC, rw);
}

} // namespace qtile
} // namespace fp4q
