// Cross-lane exchanges on CDNA4 (64-wide waves) without the LDS crossbar.
//
// max_xor<OFF>(x) returns max(x, x of lane l ^ OFF) in every lane l: the
// block-amax reductions of the quantizers.  Offsets inside a 16-lane row run
// on DPP moves (1 and 2: quad permutations; 8: the row rotated by 8),
// offsets 4 and 16 on ds_swizzle (xor within 32 lanes, no address
// register), and 32 on v_permlane32_swap.  Every lane of the wave must be
// active.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

// The values of lanes l and l ^ 32, as an unordered pair in every lane:
// v_permlane32_swap exchanges the upper half of one copy with the lower
// half of another.
__device__ __forceinline__ void swap32_pair(uint32_t x, uint32_t& a, uint32_t& b)
{
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    a = r[0];
    b = r[1];
}

template <int OFF>
__device__ __forceinline__ uint32_t max_xor(uint32_t x)
{
    static_assert(OFF == 1 || OFF == 2 || OFF == 4 || OFF == 8 || OFF == 16 || OFF == 32, "lane offset");
    if constexpr (OFF == 32) {
        uint32_t a, b;
        swap32_pair(x, a, b);
        return max(a, b);
    } else {
        int y;
        if constexpr (OFF == 1)
            y = __builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
        else if constexpr (OFF == 2)
            y = __builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
        else if constexpr (OFF == 8)
            y = __builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false);   // row_ror:8
        else
            y = __builtin_amdgcn_ds_swizzle((int)x, 0x1F | (OFF << 10));   // and 0x1F, xor OFF
        return max(x, (uint32_t)y);
    }
}

// max and sum of a float over lanes l and l ^ 32 (the two halves of the
// pair are combined in the same order in both lanes, so both get the same
// bits).
__device__ __forceinline__ float fmax_xor32(float x)
{
    uint32_t a, b;
    swap32_pair(__float_as_uint(x), a, b);
    return fmaxf(__uint_as_float(a), __uint_as_float(b));
}

__device__ __forceinline__ float fadd_xor32(float x)
{
    uint32_t a, b;
    swap32_pair(__float_as_uint(x), a, b);
    return __uint_as_float(a) + __uint_as_float(b);
}

} // namespace fp4q
