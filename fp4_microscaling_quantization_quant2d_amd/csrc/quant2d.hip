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
// lanes of its tile with DPP and ds_swizzle exchanges, derives the E8M0 byte,
// draws 8 Philox blocks and rounds its 64 elements with the hardware FP4
// converters (scale folded in; one per element for stochastic rounding, one
// per pair for round-to-nearest-even), which write the nibbles straight into
// 8 row words; an in-register nibble transpose gives the 8 column words of
// the transposed plane, so both planes and the scale grid come from one read.
//
// Random bits: element (r, c) uses the Philox block keyed by the unordered
// pair (a, b) = (min, max) and its 16-bit half b%8.  For a block strictly
// above the diagonal (block row < block col) the 8 elements of one row share
// a Philox block; below the diagonal the 8 elements of one column do; on a
// diagonal block element (i, j) uses block min(i, j), half max(i, j).  Waves
// entirely above or below the diagonal take a uniform branch and index the
// words directly; only waves on the diagonal rearrange them per lane.
#include "fp4q_launch.hpp"
#include "quant_tile.hpp"

#include <type_traits>

namespace fp4q {

namespace {

using namespace qtile;

constexpr int kThreads = 256;
constexpr int kRegion = 128;

// Loads the lane's 8x8 block at (R0, C0).  A block fully inside an aligned
// input takes 8 (bf16) or 16 (fp32) 16-byte loads off one base pointer; an
// edge block loads element by element and zero-fills the padding.
template <bool F32, bool ALIGNED>
__device__ __forceinline__ void load_block(Block8x8<F32>& blk, const Quant2dArgs& p, int R0, int C0)
{
    constexpr int esz = F32 ? 4 : 2;
    const int64_t stride = p.ldx * esz;
    const char* row = static_cast<const char*>(p.x) + ((int64_t)R0 * p.ldx + C0) * esz;
    if (ALIGNED && R0 + 8 <= p.rows && C0 + 8 <= p.cols) {
#pragma unroll
        for (int i = 0; i < 8; ++i, row += stride) {
            const uint4 a = *reinterpret_cast<const uint4*>(row);
            blk.v[i][0] = a.x; blk.v[i][1] = a.y; blk.v[i][2] = a.z; blk.v[i][3] = a.w;
            if constexpr (F32) {
                const uint4 b = *reinterpret_cast<const uint4*>(row + 16);
                blk.v[i][4] = b.x; blk.v[i][5] = b.y; blk.v[i][6] = b.z; blk.v[i][7] = b.w;
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i, row += stride) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool in = R0 + i < p.rows && C0 + j < p.cols;
            if constexpr (F32) {
                blk.v[i][j] = in ? reinterpret_cast<const uint32_t*>(row)[j] : 0u;
            } else {
                const uint32_t val = in ? reinterpret_cast<const uint16_t*>(row)[j] : 0u;
                if (j & 1)
                    blk.v[i][j >> 1] |= val << 16;
                else
                    blk.v[i][j >> 1] = val;
            }
        }
    }
}

// Position of a lane's 8x8 block inside region `region` (128x128 per
// workgroup, 64x64 per wave).
struct LanePos {
    int rr0, cc0;   // region origin
    int r0w, c0w;   // wave origin
    int R0, C0;     // block origin
    bool active;
};

__device__ __forceinline__ LanePos lane_pos(const Quant2dArgs& p, int region, int nbx)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int by = region / nbx, bx = region - by * nbx;
    LanePos q;
    q.rr0 = by * kRegion;
    q.cc0 = bx * kRegion;
    q.r0w = by * kRegion + (wave >> 1) * 64;
    q.c0w = bx * kRegion + (wave & 1) * 64;
    q.R0 = q.r0w + 8 * (lane >> 3);
    q.C0 = q.c0w + 8 * (lane & 7);
    q.active = q.R0 < p.rows_pad && q.C0 < p.cols_pad;
    return q;
}

template <bool F32, bool ALIGNED>
__device__ __forceinline__ void fetch(Block8x8<F32>& blk, const Quant2dArgs& p, const LanePos& q)
{
    if (q.active)
        load_block<F32, ALIGNED>(blk, p, q.R0, q.C0);
}

// Output staging in LDS: both planes of a region, 128 rows of 64 bytes each,
// rows padded to 68 bytes so that the lanes' dword writes hit 64 distinct
// banks.
constexpr int kStageRow = 68;
constexpr int kStagePlane = kRegion * kStageRow;
constexpr int kStageBuf = 2 * kStagePlane;

// Scale, random bits and rounding of one lane block whose data is in blk,
// then the stores of the workgroup's region.  Every lane reaches the
// barrier; lanes outside the padded matrix compute nothing and their
// staging entries are never stored.  BLK: the square block side (8, 16, 32
// or 64; a 64x64 block is exactly one wave's region).
template <bool F32, int RNE, int BLK>
__device__ __forceinline__ void process(const Block8x8<F32>& blk, const Quant2dArgs& p, const LanePos& q,
                                        uint8_t* stage)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint32_t mx = square_amax<BLK>(q.active ? block_amax<F32>(blk) : 0u);
    const int R0 = q.R0, C0 = q.C0;
    uint32_t rw[8] = {};
    if (q.active) {
        const int k = truncfree_exp_e2m1(mx);
        round_lane_block<F32, RNE>(blk, k, R0, C0, q.r0w, q.c0w, p.stream, p.key0, p.key1, rw);
        if (block_leader<BLK>(lane)) {
            constexpr int sh = BLK == 8 ? 3 : BLK == 16 ? 4 : BLK == 32 ? 5 : 6;
            p.scales[(int64_t)(R0 >> sh) * p.ld_s + (C0 >> sh)] = (uint8_t)(k + 127);
        }
    }

    // Stage the row words and (after an in-register nibble transpose) the
    // column words of the lane's block.
    const int br = lane >> 3, bc = lane & 7;
    uint8_t* srow = stage + ((wave >> 1) * 64 + 8 * br) * kStageRow + (wave & 1) * 32 + 4 * bc;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        *reinterpret_cast<uint32_t*>(srow + i * kStageRow) = rw[i];
    const bool both = p.codes_t != nullptr;
    if (both) {
        nibble_transpose8(rw);
        uint8_t* scol = stage + kStagePlane + ((wave & 1) * 64 + 8 * bc) * kStageRow + (wave >> 1) * 32 + 4 * br;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *reinterpret_cast<uint32_t*>(scol + j * kStageRow) = rw[j];
    }
    // LDS writes visible to the workgroup.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // Each plane of the region as 512 16-byte pieces: four consecutive
    // threads write one 64-byte row segment.  A piece spans 32 columns
    // (row plane) or 32 rows (transposed plane), so it lies wholly inside or
    // wholly outside the padded matrix.
    const int t = threadIdx.x;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int piece = t + kThreads * m;
        const int row = piece >> 2, seg = piece & 3;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(stage + row * kStageRow + seg * 16);
        const uint4 v = {src[0], src[1], src[2], src[3]};
        if (q.rr0 + row < p.rows_pad && q.cc0 + 32 * seg < p.cols_pad)
            *reinterpret_cast<uint4*>(p.codes + (int64_t)(q.rr0 + row) * p.ld + (q.cc0 >> 1) + 16 * seg) = v;
        if (both) {
            const uint32_t* tsrc = reinterpret_cast<const uint32_t*>(stage + kStagePlane + row * kStageRow + seg * 16);
            const uint4 u = {tsrc[0], tsrc[1], tsrc[2], tsrc[3]};
            if (q.cc0 + row < p.cols_pad && q.rr0 + 32 * seg < p.rows_pad)
                *reinterpret_cast<uint4*>(p.codes_t + (int64_t)(q.cc0 + row) * p.ld_t + (q.rr0 >> 1) + 16 * seg) = u;
        }
    }
}

// ---------------------------------------------------------------------------
// 1D activation layout (appendix "Activations": activations are quantized in
// 1D blocks along the hidden channels).  The row plane takes one scale per
// 1x32 block of a row (for the forward product, which contracts over the
// channels); the transposed plane one scale per 1x32 block of a row of x^T,
// i.e. 32 tokens of one channel (for the weight-gradient product, which
// contracts over the tokens).  An element is rounded twice, once per plane
// and scale, with the same random field as in the 2D layout.

// max over the lanes whose index differs in `mask` bits (mask < 32), via a
// bit-mode ds_swizzle: source lane = lane ^ mask within each 32-lane half.
template <int MASK>
__device__ __forceinline__ uint32_t xor_max(uint32_t v)
{
    return max(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (MASK << 10) | 0x1F));
}

// Per-row and per-column |x| maxima of the lane's block, as fp32 bit
// patterns, reduced over the 4 lanes of each 32-wide row block (lane bits 0,
// 1) and the 4 lanes of each 32-high column block (lane bits 3, 4).
template <bool F32>
__device__ __forceinline__ void line_amax(const Block8x8<F32>& blk, bool active, uint32_t rmx[8], uint32_t cmx[8])
{
    if (F32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            rmx[i] = 0;
            cmx[i] = 0;
        }
        if (active) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t a = blk.x32(i, j) & 0x7FFFFFFFu;
                    rmx[i] = max(rmx[i], a);
                    cmx[j] = max(cmx[j], a);
                }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            rmx[i] = xor_max<2>(xor_max<1>(rmx[i]));
            cmx[i] = xor_max<16>(xor_max<8>(cmx[i]));
        }
        return;
    }
    // bf16: 16-bit magnitudes, two per dword (rows 2s and 2s+1, columns 2d
    // and 2d+1), maxed as pairs; the swizzled dword max stays per half
    // because the halves are compared separately.
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    u16x2 rm[8], cm[4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        rm[i] = u16x2{0, 0};
#pragma unroll
    for (int d = 0; d < 4; ++d)
        cm[d] = u16x2{0, 0};
    if (active) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const u16x2 a = __builtin_bit_cast(u16x2, blk.v[i][d] & 0x7FFF7FFFu);
                rm[i] = __builtin_elementwise_max(rm[i], a);
                cm[d] = __builtin_elementwise_max(cm[d], a);
            }
    }
    uint32_t rp[4], cp[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        rp[s] = (uint32_t)max(rm[2 * s].x, rm[2 * s].y) | ((uint32_t)max(rm[2 * s + 1].x, rm[2 * s + 1].y) << 16);
        cp[s] = __builtin_bit_cast(uint32_t, cm[s]);
    }
    auto pmax = [](uint32_t a, uint32_t b) {
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                      __builtin_bit_cast(u16x2, b)));
    };
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        rp[s] = pmax(rp[s], (uint32_t)__builtin_amdgcn_ds_swizzle((int)rp[s], (1 << 10) | 0x1F));
        rp[s] = pmax(rp[s], (uint32_t)__builtin_amdgcn_ds_swizzle((int)rp[s], (2 << 10) | 0x1F));
        cp[s] = pmax(cp[s], (uint32_t)__builtin_amdgcn_ds_swizzle((int)cp[s], (8 << 10) | 0x1F));
        cp[s] = pmax(cp[s], (uint32_t)__builtin_amdgcn_ds_swizzle((int)cp[s], (16 << 10) | 0x1F));
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        rmx[2 * s] = rp[s] << 16;
        rmx[2 * s + 1] = rp[s] & 0xFFFF0000u;
        cmx[2 * s] = cp[s] << 16;
        cmx[2 * s + 1] = cp[s] & 0xFFFF0000u;
    }
}

// Stochastic rounding of the lane's block for both 1D planes: row word i
// (scale sr[i]) and column word j (scale sc[j], nibble i = row i), each
// element with the random bits it uses in the 2D layout.  Both conversions
// of an element follow its draw directly, so no draw outlives its element.
template <int N, typename F>
__device__ __forceinline__ void static_for_n(F&& f)
{
    if constexpr (N > 0) {
        static_for_n<N - 1>(f);
        f(std::integral_constant<int, N - 1>());
    }
}

template <bool F32, int MODE>
__device__ __forceinline__ void round_sr_1d(const Block8x8<F32>& blk, const uint32_t w[8][4], const float sr[8],
                                            const float sc[8], bool lower, bool diag, bool both, uint32_t rw[8],
                                            uint32_t cw[8])
{
    uint32_t ra[8] = {}, rb[8] = {}, ca[8] = {}, cb[8] = {};
    static_for_n<8>([&](auto I) {
        constexpr int i = decltype(I)::value;
        static_for_n<8>([&](auto J) {
            constexpr int j = decltype(J)::value;
            const uint32_t seed = seed_of<MODE>(w, i, j, lower, diag);
            const float x = __uint_as_float(blk.x32(i, j));
            cvt_sr_byte<j / 2>(j & 1 ? rb[i] : ra[i], x, seed, sr[i]);
            if (both)
                cvt_sr_byte<i / 2>(i & 1 ? cb[j] : ca[j], x, seed, sc[j]);
        });
    });
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        rw[k] = ra[k] | (rb[k] << 4);
        cw[k] = ca[k] | (cb[k] << 4);
    }
}

// Round-to-nearest-even for both 1D planes.
template <bool F32>
__device__ __forceinline__ void round_rne_1d(const Block8x8<F32>& blk, const float sr[8], const float sc[8], bool both,
                                             uint32_t rw[8], uint32_t cw[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t a = 0;
        static_for_sel([&](auto SEL) {
            constexpr int e = decltype(SEL)::value;
            if (F32)
                cvt_rne_f32_byte<e>(a, __uint_as_float(blk.x32(i, 2 * e)), __uint_as_float(blk.x32(i, 2 * e + 1)),
                                    sr[i]);
            else
                cvt_rne_bf16_byte<e>(a, blk.v[i][e], sr[i]);
        });
        rw[i] = a;
    }
    if (!both)
        return;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t a = 0;
        static_for_sel([&](auto SEL) {
            constexpr int e = decltype(SEL)::value;
            cvt_rne_f32_byte<e>(a, __uint_as_float(blk.x32(2 * e, j)), __uint_as_float(blk.x32(2 * e + 1, j)), sc[j]);
        });
        cw[j] = a;
    }
}

// Scale grids of the 1D layout are tiled for the GEMM: the bytes of 128
// rows x 4 K-blocks (one 128x128 region of a plane) form one 512-byte chunk,
// chunk (g, q) of rows 128g.. and K-blocks 4q.. at g*ld + q*512, and inside
// it the byte of (row r, K-block kb) sits at
//     (kb%2)*256 + (r%32)*8 + ((r/32)%4)*2 + (kb/2)%2,
// so that one 8-byte word holds what one MFMA lane needs for a 64-K-byte
// stage: its row in each of four 32-row slabs, for both K-steps.  A region
// stages its chunk of each grid in LDS, then writes it with 16-byte stores.
constexpr int kStageScales = 2 * 512;

__device__ __forceinline__ int act1d_chunk_pos(int r, int kb)
{
    return (kb & 1) * 256 + (r & 31) * 8 + ((r >> 5) & 3) * 2 + ((kb >> 1) & 1);
}

// 1D counterpart of process(): both planes and both scale grids of the
// lane's block, the planes staged and stored as in the 2D layout, the scale
// bytes as one 512-byte chunk per grid and region.
template <bool F32, int RNE>
__device__ __forceinline__ void process1d(const Block8x8<F32>& blk, const Quant2dArgs& p, const LanePos& q,
                                          uint8_t* stage)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int br = lane >> 3, bc = lane & 7;
    const bool both = p.codes_t != nullptr;
    uint32_t rmx[8], cmx[8];
    line_amax<F32>(blk, q.active, rmx, cmx);
    int kr[8], kc[8];
    float sr[8], sc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        kr[i] = truncfree_exp_e2m1(rmx[i]);
        kc[i] = truncfree_exp_e2m1(cmx[i]);
        sr[i] = e8m0_scale(kr[i]);
        sc[i] = e8m0_scale(kc[i]);
    }
    const int R0 = q.R0, C0 = q.C0;
    uint32_t rw[8] = {}, cw[8] = {};
    if (q.active) {
        if (RNE) {
            round_rne_1d<F32>(blk, sr, sc, both, rw, cw);
        } else {
            const int BR = R0 >> 3, BC = C0 >> 3;
            uint32_t w[8][4];
            philox_words(w, R0, C0, p.stream, p.key0, p.key1);
            const int WR = q.r0w >> 6, WC = q.c0w >> 6;
            if (WR < WC)
                round_sr_1d<F32, kRows>(blk, w, sr, sc, false, false, both, rw, cw);
            else if (WR > WC)
                round_sr_1d<F32, kCols>(blk, w, sr, sc, true, false, both, rw, cw);
            else
                round_sr_1d<F32, kMixed>(blk, w, sr, sc, BR > BC, BR == BC, both, rw, cw);
        }
    }

    uint8_t* srow = stage + ((wave >> 1) * 64 + 8 * br) * kStageRow + (wave & 1) * 32 + 4 * bc;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        *reinterpret_cast<uint32_t*>(srow + i * kStageRow) = rw[i];
    if (both) {
        uint8_t* scol = stage + kStagePlane + ((wave & 1) * 64 + 8 * bc) * kStageRow + (wave >> 1) * 32 + 4 * br;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *reinterpret_cast<uint32_t*>(scol + j * kStageRow) = cw[j];
    }
    // Scale bytes: the first lane of each row block's four lanes writes its
    // 8 rows (region rows 64wr + 8br + i, K-block 2wc + bc/4), the first lane
    // of each column block's four its 8 columns (transposed-plane rows
    // 64wc + 8bc + j, K-block 2wr + br/4); consecutive rows are 8 bytes apart.
    uint8_t* ss = stage + kStageBuf;
    const int wr = wave >> 1, wc = wave & 1;
    if ((bc & 3) == 0) {
        uint8_t* d = ss + act1d_chunk_pos(64 * wr + 8 * br, 2 * wc + (bc >> 2));
#pragma unroll
        for (int i = 0; i < 8; ++i)
            d[8 * i] = (uint8_t)(kr[i] + 127);
    }
    if (both && (br & 3) == 0) {
        uint8_t* d = ss + 512 + act1d_chunk_pos(64 * wc + 8 * bc, 2 * wr + (br >> 2));
#pragma unroll
        for (int j = 0; j < 8; ++j)
            d[8 * j] = (uint8_t)(kc[j] + 127);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    const int t = threadIdx.x;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int piece = t + kThreads * m;
        const int row = piece >> 2, seg = piece & 3;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(stage + row * kStageRow + seg * 16);
        const uint4 v = {src[0], src[1], src[2], src[3]};
        if (q.rr0 + row < p.rows_pad && q.cc0 + 32 * seg < p.cols_pad)
            *reinterpret_cast<uint4*>(p.codes + (int64_t)(q.rr0 + row) * p.ld + (q.cc0 >> 1) + 16 * seg) = v;
        if (both) {
            const uint32_t* tsrc = reinterpret_cast<const uint32_t*>(stage + kStagePlane + row * kStageRow + seg * 16);
            const uint4 u = {tsrc[0], tsrc[1], tsrc[2], tsrc[3]};
            if (q.cc0 + row < p.cols_pad && q.rr0 + 32 * seg < p.rows_pad)
                *reinterpret_cast<uint4*>(p.codes_t + (int64_t)(q.cc0 + row) * p.ld_t + (q.rr0 >> 1) + 16 * seg) = u;
        }
    }
    // Threads 0..31 store the row grid's chunk (g, q) = (rr0/128, cc0/128),
    // threads 32..63 the transposed grid's chunk (cc0/128, rr0/128).  Rows and
    // K-blocks of the chunk past the matrix hold 0 (their lanes saw no data).
    if (t < 32) {
        const uint4 v = reinterpret_cast<const uint4*>(ss)[t];
        *reinterpret_cast<uint4*>(p.scales + (int64_t)(q.rr0 >> 7) * p.ld_s + (q.cc0 >> 7) * 512 + 16 * t) = v;
    } else if (both && t < 64) {
        const uint4 v = reinterpret_cast<const uint4*>(ss)[t];
        *reinterpret_cast<uint4*>(p.scales_t + (int64_t)(q.cc0 >> 7) * p.ld_st + (q.rr0 >> 7) * 512 +
                                  16 * (t - 32)) = v;
    }
}

// One workgroup per 128x128 region.  The hardware dispatcher hands regions
// to compute units as earlier ones retire, which balances the device better
// than a persistent grid walking the regions with a fixed stride: there the
// oldest-first wave priority inside a compute unit lets some workgroups
// finish well before others.  A batch launch covers the regions of several
// matrices, so their ramps and tails overlap.
// LAYOUT: 0 = 32x32 blocks, 1 = 64x64 blocks, 2 = 1D activation layout,
// 3 = 16x16 blocks, 4 = 8x8 blocks.
template <bool F32, int RNE, bool ALIGNED, int LAYOUT>
__global__ __launch_bounds__(kThreads) void quant2d_kernel(Quant2dBatch b)
{
    __shared__ __attribute__((aligned(16))) uint8_t stage[LAYOUT == 2 ? kStageBuf + kStageScales : kStageBuf];
    int i = 0;
    while (i + 1 < b.n && (int)blockIdx.x >= b.first[i + 1])
        ++i;
    Quant2dArgs p = b.item[i];
    if (b.seed_dev) {
        // device-resident seed (graph replays draw fresh bits): key += *seed_dev
        const uint64_t k = ((uint64_t)p.key1 << 32 | p.key0) + *b.seed_dev;
        p.key0 = (uint32_t)k;
        p.key1 = (uint32_t)(k >> 32);
    }
    const int nbx = (p.cols_pad + kRegion - 1) / kRegion;
    Block8x8<F32> blk;
    const LanePos q = lane_pos(p, (int)blockIdx.x - b.first[i], nbx);
    fetch<F32, ALIGNED>(blk, p, q);
    if constexpr (LAYOUT == 2)
        process1d<F32, RNE>(blk, p, q, stage);
    else
        process<F32, RNE, LAYOUT == 1 ? 64 : LAYOUT == 3 ? 16 : LAYOUT == 4 ? 8 : 32>(blk, p, q, stage);
}

template <bool F32, int RNE, bool ALIGNED, int LAYOUT>
hipError_t launch_t(const Quant2dBatch& b, hipStream_t s)
{
    hipLaunchKernelGGL((quant2d_kernel<F32, RNE, ALIGNED, LAYOUT>), dim3(b.first[b.n]), dim3(kThreads), 0, s, b);
    return hipGetLastError();
}

template <bool F32, int RNE, int LAYOUT>
hipError_t launch_a(const Quant2dBatch& b, bool aligned, hipStream_t s)
{
    return aligned ? launch_t<F32, RNE, true, LAYOUT>(b, s) : launch_t<F32, RNE, false, LAYOUT>(b, s);
}

template <bool F32, int RNE>
hipError_t launch_b(const Quant2dBatch& b, bool aligned, int layout, hipStream_t s)
{
    switch (layout) {
    case kLayout1D: return launch_a<F32, RNE, 2>(b, aligned, s);
    case kLayout2D64: return launch_a<F32, RNE, 1>(b, aligned, s);
    case kLayout2D16: return launch_a<F32, RNE, 3>(b, aligned, s);
    case kLayout2D8: return launch_a<F32, RNE, 4>(b, aligned, s);
    default: return launch_a<F32, RNE, 0>(b, aligned, s);
    }
}

} // namespace

int64_t quant2d_regions(int64_t rows_pad, int64_t cols_pad)
{
    return ((rows_pad + kRegion - 1) / kRegion) * ((cols_pad + kRegion - 1) / kRegion);
}

hipError_t launch_quant2d(const Quant2dBatch& b, bool f32, bool rne, bool aligned, int layout, hipStream_t s)
{
    if (f32)
        return rne ? launch_b<true, 1>(b, aligned, layout, s) : launch_b<true, 0>(b, aligned, layout, s);
    return rne ? launch_b<false, 1>(b, aligned, layout, s) : launch_b<false, 0>(b, aligned, layout, s);
}

} // namespace fp4q
