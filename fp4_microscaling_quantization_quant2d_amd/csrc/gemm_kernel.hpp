// Block-scaled MXFP4 / MXFP8 GEMM for gfx950:  C[M x N] = A[M x K] . B[N x K]^T
// with both operands stored contraction-contiguous, fp32 accumulation.
//
// "Stable FP4 Training via Transposition-Invariant Block Quantization",
// Sec. 3 "Application to linear layers": Y = X W^T, dX = dY W, dW = dY^T X.
// With the row plane and the transposed plane of every 2D-quantized tensor,
// all three products take this one form (FWD: X, W rows; DGRAD: dY rows and
// W's transposed plane; WGRAD: the transposed planes of dY and X), so each
// tensor is quantized exactly once.  A 32x32 block shares one scale, which is
// a 1x32 K-block scale repeated over 32 rows -- exactly what the hardware's
// per-lane scale operand consumes, taken straight from the 2D grid (or from
// the grid read transposed).  Sec. 3.2's MXFP8 Q/K operands use the same
// kernel with E4M3 operands and per-row 1x32 scales.
//
// Tiling (CDNA4): a 256-thread workgroup (4 waves, 2x2) computes a 256x256
// tile; each wave owns 128x128 = 4x4 tiles of v_mfma_scale_f32_32x32x64_f8f6f4
// (256 fp32 accumulators per lane).  Operands go from HBM straight into LDS
// with buffer->LDS loads (XOR-swizzled 16-byte chunks, 128 KB of ring):
//   FP4: two slots of 128 K-bytes per row (256 FP4 values) for 256 A rows and
//   256 B rows, so every load instruction fills whole cache lines; each slot
//   is multiplied as two 64-byte half stages while the other slot fills.
//   MXFP8: four slots of 64 K-bytes per row, three in flight.
// The raw buffer range check zero-fills rows and K chunks beyond the
// operand, so the loop has no branches; the tile's scale bytes for its whole
// K range sit in LDS.  An FP4 operand in the 1D activation layout (one scale
// per row and K-block) has 256 rows x K/32 bytes per tile, too many to keep;
// its tiled scale grid streams into a two-slot ring beside the pair ring,
// 2 KB per pair, already in the byte order of the 2D path's per-stage words.
// Tiles are ordered so each XCD walks a contiguous, M-grouped range of the
// tile grid, keeping A/B panels resident in that XCD's L2.
#pragma once

#include "fp4q_launch.hpp"
#include "quant_tile.hpp"

#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

namespace fp4q {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 256, kBN = 256;
constexpr int kThreads = 256;
constexpr int kRowBytes = 64;                       // K bytes per row per stage
constexpr int kTileBytes = kBM * kRowBytes;         // 16 KB per operand per stage
constexpr int kStages = 4;                          // LDS ring depth
constexpr int kStageBytes = 2 * kTileBytes;         // A then B
constexpr int kTileLds = kStages * kStageBytes;     // 128 KB
constexpr uint32_t kOob = 0x80000000u;              // buffer offset that reads as zero
constexpr int kDmaPerStage = 8;                     // buffer->LDS loads per wave per stage
constexpr int kTileCpol = 16;                       // sc1 on the streamed tile loads (default: same time; nt: 16% slower)

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// The other ring slot, at compile time when the slot is known there.
template <int V>
__device__ __forceinline__ std::integral_constant<int, 1 - V> other_slot(std::integral_constant<int, V>)
{
    return {};
}
__device__ __forceinline__ int other_slot(int slot) { return 1 - slot; }

// f(std::integral_constant<int, i>) for i = 0..N-1, unrolled, so i can feed
// instruction immediates.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>()), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>());
}

// Byte offset of 16-byte chunk c of row r inside a stage tile (64-byte
// rows).  The xor key makes any 8 consecutive rows hit 8 distinct 16-byte
// bank groups of a 128-byte window and any 16 consecutive rows 16 distinct
// groups of a 256-byte window, so an MFMA operand fetch (one chunk of 32
// consecutive rows) is conflict-free with 32 or 64 LDS banks.
__device__ __forceinline__ int swz_x(int r) { return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1); }
__device__ __forceinline__ int swz(int r, int c) { return r * kRowBytes + ((c ^ swz_x(r)) << 4); }

// FP4 ring: two slots of 128 K-bytes per row (two 64-byte half stages), so
// that one buffer->LDS instruction fills 8 rows x 128 bytes, i.e. 8 whole
// cache lines.  On MI355X such an instruction streams at twice the rate of
// one covering 16 half lines (16 rows x 64 bytes), measured with every CU
// refilling.  Chunk c of row r sits at 16-byte position c ^ swz2_x(r): any 8
// aligned consecutive rows use 8 distinct positions, and any 16 aligned
// consecutive rows 16 distinct 16-byte groups of a 256-byte window, so the
// MFMA operand fetch (one chunk of 32 consecutive rows) is conflict-free.
constexpr int kPairRowBytes = 2 * kRowBytes;
constexpr int kPairTileBytes = kBM * kPairRowBytes;  // 32 KB per operand and slot
constexpr int kPairB = 2 * kPairTileBytes;           // A slots 0, 1, then B slots 0, 1
static_assert(4 * kPairTileBytes == kTileLds, "two pair slots fill the tile ring");
__device__ __forceinline__ int swz2_x(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz2(int r, int c) { return r * kPairRowBytes + ((c ^ swz2_x(r)) << 4); }

// Scale bytes kept in LDS for the whole K range of a tile: FP4 stores one
// byte per (32-row slab, K-block), MXFP8 one per (row, K-block).  Rows are
// padded so the reads for the two stages prefetched past the end of K stay
// inside the row.
__host__ __device__ __forceinline__ int scale_kb_pad(int kblocks) { return ((kblocks + 3) & ~3) + 12; }
__host__ __device__ __forceinline__ int scale_rows(int fmt) { return fmt == 1 ? kBM / 32 : kBM; }
// LDS ring of a 1D-layout operand's scale chunks: two slots of one pair
// (256 rows x 8 K-blocks).
constexpr int kRing1D = 2 * 2048;

struct Problem {
    const uint8_t* a;
    const uint8_t* b;
    const uint8_t* sa;
    const uint8_t* sb;
    float* c;
    int M, N, K;
    int a_rows, b_rows;   // rows readable from a / b
    int tm, tn;           // tile coordinates
};

// Scale byte of (row, kb) for one operand.  FP4 grids hold one byte per
// square block of side 2^sh (sh = 5 for 32x32, 6 for 64x64): a 64x64 block's
// byte serves both of its 32-row slabs and both of its 32-wide K-blocks.
template <int FMT, bool ST>
__device__ __forceinline__ uint32_t scale_at(const uint8_t* s, int64_t lds, int row, int kb, int sh)
{
    if (FMT == 2)
        return s[(int64_t)row * lds + kb];
    if (ST)
        return s[(int64_t)(kb >> (sh - 5)) * lds + (row >> sh)];
    return s[(int64_t)(row >> sh) * lds + (kb >> (sh - 5))];
}

// Copy the tile's scale bytes for its whole K range into LDS, [slab or
// row][K-block], K-blocks kblocks..kbpad-1 zero.  FP4: thread t covers slab
// t/32 and K-blocks t%32 + 32u; MXFP8: thread t covers row t.  Each thread
// issues its loads for both operands in batches of 8 before storing any, so
// they overlap each other and the tile loads already in flight.
template <int FMT, bool ST>
__device__ __forceinline__ void scale_batch_load(uint32_t (&v)[8], const uint8_t* s, int64_t lds, int row,
                                                 bool row_ok, int kb0, int kstep, int kblocks, int sh)
{
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int kb = kb0 + u * kstep;
        v[u] = (row_ok && kb < kblocks) ? scale_at<FMT, ST>(s, lds, row, kb, sh) : 0u;
    }
}

// LDS byte of K-block kb in an operand's scale area.  FP4 (8 slabs): K-block
// kb = 4q + 2j + h sits at [q][h][slab][j], so for half stage q a lane of MFMA
// lane half h finds the bytes of the wave's four slabs in one 8-byte word,
// slab i's K-step-j byte at byte 2(i%2) + j of dword i/2 -- directly the
// MFMA's scale byte select.  MXFP8: [row][kb].
template <int FMT>
__device__ __forceinline__ int scale_lds_index(int kb)
{
    return FMT == 1 ? (kb >> 2) * 32 + (kb & 1) * 16 + ((kb >> 1) & 1) : kb;
}

template <int FMT>
__device__ __forceinline__ void scale_batch_store(const uint32_t (&v)[8], uint8_t* dst, int kb0, int kstep,
                                                  int kbpad)
{
#pragma unroll
    for (int u = 0; u < 8; ++u)
        if (kb0 + u * kstep < kbpad)
            dst[scale_lds_index<FMT>(kb0 + u * kstep)] = (uint8_t)v[u];
}

// The tile's scale bytes in registers: thread t covers (FP4) slab t/32 and
// K-blocks t%32 + 32u, or (MXFP8) row t, for both operands, in up to two
// batches of 8 loads per operand.  Loading them before the first tile loads
// are issued lets the LDS stores wait for these loads alone.
struct ScaleStage {
    uint32_t va[2][8], vb[2][8];
};

template <int FMT>
__device__ __forceinline__ void scale_geometry(int& r, int& kb0, int& kstep)
{
    const int t = threadIdx.x;
    r = FMT == 1 ? t >> 5 : t;
    kb0 = FMT == 1 ? t & 31 : 0;
    kstep = FMT == 1 ? 32 : 1;
}

template <int FMT, bool A_ST, bool B_ST, bool A1D, bool B1D>
__device__ __forceinline__ void scales_load(ScaleStage& st, const GemmArgs& g, const Problem& P, int m0, int n0,
                                            int kblocks, int kbpad)
{
    int r, kb0, kstep;
    scale_geometry<FMT>(r, kb0, kstep);
    const int ra = m0 + (FMT == 1 ? 32 * r : r), rb = n0 + (FMT == 1 ? 32 * r : r);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int k = kb0 + b * 8 * kstep;
        if constexpr (!A1D)
            scale_batch_load<FMT, A_ST>(st.va[b], P.sa, g.lds_a, ra, ra < P.a_rows && k < kbpad, k, kstep, kblocks,
                                        g.sh_a);
        if constexpr (!B1D)
            scale_batch_load<FMT, B_ST>(st.vb[b], P.sb, g.lds_b, rb, rb < P.b_rows && k < kbpad, k, kstep, kblocks,
                                        g.sh_b);
    }
}

// Stores the batches loaded by scales_load, then loads and stores any
// K-blocks beyond them.
template <int FMT, bool A_ST, bool B_ST, bool A1D, bool B1D>
__device__ __forceinline__ void scales_store(const ScaleStage& st, const GemmArgs& g, const Problem& P,
                                             uint8_t* sla, uint8_t* slb, int m0, int n0, int kblocks, int kbpad)
{
    int r, kb0, kstep;
    scale_geometry<FMT>(r, kb0, kstep);
    uint8_t* da = FMT == 1 ? sla + 2 * r : sla + r * kbpad;
    uint8_t* db = FMT == 1 ? slb + 2 * r : slb + r * kbpad;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        if constexpr (!A1D)
            scale_batch_store<FMT>(st.va[b], da, kb0 + b * 8 * kstep, kstep, kbpad);
        if constexpr (!B1D)
            scale_batch_store<FMT>(st.vb[b], db, kb0 + b * 8 * kstep, kstep, kbpad);
    }
    if constexpr (A1D && B1D)
        return;
    const int ra = m0 + (FMT == 1 ? 32 * r : r), rb = n0 + (FMT == 1 ? 32 * r : r);
    for (int k = kb0 + 16 * kstep; k < kbpad; k += 8 * kstep) {
        uint32_t va[8], vb[8];
        if constexpr (!A1D)
            scale_batch_load<FMT, A_ST>(va, P.sa, g.lds_a, ra, ra < P.a_rows, k, kstep, kblocks, g.sh_a);
        if constexpr (!B1D)
            scale_batch_load<FMT, B_ST>(vb, P.sb, g.lds_b, rb, rb < P.b_rows, k, kstep, kblocks, g.sh_b);
        if constexpr (!A1D)
            scale_batch_store<FMT>(va, da, k, kstep, kbpad);
        if constexpr (!B1D)
            scale_batch_store<FMT>(vb, db, k, kstep, kbpad);
    }
}

// Operands in 16x16 (SUB = 2) or 8x8 (SUB = 4) blocks.  The block-scaled
// MFMA takes one scale per lane (row) and 32 K values, so each 32-K MFMA
// becomes SUB MFMAs whose A operand keeps one 32/SUB-wide sub-block of its
// codes (the others zero) and whose scale bytes are that sub-block's: every
// product is formed with its own blocks' scales, exactly.  A lane's row
// lies in row-group row / (32/SUB) of each operand grid.  The tile's bytes
// for its K range sit in LDS ordered
//   [h][wm][lsub][khalf][mi][j][s]     (per operand; wm: the wave-row half of
//                                       the 256 rows, lsub = (row % 32) / b,
//                                       mi: 32-row slab, j: K-step,
//                                       s: sub-block of the K-block)
// so that a lane reads the bytes of its four slabs for one half stage h with
// one (SUB = 2) or two (SUB = 4) 16-byte LDS reads, each byte directly an
// MFMA scale-byte select.  Half stages past K must not hold 0xFF (E8M0 NaN
// would poison zero products), so every byte of the used half stages is
// written (0 past the operand).
template <int SUB>
__host__ __device__ __forceinline__ int sub_half_bytes() { return 32 * SUB * SUB; }
template <int SUB>
__host__ __device__ __forceinline__ int sub_scale_bytes(int K) { return ((K + 127) / 128 + 2) * sub_half_bytes<SUB>(); }

template <int SUB, bool ST>
__device__ __forceinline__ void sub_scales_stage(const uint8_t* src, int64_t ld, int rg0, int rg_valid, int ks_valid,
                                                 int nh, uint8_t* dst)
{
    constexpr int kB = 32 / SUB;             // block side
    constexpr int kNRG = 256 / kB;           // row-groups of the tile
    const int nks = nh * 4 * SUB;            // sub-blocks of the used half stages
    const int total = kNRG * nks;
    for (int base = 0; base < total; base += 8 * kThreads) {
        uint32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int idx = base + u * kThreads + (int)threadIdx.x;
            const int rg = ST ? idx % kNRG : idx / nks, ks = ST ? idx / kNRG : idx % nks;
            v[u] = idx < total && rg0 + rg < rg_valid && ks < ks_valid
                       ? (ST ? src[(int64_t)ks * ld + rg0 + rg] : src[(int64_t)(rg0 + rg) * ld + ks])
                       : 0u;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int idx = base + u * kThreads + (int)threadIdx.x;
            if (idx >= total)
                continue;
            const int rg = ST ? idx % kNRG : idx / nks, ks = ST ? idx / kNRG : idx % nks;
            const int kb = ks / SUB, sb = ks % SUB;
            const int h = kb >> 2, j = (kb >> 1) & 1, kh = kb & 1;
            const int wmh = rg / (4 * SUB), rem = rg % (4 * SUB), mi = rem / SUB, lsub = rem % SUB;
            dst[h * sub_half_bytes<SUB>() + ((((wmh * SUB + lsub) * 2 + kh) * 4 + mi) * 2 + j) * SUB + sb] =
                (uint8_t)v[u];
        }
    }
}

// Wait until at most N buffer->LDS loads of this wave are outstanding, then
// meet the other waves.  The empty asm statements keep the compiler from
// moving LDS accesses across the barrier.
template <int N>
__device__ __forceinline__ void wait_vm_and_barrier()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
    asm volatile("s_barrier" ::: "memory");
}

// KT: K may end inside an FP4 pair (K % 256 != 0), so loads check the K
// range; without it only pairs past the end of K (loaded but never
// multiplied) may read past a row's K bytes.
// ONED: bit 0 -- A is an FP4 operand in the 1D activation layout, bit 1 -- B.
// ACC: C += A B^T (C is read in the epilogue) instead of C = A B^T.
// OBF: C is bf16 (each fp32 sum rounded to nearest even), ldc in bf16 elements.
// QEP: the epilogue quantizes C into 2D 32x32 FP4 planes (the q_* fields of
// GemmArgs) instead of writing C.
// SUB: operands in (32/SUB)x(32/SUB) blocks (2: 16x16, 4: 8x8; FP4, dense).
// MSKIP: a wave skips the MFMAs of its 32-row blocks that lie wholly past
// row M (their sums are never stored), so the last, mostly empty row tile
// of an expert segment costs the MFMA time of its valid blocks only.
template <int FMT, bool A_ST, bool B_ST, bool KT, int ONED, bool ACC = false, bool OBF = false, bool QEP = false,
          int SUB = 1, bool MSKIP = false>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, const Problem& P)
{
    constexpr bool A1D = FMT == 1 && (ONED & 1), B1D = FMT == 1 && (ONED & 2);
    constexpr int kS1D = 2 * ((int)A1D + (int)B1D);  // 1D scale loads per wave and pair
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = P.tm * kBM, n0 = P.tn * kBN;
    const int kbytes = FMT == 1 ? P.K / 2 : P.K;    // K bytes per row
    const int nst = (kbytes + kRowBytes - 1) / kRowBytes;
    const int kblocks = P.K / 32;
    const int kbpad = scale_kb_pad(kblocks);
    uint8_t* sla = lds + kTileLds;
    uint8_t* slb = sla + (SUB > 1 ? sub_scale_bytes<SUB>(P.K) : A1D ? kRing1D : scale_rows(FMT) * kbpad);

    // Buffer->LDS loads.  One instruction of a wave fills 1 KB of LDS, lane l
    // at byte 16*l; wave w issues instructions 4w..4w+3 of each operand tile,
    // so lane l of instruction i lands on tile row r = 16i + l/4, LDS chunk
    // l%4.  To realize the swizzle the lane fetches global chunk
    // (l%4) ^ swz_x(r) of that row.  Rows past the operand and chunks past K
    // read as zero (raw buffer range check), so every stage issues exactly
    // kDmaPerStage loads per wave and vmcnt counts stay uniform.
    const __amdgpu_buffer_rsrc_t rA =
        __builtin_amdgcn_make_buffer_rsrc((void*)P.a, (short)0, (int)((int64_t)P.a_rows * g.lda), 0x00020000);
    const __amdgpu_buffer_rsrc_t rB =
        __builtin_amdgcn_make_buffer_rsrc((void*)P.b, (short)0, (int)((int64_t)P.b_rows * g.ldb), 0x00020000);
    uint32_t offA[4], offB[4];
    int lchunk[4];
    if (FMT == 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = 16 * (4 * wave + q) + (lane >> 2);
            const int c = (lane & 3) ^ swz_x(r);
            lchunk[q] = c;
            const int ar = m0 + r, br = n0 + r;
            offA[q] = ar < P.a_rows ? (uint32_t)(ar * g.lda + c * 16) : kOob;
            offB[q] = br < P.b_rows ? (uint32_t)(br * g.ldb + c * 16) : kOob;
        }
    }
    // FP4 pair loads: wave w fills rows 64w..64w+63 of each operand tile with
    // 8 instructions; lane l of instruction q lands on row
    // r = 64w + 8q + l/8, LDS position l%8, and fetches global chunk
    // (l%8) ^ swz2_x(r) = (l%8) ^ (l/8) ^ (q%2) of the pair.  Rows past the
    // operand lie past the buffer's end and read as zero.
    uint32_t pbA[2], pbB[2];
    int pchunk[2];
    if (FMT == 1) {
        pchunk[0] = (lane & 7) ^ (lane >> 3);
        pchunk[1] = pchunk[0] ^ 1;
        const int r = 64 * wave + (lane >> 3);
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            pbA[par] = (uint32_t)((m0 + r) * g.lda + pchunk[par] * 16);
            pbB[par] = (uint32_t)((n0 + r) * g.ldb + pchunk[par] * 16);
        }
    }
    // 1D scale chunks: pair p needs chunks (2tm + gl, 2p + par) of the tiled
    // grid for gl, par in {0, 1} -- 2 KB, eight 256-byte DMA loads.  Wave w
    // issues two: chunk-row gl = w/2, half stage par = w%2, quarters v = 0, 1;
    // in the ring slot they land at gl*1024 + par*512 + v*256.  Chunks past
    // the K-blocks of the operand, and rows past its groups, read as zero.
    const int nq = (kblocks + 3) >> 2;
    uint32_t s1a = 0, s1b = 0;
    __amdgpu_buffer_rsrc_t rSA = rA, rSB = rB;
    if constexpr (A1D) {
        rSA = __builtin_amdgcn_make_buffer_rsrc((void*)P.sa, (short)0,
                                                (int)((int64_t)((P.a_rows + 127) >> 7) * g.lds_a), 0x00020000);
        s1a = (uint32_t)((2 * P.tm + (wave >> 1)) * g.lds_a + (wave & 1) * 512 + 4 * lane);
    }
    if constexpr (B1D) {
        rSB = __builtin_amdgcn_make_buffer_rsrc((void*)P.sb, (short)0,
                                                (int)((int64_t)((P.b_rows + 127) >> 7) * g.lds_b), 0x00020000);
        s1b = (uint32_t)((2 * P.tn + (wave >> 1)) * g.lds_b + (wave & 1) * 512 + 4 * lane);
    }
    auto issue_scales1d = [&](int p, int wv) {
        const uint32_t far = 2 * p + (wv & 1) >= nq ? kOob : 0u;
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const int dst = (p & 1) * 2048 + (wv >> 1) * 1024 + (wv & 1) * 512 + v * 256;
            if constexpr (A1D)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rSA, LDS_PTR(sla + dst), 4,
                                                         (int)((s1a + (uint32_t)(p * 1024 + v * 256)) | far), 0, 0, 0);
            if constexpr (B1D)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rSB, LDS_PTR(slb + dst), 4,
                                                         (int)((s1b + (uint32_t)(p * 1024 + v * 256)) | far), 0, 0, 0);
        }
    };
    // Loads q of both operands for pair p (128 K-bytes per row) into slot p%2.
    // Load k (0..15) of pair p into slot p%2: instruction k/2 of operand A
    // (k even) or B (k odd).
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // LDS addresses in scalar registers
    // MSKIP: 32-row blocks of this wave holding at least one row below M (0..4)
    const int nmi_s = __builtin_amdgcn_readfirstlane(min(4, max(0, (P.M - m0 - (wave_s >> 1) * 128 + 31) >> 5)));
    auto issue_load = [&](int p, int k) {
        // a pair's 1D scale loads go out just before its first data load, so
        // every wait that covers the pair's data covers them as well
        if (A1D || B1D)
            if (k == 0)
                issue_scales1d(p, wave_s);
        const int q = k >> 1;
        uint8_t* base = lds + (p & 1) * kPairTileBytes + (8 * wave_s + q) * 1024;
        const uint32_t kfar =
            KT && ((uint32_t)(p * kPairRowBytes + pchunk[q & 1] * 16 - kbytes) >> 31) == 0 ? kOob : 0u;
        if ((k & 1) == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rA, LDS_PTR(base), 16, (int)((pbA[q & 1] + (uint32_t)(8 * q * g.lda + p * kPairRowBytes)) | kfar),
                0, 0, kTileCpol);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rB, LDS_PTR(base + kPairB), 16,
                (int)((pbB[q & 1] + (uint32_t)(8 * q * g.ldb + p * kPairRowBytes)) | kfar), 0, 0, kTileCpol);
    };
    auto issue = [&](int s) {
        uint8_t* base = lds + (s % kStages) * kStageBytes + (4 * wave) * 1024;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t kfar = (uint32_t)(s * kRowBytes + lchunk[q] * 16 - kbytes) >> 31 ? 0u : kOob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, LDS_PTR(base + q * 1024), 16,
                                                     (int)((offA[q] + s * kRowBytes) | kfar), 0, 0, kTileCpol);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, LDS_PTR(base + kTileBytes + q * 1024), 16,
                                                     (int)((offB[q] + s * kRowBytes) | kfar), 0, 0, kTileCpol);
        }
    };

    const int lrow32 = lane & 31, khalf = lane >> 5;
    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;

    // FP4 operands of one half stage s in registers: A/B fragments of both
    // MFMA K-steps (16 x 16 bytes; lane half h holds the 32 codes of K-block
    // h of the step) and the scale bytes of the wave's four slabs of A and of
    // B for the lane's K-blocks 4s + 2j + h (layout at scale_lds_index).  The
    // vector types keep the compiler's view of these LDS reads precise, so it
    // adds no waits for the buffer->LDS loads in flight.
    struct Frag {
        v4u a[2][4], b[2][4];
        v2u sa, sb;
        v4u sa2[SUB > 2 ? 2 : 1], sb2[SUB > 2 ? 2 : 1];  // SUB > 1: sub-block scale bytes
    };
    constexpr int kLsubShift = SUB == 4 ? 3 : 4;  // row-group of a lane inside its slab: lrow32 >> shift
    // Half stage h of the FP4 ring: pair h/2 in slot (h/2)%2, chunks 4(h%2)..4(h%2)+3.
    // Fragment (i, j) of a half stage held in slot SLOT, half PAR of its pair
    // (chunks 4 PAR .. 4 PAR + 3).  With SLOT and PAR fixed at compile time the
    // address is a per-lane offset plus an instruction immediate.
    auto half_a = [&](int slot, int par, int i, int j) {
        return *reinterpret_cast<const v4u*>(lds + slot * kPairTileBytes +
                                             swz2(wm * 128 + i * 32 + lrow32, 4 * par + 2 * j + khalf));
    };
    auto half_b = [&](int slot, int par, int i, int j) {
        return *reinterpret_cast<const v4u*>(lds + kPairB + slot * kPairTileBytes +
                                             swz2(wn * 128 + i * 32 + lrow32, 4 * par + 2 * j + khalf));
    };
    // LDS reads of half h (in slot SLOT, half PAR of its pair) into N, in the
    // order the next half consumes them: the scale words, then K-step 0's
    // fragments (a0, b0..b3, a1..a3), then K-step 1's likewise.  Item e of 18.
    auto read_item = [&](int h, auto SLOT, auto PAR, int e, Frag& N) {
        const int slot = SLOT, par = PAR;  // compile-time constants or (the slot) a uniform value
        if (SUB > 1 && e < 2) {
            // this lane's sub-block scale bytes of its four slabs, half h
            uint8_t* base = (e == 0 ? sla : slb) + h * sub_half_bytes<SUB>() +
                            (((e == 0 ? wm : wn) * SUB + (lrow32 >> kLsubShift)) * 2 + khalf) * (8 * SUB);
            v4u* d = e == 0 ? N.sa2 : N.sb2;
#pragma unroll
            for (int q = 0; q < (SUB > 2 ? 2 : 1); ++q)
                d[q] = *reinterpret_cast<const v4u*>(base + 16 * q);
        } else if (e == 0) {
            if constexpr (A1D)
                N.sa = *reinterpret_cast<const v2u*>(sla + slot * 2048 + wm * 1024 + par * 512 + khalf * 256 +
                                                     lrow32 * 8);
            else
                N.sa = *reinterpret_cast<const v2u*>(sla + h * 32 + khalf * 16 + wm * 8);
        } else if (e == 1) {
            if constexpr (B1D)
                N.sb = *reinterpret_cast<const v2u*>(slb + slot * 2048 + wn * 1024 + par * 512 + khalf * 256 +
                                                     lrow32 * 8);
            else
                N.sb = *reinterpret_cast<const v2u*>(slb + h * 32 + khalf * 16 + wn * 8);
        } else {
            const int j = (e - 2) >> 3, k = (e - 2) & 7;
            if (k == 0)
                N.a[j][0] = half_a(slot, par, 0, j);
            else if (k <= 4)
                N.b[j][k - 1] = half_b(slot, par, k - 1, j);
            else
                N.a[j][k - 4] = half_a(slot, par, k - 4, j);
        }
    };
    auto load_frags0 = [&](Frag& F) {
#pragma unroll
        for (int e = 0; e < 18; ++e)
            read_item(0, std::integral_constant<int, 0>(), std::integral_constant<int, 0>(), e, F);
    };

    auto scale_f32 = [](uint32_t b) {
        // 2^(b-127); b = 0 is the fp32 subnormal 2^-127
        return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
    };
    auto mma_fp8 = [&](int s) {
        const uint8_t* la = lds + (s % kStages) * kStageBytes;
        const uint8_t* lb = la + kTileBytes;
        float ca[4], cb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if ((t & 1) == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ca[i] = scale_f32(sla[(wm * 128 + i * 32 + lrow32) * kbpad + 2 * s + (t >> 1)]);
                    cb[i] = scale_f32(slb[(wn * 128 + i * 32 + lrow32) * kbpad + 2 * s + (t >> 1)]);
                }
            }
            v8bf fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint2 ra = *reinterpret_cast<const uint2*>(la + swz(wm * 128 + i * 32 + lrow32, t) + 8 * khalf);
                const uint2 rb = *reinterpret_cast<const uint2*>(lb + swz(wn * 128 + i * 32 + lrow32, t) + 8 * khalf);
                const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ra.x, ca[i], false);
                const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ra.x, ca[i], true);
                const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ra.y, ca[i], false);
                const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ra.y, ca[i], true);
                const bf16x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(rb.x, cb[i], false);
                const bf16x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(rb.x, cb[i], true);
                const bf16x2 b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(rb.y, cb[i], false);
                const bf16x2 b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(rb.y, cb[i], true);
                fa[i] = __builtin_bit_cast(v8bf, (v4u){__builtin_bit_cast(uint32_t, a0), __builtin_bit_cast(uint32_t, a1),
                                                      __builtin_bit_cast(uint32_t, a2), __builtin_bit_cast(uint32_t, a3)});
                fb[i] = __builtin_bit_cast(v8bf, (v4u){__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1),
                                                      __builtin_bit_cast(uint32_t, b2), __builtin_bit_cast(uint32_t, b3)});
            }
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
        }
    };

    // FP4 half-stage bodies.  The 32 MFMAs held in C run as 8 groups of 4
    // (K-step j, A fragment mi, all four B fragments); the memory work of the
    // half is placed between the groups, and the scheduling barriers keep
    // that mix so the matrix unit never waits behind a burst of memory
    // instructions.
    // MFMAs lo..hi-1 of group G (K-step j = G/4, A fragment mi = G%4, B
    // fragments ni); a group's refill load goes between its second and third
    // MFMA (measured ~2% faster than after the fourth).
    auto mfma_group = [&](const Frag& C, auto G, int lo, int hi) {
        constexpr int j = decltype(G)::value >> 2, mi = decltype(G)::value & 3;
        if constexpr (SUB > 1) {
            // SUB MFMAs per (mi, ni): A keeps sub-block s of its 32 codes
            // (dwords 2s, 2s+1 for 16-wide blocks, dword s for 8-wide), and
            // both operands take sub-block s's scale bytes
            static_for<4>([&](auto NI) {
                constexpr int ni = decltype(NI)::value;
                if (ni < lo || ni >= hi) return;
                const v4u xa = C.a[j][mi], xb = C.b[j][ni];
                const v8i fb = v8i{(int)xb.x, (int)xb.y, (int)xb.z, (int)xb.w, 0, 0, 0, 0};
                static_for<SUB>([&](auto S) {
                    constexpr int sb = decltype(S)::value;
                    v8i fa = v8i{0, 0, 0, 0, 0, 0, 0, 0};
                    if constexpr (SUB == 2) {
                        fa[2 * sb] = (int)xa[2 * sb];
                        fa[2 * sb + 1] = (int)xa[2 * sb + 1];
                        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fa, fb, acc[mi][ni], 4, 4, 2 * j + sb, (int)C.sa2[0][mi], 2 * j + sb, (int)C.sb2[0][ni]);
                    } else {
                        fa[sb] = (int)xa[sb];
                        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fa, fb, acc[mi][ni], 4, 4, sb, (int)C.sa2[mi >> 1][(mi & 1) * 2 + j], sb,
                            (int)C.sb2[ni >> 1][(ni & 1) * 2 + j]);
                    }
                });
            });
            return;
        }
        if constexpr (MSKIP)
            if (mi >= nmi_s)
                return;
        const int ssa = (int)(mi >> 1 ? C.sa.y : C.sa.x);
        static_for<4>([&](auto NI) {
            constexpr int ni = decltype(NI)::value;
            if (ni < lo || ni >= hi) return;
            const int ssb = (int)(ni >> 1 ? C.sb.y : C.sb.x);
            const v4u xa = C.a[j][mi], xb = C.b[j][ni];
            const v8i fa = v8i{(int)xa.x, (int)xa.y, (int)xa.z, (int)xa.w, 0, 0, 0, 0};
            const v8i fb = v8i{(int)xb.x, (int)xb.y, (int)xb.z, (int)xb.w, 0, 0, 0, 0};
            // slab i's K-step-j scale: byte 2(i%2) + j of dword i/2
            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fa, fb, acc[mi][ni], 4, 4, 2 * (mi & 1) + j, ssa, 2 * (ni & 1) + j, ssb);
        });
    };
    // Quarter u (0..3) of the reads of half h: items [kq[u], kq[u+1]).
    auto read_quarter = [&](int h, auto SLOT, auto PAR, int u, Frag& N) {
        constexpr int kq[5] = {0, 5, 9, 14, 18};
#pragma unroll
        for (int e = kq[u]; e < kq[u + 1]; ++e)
            read_item(h, SLOT, PAR, e, N);
    };
    // The two halves of pair P.  Every group issues one 1 KB load, so each
    // pair streams in over 16 groups: pair P+1's loads 12..15 in the even
    // half's first four groups, pair P+2's loads 0..3 in its last four (slot
    // P%2 is free from the even half's barrier on) and 4..11 in the odd half.
    // LOADS: 2 with both pairs, 1 with pair P+1 only (P+2 is past K), 0 none.
    //   Even half 2P (C): the first four groups read half 2P+1 (the rest of
    //   pair P) into N; then every wave is done with slot P%2.
    //   Odd half 2P+1 (C): after four groups each wave waits for its loads of
    //   pair P+1 (pair P+2's eight may stay outstanding), the barrier
    //   publishes pair P+1, and the last four groups read its first half
    //   into N.
    // SLOT: P%2, the slot of pair P, a compile-time constant where the loop
    // is unrolled over two pairs, else a uniform value.
    auto half_even = [&](auto loads, auto SLOT, int h_next, int p, const Frag& C, Frag& N) {
        constexpr int L = decltype(loads)::value;
        static_for<8>([&](auto G) {
            constexpr int g8 = decltype(G)::value;
            mfma_group(C, G, 0, 2);
            __builtin_amdgcn_sched_barrier(0);
            if (g8 < 4) {
                if constexpr (L >= 1)
                    issue_load(p + 1, 12 + g8);
            }
            if constexpr (L == 2)
                if (g8 >= 4)
                    issue_load(p + 2, g8 - 4);
            __builtin_amdgcn_sched_barrier(0);
            mfma_group(C, G, 2, 4);
            if (g8 < 4)
                read_quarter(h_next, SLOT, std::integral_constant<int, 1>(), g8, N);
            if (g8 == 3)
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    auto half_odd = [&](auto loads, auto SLOT, int h_next, int p, const Frag& C, Frag& N) {
        const auto next_slot = other_slot(SLOT);
        constexpr int L = decltype(loads)::value;
        static_for<8>([&](auto G) {
            constexpr int g8 = decltype(G)::value;
            mfma_group(C, G, 0, 2);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (L == 2)
                issue_load(p + 2, 4 + g8);
            __builtin_amdgcn_sched_barrier(0);
            mfma_group(C, G, 2, 4);
            if (g8 == 3) {
                if constexpr (L == 2)
                    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(8 + kS1D) : "memory");
                else
                    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
            }
            if (g8 >= 4)
                read_quarter(h_next, next_slot, std::integral_constant<int, 0>(), g8 - 4, N);
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // Pipelines.  The first stages (FP4: pairs 0 and 1) and the scale bytes
    // are loaded up front.
    //   FP4: half stages h = 0, 1, ... of 64 K-bytes; pair h/2 lives in slot
    //   (h/2)%2.  While half h is multiplied from registers, half h+1 is read
    //   out of LDS into the other register set.  An even half's successor is
    //   in its own pair, so it runs without waiting.  Before an odd half h+1
    //   each wave waits for its loads of pair h/2+1 and for its LDS reads; the
    //   barrier then publishes that pair and guarantees that every wave is
    //   done with pair h/2, whose slot the odd half refills with pair h/2+2.
    //   MXFP8: a 4-slot ring of 64-byte stages, three in flight.
    const int npair = (kbytes + kPairRowBytes - 1) / kPairRowBytes;
    if constexpr (SUB > 1) {
        // operand loads of pairs 0 and 1 first; the scale bytes are staged
        // while they fly (the waits the compiler adds for the byte loads also
        // cover them)
#pragma unroll
        for (int k = 0; k < 16; ++k)
            issue_load(0, k);
#pragma unroll
        for (int k = 0; k < 12; ++k)
            issue_load(1, k);
        constexpr int kB = 32 / SUB;
        const int nh = (P.K + 127) / 128;
        sub_scales_stage<SUB, A_ST>(P.sa, g.lds_a, m0 / kB, P.a_rows / kB, P.K / kB, nh, sla);
        sub_scales_stage<SUB, B_ST>(P.sb, g.lds_b, n0 / kB, P.b_rows / kB, P.K / kB, nh, slb);
    } else {
        ScaleStage st;
        scales_load<FMT, A_ST, B_ST, A1D, B1D>(st, g, P, m0, n0, kblocks, kbpad);
        __builtin_amdgcn_sched_barrier(0);
        if (FMT == 1) {
#pragma unroll
            for (int k = 0; k < 16; ++k)
                issue_load(0, k);
#pragma unroll
            for (int k = 0; k < 12; ++k)
                issue_load(1, k);
        } else {
            issue(0);
            issue(1);
            issue(2);
        }
        __builtin_amdgcn_sched_barrier(0);
        scales_store<FMT, A_ST, B_ST, A1D, B1D>(st, g, P, sla, slb, m0, n0, kblocks, kbpad);
    }
    // Stage 0 and the scale bytes must be in LDS; the later stages may still
    // be in flight.
    if (FMT == 1)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(12 + kS1D) : "memory");
    else
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * kDmaPerStage) : "memory");
    int s = 0;
    if (FMT == 1) {
        Frag F0, F1;
        load_frags0(F0);
        // Every pair issues the loads of the two pairs after it; loads of
        // pairs past the end of K read as zero or are never multiplied, so
        // the body is the same for every pair.
        const std::integral_constant<int, 2> both;
        const std::integral_constant<int, 0> none;
        int p = 0;
        if constexpr (!KT) {
            // Whole pairs only: two pairs per iteration fix each half's slot
            // at compile time, then at most one more pair, in slot 0.
            const std::integral_constant<int, 0> slot0;
            const std::integral_constant<int, 1> slot1;
            for (; 2 * p + 3 < nst; p += 2) {
                half_even(both, slot0, 2 * p + 1, p, F0, F1);
                half_odd(both, slot0, 2 * p + 2, p, F1, F0);
                half_even(both, slot1, 2 * p + 3, p + 1, F0, F1);
                half_odd(both, slot1, 2 * p + 4, p + 1, F1, F0);
            }
            if (2 * p + 1 < nst) {
                half_even(both, slot0, 2 * p + 1, p, F0, F1);
                half_odd(both, slot0, 2 * p + 2, p, F1, F0);
            }
        } else {
            for (; 2 * p + 1 < nst; ++p) {
                half_even(both, p & 1, 2 * p + 1, p, F0, F1);
                half_odd(both, p & 1, 2 * p + 2, p, F1, F0);
            }
            if (2 * p < nst)  // odd count: the last half (its successor reads are unused)
                half_even(none, p & 1, 2 * p + 1, p, F0, F1);
        }
    } else {
        // MXFP8: products are formed exactly.  Each 16-wide K step, a lane
        // converts its 8 E4M3 bytes (row lane%32, K bytes [16t + 8h, +8)) to
        // bf16 with its row's E8M0 scale folded in -- exact, E4M3 has 4
        // significant bits -- and the bf16 MFMA accumulates in fp32.  (The
        // block-scaled FP8 MFMA rounds inside its dot product, ~1e-4 of
        // sum |a||b| on full-range E4M3, so it is not used here.)
        for (; s < nst; ++s) {
            if (s > 0)
                wait_vm_and_barrier<(kStages - 2) * kDmaPerStage>();
            issue(s + kStages - 1);
            mma_fp8(s);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // epilogue: lane holds C[8(r/4) + 4(lane/32) + r%4][lane%32] of each 32x32 tile.
    // C is written non-temporally: the fp32 output streams to memory while
    // the kernel runs instead of staying dirty in the caches for the next
    // kernel to write back.  Every store instruction covers two full 128-byte
    // row segments.  Interior tiles address each store as one per-lane base
    // plus a wave-uniform row offset and a constant column offset.
    if constexpr (QEP) {
        // Quantize-in-epilogue.  Each wave walks its 128x128 sub-tile as four
        // 64-aligned 64x64 quadrants.  A quadrant's four 32x32 accumulator
        // blocks are staged as fp32 in the wave's part of the (now idle)
        // operand ring; each lane then reads back one 8x8 block and runs the
        // 2D quantizer's per-lane steps on it (tile amax over the tile's 16
        // lanes, truncation-free scale, Philox draws keyed by global
        // coordinates, SR or RNE conversion, nibble transpose), so the planes
        // are exactly those the quantizer writes for this fp32 C.
        constexpr int kQPitch = 68;  // floats per staged row
        __syncthreads();             // every wave has finished reading the ring
        float* stg = reinterpret_cast<float*>(lds + wave * (64 * kQPitch * 4));
        uint32_t key0 = g.q_key0, key1 = g.q_key1;
        if (g.q_seed_dev) {
            const uint64_t k = ((uint64_t)key1 << 32 | key0) + *g.q_seed_dev;
            key0 = (uint32_t)k;
            key1 = (uint32_t)(k >> 32);
        }
        const int br = lane >> 3, bc = lane & 7;
        static_for<4>([&](auto QD) {
            constexpr int mp = decltype(QD)::value >> 1, np = decltype(QD)::value & 1;
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        stg[(a * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3)) * kQPitch + b * 32 + lrow32] =
                            acc[2 * mp + a][2 * np + b][r];
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave reads back only its own writes
            qtile::Block8x8<true> blk;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const v4u lo = *reinterpret_cast<const v4u*>(stg + (8 * br + i) * kQPitch + 8 * bc);
                const v4u hi = *reinterpret_cast<const v4u*>(stg + (8 * br + i) * kQPitch + 8 * bc + 4);
                blk.v[i][0] = lo.x; blk.v[i][1] = lo.y; blk.v[i][2] = lo.z; blk.v[i][3] = lo.w;
                blk.v[i][4] = hi.x; blk.v[i][5] = hi.y; blk.v[i][6] = hi.z; blk.v[i][7] = hi.w;
            }
            const int r0w = m0 + wm * 128 + mp * 64, c0w = n0 + wn * 128 + np * 64;
            const int R0 = r0w + 8 * br, C0 = c0w + 8 * bc;
            const bool active = R0 < g.q_rows_pad && C0 < g.q_cols_pad;
            const uint32_t mx = qtile::square_amax<32>(active ? qtile::block_amax<true>(blk) : 0u);
            if (active) {
                const int k = truncfree_exp_e2m1(mx);
                uint32_t rw[8];
                if (g.q_rne)
                    qtile::round_lane_block<true, 1>(blk, k, R0, C0, r0w, c0w, g.q_stream, key0, key1, rw);
                else
                    qtile::round_lane_block<true, 0>(blk, k, R0, C0, r0w, c0w, g.q_stream, key0, key1, rw);
                if (qtile::block_leader<32>(lane))
                    g.q_scales[(int64_t)(R0 >> 5) * g.q_ld_s + (C0 >> 5)] = (uint8_t)(k + 127);
                uint8_t* cr = g.q_codes + (int64_t)R0 * g.q_ld + (C0 >> 1);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    *reinterpret_cast<uint32_t*>(cr + i * g.q_ld) = rw[i];
                if (g.q_codes_t) {
                    nibble_transpose8(rw);
                    uint8_t* ct = g.q_codes_t + (int64_t)C0 * g.q_ld_t + (R0 >> 1);
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        *reinterpret_cast<uint32_t*>(ct + j * g.q_ld_t) = rw[j];
                }
            }
        });
        return;
    }
    if constexpr (OBF) {
        // bf16 output.  A lane holds one column of each 32x32 block, so direct
        // 2-byte stores would write half lines; instead each wave stages its
        // 128x128 bf16 sub-tile in its 32 KB of the (now idle) operand ring
        // and writes whole 128-byte lines with 16-byte stores.  Rows 4..7 of
        // every 8 are XOR-shifted by 64 bytes so the two lane halves' LDS
        // writes fall in different banks.
        __syncthreads();  // every wave has finished reading the ring
        uint8_t* st = lds + wave * (128 * 256);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = mi * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
                    const int cb = (ni * 32 + lrow32) * 2;
                    *reinterpret_cast<__bf16*>(st + row * 256 + (cb ^ (((row >> 2) & 1) << 6))) =
                        (__bf16)acc[mi][ni][r];
                }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave reads back only its own rows
        __bf16* ch = reinterpret_cast<__bf16*>(P.c);
        const int rbase = m0 + wm * 128, cbase = n0 + wn * 128;
        const bool vec = m0 + kBM <= P.M && n0 + kBN <= P.N && (g.ldc & 7) == 0 &&
                         (reinterpret_cast<uintptr_t>(P.c) & 15) == 0;
        const int k = lane & 15;
#pragma unroll 4
        for (int it = 0; it < 32; ++it) {
            const int row = it * 4 + (lane >> 4);
            const v4u v = *reinterpret_cast<const v4u*>(st + row * 256 + ((k * 16) ^ (((row >> 2) & 1) << 6)));
            __bf16* dst = ch + (int64_t)(rbase + row) * g.ldc + cbase + 8 * k;
            if (vec) {
                __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(dst));
            } else if (rbase + row < P.M) {
                const __bf16* e = reinterpret_cast<const __bf16*>(&v);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (cbase + 8 * k + j < P.N)
                        dst[j] = e[j];
            }
        }
        return;
    }
    if (m0 + kBM <= P.M && n0 + kBN <= P.N) {
        // The store phases of all CUs coincide, and tiles otherwise write
        // the same relative rows at the same moment; for leading dimensions
        // near powers of two those writes crowd the same memory channels.
        // Each tile therefore starts at 32-row block (tm + tn) % 4 of its
        // wave's quarter (measured 7-9% faster for N = 4096 outputs, 3% for
        // N = 11008, like padding the rows of C).
        float* cb = P.c + (int64_t)(m0 + wm * 128 + 4 * khalf) * g.ldc + (n0 + wn * 128 + lrow32);
        auto store_from = [&](auto ROT) {
            static_for<4>([&](auto B) {
                constexpr int mi = (decltype(B)::value + decltype(ROT)::value) & 3;
                if constexpr (ACC) {
                    // C += A B^T: all 64 old values of the 32-row block are
                    // loaded before any sum is stored (the operand registers
                    // are free by now), so a block costs one memory round
                    // trip.  Loading the next block's values before these
                    // stores measured the same: the cost is the extra read.
                    float old[16][4];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float* rp = cb + (int64_t)(mi * 32 + 8 * (r >> 2) + (r & 3)) * g.ldc;
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni)
                            old[r][ni] = __builtin_nontemporal_load(rp + ni * 32);
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float* rp = cb + (int64_t)(mi * 32 + 8 * (r >> 2) + (r & 3)) * g.ldc;
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni)
                            __builtin_nontemporal_store(acc[mi][ni][r] + old[r][ni], rp + ni * 32);
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float* rp = cb + (int64_t)(mi * 32 + 8 * (r >> 2) + (r & 3)) * g.ldc;
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni)
                            __builtin_nontemporal_store(acc[mi][ni][r], rp + ni * 32);
                    }
                }
            });
        };
        switch ((P.tm + P.tn) & 3) {
        case 0: store_from(std::integral_constant<int, 0>()); break;
        case 1: store_from(std::integral_constant<int, 1>()); break;
        case 2: store_from(std::integral_constant<int, 2>()); break;
        default: store_from(std::integral_constant<int, 3>()); break;
        }
        return;
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const int col = n0 + wn * 128 + ni * 32 + lrow32;
            if (col >= P.N)
                continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 128 + mi * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
                if (row < P.M) {
                    float* cp = &P.c[(int64_t)row * g.ldc + col];
                    if constexpr (ACC)
                        __builtin_nontemporal_store(acc[mi][ni][r] + __builtin_nontemporal_load(cp), cp);
                    else
                        __builtin_nontemporal_store(acc[mi][ni][r], cp);
                }
            }
        }
    }
}

// Workgroup `id` of a 1-D grid runs on XCD id % 8.  Tile xcd_tile(id, n)
// gives XCD x the contiguous tile range [x*q + min(x, r), ..) of n = 8q + r
// tiles (a bijection on [0, n)), so consecutive tiles, which share operand
// panels (a band of one product, an expert's tiles), meet in one XCD's L2.
__device__ __forceinline__ int xcd_tile(int id, int n)
{
    const int x = id & 7, q = n >> 3, r = n & 7;
    return x * q + min(x, r) + (id >> 3);
}

// Tile order: each XCD (dispatch id mod 8) receives a contiguous range of
// tile ids; inside it tiles are M-grouped in bands of BAND tile rows.  FP4
// takes 4 (1% faster on the 7B step than 8 or 2; 16 slower), the batched
// MXFP8 S = QK^T 8 (1% faster there than 4).
template <int BAND>
__device__ __forceinline__ void tile_of(int pid, int ntm, int ntn, int& tm, int& tn)
{
    constexpr int kBandRows = BAND;
    const int nt = ntm * ntn;
    pid = xcd_tile(pid, nt);
    const int band = kBandRows * ntn;
    const int first = (pid / band) * kBandRows;
    const int rows = min(ntm - first, kBandRows);
    const int in = pid - (pid / band) * band;
    tm = first + in % rows;
    tn = in / rows;
}

template <int FMT, bool A_ST, bool B_ST, bool KT, int ONED, bool ACC, bool OBF>
__global__ __launch_bounds__(kThreads, 1) void gemm_dense_kernel(GemmArgs g)
{
    const int bz = blockIdx.y;
    Problem P;
    P.a = g.a + bz * g.bs_a;
    P.b = g.b + bz * g.bs_b;
    P.sa = g.sa + bz * g.bs_sa;
    P.sb = g.sb + bz * g.bs_sb;
    P.c = OBF ? reinterpret_cast<float*>(reinterpret_cast<__bf16*>(g.c) + bz * g.bs_c) : g.c + bz * g.bs_c;
    P.M = g.M;
    P.N = g.N;
    P.K = g.K;
    P.a_rows = g.a_rows;
    P.b_rows = g.b_rows;
    const int ntm = (g.M + kBM - 1) / kBM, ntn = (g.N + kBN - 1) / kBN;
    tile_of<FMT == 1 ? 4 : 8>(blockIdx.x, ntm, ntn, P.tm, P.tn);
    gemm_tile<FMT, A_ST, B_ST, KT, ONED, ACC, OBF>(g, P);
}

// Dense product whose epilogue quantizes C (QEP); batch 1.
template <bool A_ST, bool B_ST, bool KT>
__global__ __launch_bounds__(kThreads, 1) void gemm_quant_kernel(GemmArgs g)
{
    Problem P;
    P.a = g.a;
    P.b = g.b;
    P.sa = g.sa;
    P.sb = g.sb;
    P.c = nullptr;
    P.M = g.M;
    P.N = g.N;
    P.K = g.K;
    P.a_rows = g.a_rows;
    P.b_rows = g.b_rows;
    const int ntm = (g.M + kBM - 1) / kBM, ntn = (g.N + kBN - 1) / kBN;
    tile_of<4>(blockIdx.x, ntm, ntn, P.tm, P.tn);
    gemm_tile<1, A_ST, B_ST, KT, 0, false, false, true>(g, P);
}

// Dense product of operands in 16x16 (SUB = 2) or 8x8 (SUB = 4) blocks;
// batch 1.  ACC: C += A B^T (the host splits long contractions into chunks
// that accumulate).
template <int SUB, bool A_ST, bool B_ST, bool KT, bool ACC>
__global__ __launch_bounds__(kThreads, 1) void gemm_sub_kernel(GemmArgs g)
{
    Problem P;
    P.a = g.a;
    P.b = g.b;
    P.sa = g.sa;
    P.sb = g.sb;
    P.c = g.c;
    P.M = g.M;
    P.N = g.N;
    P.K = g.K;
    P.a_rows = g.a_rows;
    P.b_rows = g.b_rows;
    const int ntm = (g.M + kBM - 1) / kBM, ntn = (g.N + kBN - 1) / kBN;
    tile_of<4>(blockIdx.x, ntm, ntn, P.tm, P.tn);
    gemm_tile<1, A_ST, B_ST, KT, 0, ACC, false, false, SUB>(g, P);
}

// Grouped (expert) products.  Group g owns token rows [row_off[g], row_off[g+1]).
//   FWD:   A = X rows of g,  B = W rows [g*gn, (g+1)*gn),       C rows of g
//   DGRAD: A = dY rows of g, B = W^T plane, K range of expert g, C rows of g
//   WGRAD: A = dY^T, B = X^T planes over the token range of g,  C rows [g*gn, ..)
// DEV: the offsets are in device memory (g.row_off_dev).  Every workgroup
// then builds the group -> tile table itself in LDS: group t's offsets are
// clamped into [0, tok_rows], rounded down to multiples of 32 and made
// non-decreasing pairwise (a WGRAD group also to at most max_rows rows, the
// K its LDS was sized for), so every access stays inside the operands for
// any offsets; workgroups past the last tile exit.
// Element `off` of C, fp32 or (OBF) bf16.
template <bool OBF>
__device__ __forceinline__ float* c_elem(float* c, int64_t off)
{
    return OBF ? reinterpret_cast<float*>(reinterpret_cast<__bf16*>(c) + off) : c + off;
}

template <int OP, bool A_ST, bool B_ST, bool DEV, bool OBF = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_grouped_kernel(GemmArgs g)
{
    int pid = blockIdx.x;
    int grp, r0, r1, local;
    const int ntn_g = ((OP == kGemmFwd ? g.group_n : g.N) + kBN - 1) / kBN;
    if constexpr (DEV) {
        extern __shared__ __attribute__((aligned(16))) uint8_t lds_tab[];
        int* incl = reinterpret_cast<int*>(lds_tab);  // inclusive tile prefix per group
        int* lo_s = incl + kThreads;
        int* hi_s = lo_s + kThreads;
        const int t = threadIdx.x, n = g.n_groups;
        int cnt = 0;
        if (t < n) {
            const int64_t tok = g.tok_rows;
            int64_t a = g.row_off_dev[t], b = g.row_off_dev[t + 1];
            a = (a < 0 ? 0 : (a > tok ? tok : a)) & ~(int64_t)31;
            b = (b < a ? a : (b > tok ? tok : b)) & ~(int64_t)31;
            if (OP == kGemmWgrad && b - a > g.max_rows)
                b = a + g.max_rows;
            lo_s[t] = (int)a;
            hi_s[t] = (int)b;
            cnt = (OP == kGemmWgrad ? (g.group_n + kBM - 1) / kBM : (int)((b - a + kBM - 1) / kBM)) * ntn_g;
        }
        incl[t] = cnt;
        __syncthreads();
        for (int off = 1; off < kThreads; off <<= 1) {
            const int v = t >= off ? incl[t - off] : 0;
            __syncthreads();
            incl[t] += v;
            __syncthreads();
        }
        if (pid >= incl[n - 1])
            return;  // uniform over the workgroup
        pid = xcd_tile(pid, incl[n - 1]);
        int lo = 0, hi = n - 1;  // first group whose inclusive count exceeds pid
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (incl[mid] > pid)
                hi = mid;
            else
                lo = mid + 1;
        }
        grp = lo;
        r0 = lo_s[grp];
        r1 = hi_s[grp];
        local = pid - (grp ? incl[grp - 1] : 0);
        __syncthreads();  // the tile reuses this LDS
    } else {
        pid = xcd_tile(pid, g.tile_start[g.n_groups]);  // the grid holds exactly these tiles
        int lo = 0, hi = g.n_groups;  // find grp with tile_start[grp] <= pid < tile_start[grp+1]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (g.tile_start[mid] <= pid)
                lo = mid;
            else
                hi = mid;
        }
        grp = lo;
        r0 = g.row_off[grp];
        r1 = g.row_off[grp + 1];
        local = pid - g.tile_start[grp];
    }
    const int gn = g.group_n;
    Problem P;
    if (OP == kGemmFwd || OP == kGemmDgrad) {
        P.M = r1 - r0;
        P.a = g.a + (int64_t)r0 * g.lda;
        P.sa = g.sa + (int64_t)(r0 >> 5) * g.lds_a;
        P.a_rows = g.a_rows - r0;
        P.c = c_elem<OBF>(g.c, (int64_t)r0 * g.ldc);
        if (OP == kGemmFwd) {
            P.N = gn;
            P.K = g.K;
            P.b = g.b + (int64_t)grp * gn * g.ldb;
            P.sb = g.sb + (int64_t)(grp * gn >> 5) * g.lds_b;
            P.b_rows = gn;
        } else {
            P.N = g.N;
            P.K = gn;
            P.b = g.b + (int64_t)grp * gn / 2;
            P.sb = g.sb + (int64_t)(grp * gn >> 5) * g.lds_b;
            P.b_rows = g.b_rows;
        }
    } else {
        P.M = gn;
        P.N = g.N;
        P.K = r1 - r0;
        P.a = g.a + r0 / 2;
        P.sa = g.sa + (int64_t)(r0 >> 5) * g.lds_a;
        P.b = g.b + r0 / 2;
        P.sb = g.sb + (int64_t)(r0 >> 5) * g.lds_b;
        P.a_rows = g.a_rows;
        P.b_rows = g.b_rows;
        P.c = c_elem<OBF>(g.c, (int64_t)grp * gn * g.ldc);
    }
    const int ntn = (P.N + kBN - 1) / kBN;
    P.tm = local / ntn;
    P.tn = local - P.tm * ntn;
    gemm_tile<1, A_ST, B_ST, true, 0, false, OBF, false, 1, OP != kGemmWgrad>(g, P);
}

// Dynamic LDS: two stage buffers plus, per operand, the tile's scale bytes
// for its K range or (1D layout) the scale chunk ring.
inline size_t lds_bytes(int fmt, int K, int oned = 0)
{
    const size_t full = (size_t)scale_rows(fmt) * scale_kb_pad(K / 32);
    return kTileLds + ((oned & 1) ? kRing1D : full) + ((oned & 2) ? kRing1D : full);
}

// Raises a kernel's dynamic LDS limit to the whole 160 KB of a CU, once per
// (kernel, device).
inline hipError_t allow_lds_raw(const void* fn, size_t bytes)
{
    constexpr int kLdsMax = 160 * 1024;
    if (bytes <= 65536)
        return hipSuccess;
    if (bytes > (size_t)kLdsMax)
        return hipErrorInvalidValue;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    static std::mutex mu;
    static std::vector<std::pair<const void*, int>> done;
    std::lock_guard<std::mutex> lock(mu);
    for (const auto& d : done)
        if (d.first == fn && d.second == dev)
            return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax);
    if (e == hipSuccess)
        done.emplace_back(fn, dev);
    return e;
}

template <typename F>
hipError_t allow_lds(F* fn, size_t bytes)
{
    return allow_lds_raw(reinterpret_cast<const void*>(fn), bytes);
}

template <int FMT, bool A_ST, bool B_ST, bool KT, int ONED, bool ACC, bool OBF>
hipError_t launch_dense_k(const GemmArgs& g, int batch, hipStream_t s)
{
    const int ntm = (g.M + kBM - 1) / kBM, ntn = (g.N + kBN - 1) / kBN;
    const size_t lb = lds_bytes(FMT, g.K, ONED);
    hipError_t e = allow_lds(gemm_dense_kernel<FMT, A_ST, B_ST, KT, ONED, ACC, OBF>, lb);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((gemm_dense_kernel<FMT, A_ST, B_ST, KT, ONED, ACC, OBF>), dim3(ntm * ntn, batch),
                       dim3(kThreads), lb, s, g);
    return hipGetLastError();
}

// force_kt: take the K-checked variant even for K % 256 == 0 (a launch over
// one chunk of a longer contraction, whose operand bases start inside the
// planes, so the buffer range no longer ends at the planes' end).
template <int FMT, bool A_ST, bool B_ST, int ONED = 0, bool ACC = false, bool OBF = false>
hipError_t launch_dense(const GemmArgs& g, int batch, hipStream_t s, bool force_kt = false)
{
    if (FMT == 1 && g.K % 256 == 0 && !force_kt)
        return launch_dense_k<FMT, A_ST, B_ST, false, ONED, ACC, OBF>(g, batch, s);
    return launch_dense_k<FMT, A_ST, B_ST, true, ONED, ACC, OBF>(g, batch, s);
}

template <int OP, bool A_ST, bool B_ST, bool DEV, bool OBF = false>
hipError_t launch_grouped(const GemmArgs& g, hipStream_t s)
{
    // Host offsets: the exact tile count.  Device offsets: the bound the host
    // computed (g.tile_bound); surplus workgroups exit.
    const int ntiles = DEV ? g.tile_bound : g.tile_start[g.n_groups];
    if (ntiles == 0)
        return hipSuccess;
    // K of a group: FWD the full K, DGRAD the expert width, WGRAD the largest
    // token segment (device offsets: the caller's bound max_rows)
    int kmax = g.K;
    if (OP == kGemmDgrad)
        kmax = g.group_n;
    if (OP == kGemmWgrad) {
        kmax = 32;
        if (DEV)
            kmax = max(kmax, g.max_rows);
        else
            for (int i = 0; i < g.n_groups; ++i)
                kmax = max(kmax, g.row_off[i + 1] - g.row_off[i]);
    }
    const size_t lb = lds_bytes(1, kmax);
    hipError_t e = allow_lds(gemm_grouped_kernel<OP, A_ST, B_ST, DEV, OBF>, lb);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((gemm_grouped_kernel<OP, A_ST, B_ST, DEV, OBF>), dim3(ntiles), dim3(kThreads), lb, s, g);
    return hipGetLastError();
}

template <bool A_ST, bool B_ST, bool KT>
hipError_t launch_quant_k(const GemmArgs& g, hipStream_t s)
{
    const int ntm = (g.M + kBM - 1) / kBM, ntn = (g.N + kBN - 1) / kBN;
    const size_t lb = lds_bytes(1, g.K, 0);
    hipError_t e = allow_lds(gemm_quant_kernel<A_ST, B_ST, KT>, lb);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((gemm_quant_kernel<A_ST, B_ST, KT>), dim3(ntm * ntn), dim3(kThreads), lb, s, g);
    return hipGetLastError();
}

// Largest contraction one sub-block launch stages in LDS (a multiple of 256).
template <int SUB>
constexpr int sub_k_chunk()
{
    return SUB == 2 ? 15872 : 3840;
}

template <int SUB, bool A_ST, bool B_ST, bool KT, bool ACC>
hipError_t launch_sub_k(const GemmArgs& g, hipStream_t s)
{
    const int ntm = (g.M + kBM - 1) / kBM, ntn = (g.N + kBN - 1) / kBN;
    const size_t lb = kTileLds + 2 * (size_t)sub_scale_bytes<SUB>(g.K);
    hipError_t e = allow_lds(gemm_sub_kernel<SUB, A_ST, B_ST, KT, ACC>, lb);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((gemm_sub_kernel<SUB, A_ST, B_ST, KT, ACC>), dim3(ntm * ntn), dim3(kThreads), lb, s, g);
    return hipGetLastError();
}

// C = A B^T (or C += A B^T) for sub-block operands: the contraction in chunks
// of at most sub_k_chunk<SUB>(), every chunk after the first accumulating.
template <int SUB, bool A_ST, bool B_ST>
hipError_t launch_sub(const GemmArgs& g, bool accumulate, hipStream_t s)
{
    constexpr int kB = 32 / SUB;
    for (int k0 = 0; k0 < g.K; k0 += sub_k_chunk<SUB>()) {
        GemmArgs c = g;
        c.K = min(sub_k_chunk<SUB>(), g.K - k0);
        c.a = g.a + k0 / 2;
        c.b = g.b + k0 / 2;
        c.sa = g.sa + (A_ST ? (int64_t)(k0 / kB) * g.lds_a : k0 / kB);
        c.sb = g.sb + (B_ST ? (int64_t)(k0 / kB) * g.lds_b : k0 / kB);
        const bool acc = accumulate || k0 > 0;
        // A chunk after the first starts its operands k0/2 bytes into each
        // row while the buffer range stays a_rows * ld bytes from there, so
        // the range would reach past the end of the planes: such chunks take
        // the K-checked variant, whose loads past the chunk's K read as zero
        // and never touch memory.  The first chunk's loads past its K stay
        // inside the row or fall past the range and read as zero.
        const bool kt = k0 > 0 || c.K % 256 != 0;
        hipError_t e = acc ? (kt ? launch_sub_k<SUB, A_ST, B_ST, true, true>(c, s)
                                 : launch_sub_k<SUB, A_ST, B_ST, false, true>(c, s))
                           : (kt ? launch_sub_k<SUB, A_ST, B_ST, true, false>(c, s)
                                 : launch_sub_k<SUB, A_ST, B_ST, false, false>(c, s));
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <int SUB>
hipError_t launch_sub_any(const GemmArgs& g, bool a_st, bool b_st, bool accumulate, hipStream_t s)
{
    if (!a_st && !b_st)
        return launch_sub<SUB, false, false>(g, accumulate, s);
    if (!a_st && b_st)
        return launch_sub<SUB, false, true>(g, accumulate, s);
    if (a_st && b_st)
        return launch_sub<SUB, true, true>(g, accumulate, s);
    return launch_sub<SUB, true, false>(g, accumulate, s);
}

} // namespace

// Launchers of the kernel families, one translation unit each (they compile
// in parallel): plain products, bf16 output, accumulation, 1D-layout
// operands and grouped products.  launch_gemm (gemm.hip) picks one.
hipError_t launch_gemm_plain(const GemmArgs& g, int fmt, bool a_st, bool b_st, int batch, hipStream_t s,
                             bool force_kt = false);
hipError_t launch_gemm_obf(const GemmArgs& g, int fmt, bool a_st, bool b_st, int batch, hipStream_t s);
hipError_t launch_gemm_acc(const GemmArgs& g, bool a_st, bool b_st, int oned, int batch, hipStream_t s,
                           bool force_kt = false);
hipError_t launch_gemm_1d(const GemmArgs& g, bool a_st, bool b_st, int oned, int batch, hipStream_t s,
                          bool force_kt = false);
hipError_t launch_gemm_grouped(const GemmArgs& g, int op, bool out_bf16, hipStream_t s);
hipError_t launch_gemm_sub16(const GemmArgs& g, bool a_st, bool b_st, bool accumulate, hipStream_t s);
hipError_t launch_gemm_sub8(const GemmArgs& g, bool a_st, bool b_st, bool accumulate, hipStream_t s);

} // namespace fp4q
