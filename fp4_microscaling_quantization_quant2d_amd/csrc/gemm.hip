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
// (256 fp32 accumulators per lane).  Each pipeline stage moves 64 bytes of K
// per row (128 FP4 or 64 FP8 values) for 256 A rows and 256 B rows from HBM
// into one of two LDS buffers (XOR-swizzled 16-byte chunks, 64 KB total);
// global loads for stage s+1 are in flight while stage s is multiplied.
// Tiles are ordered so each XCD walks a contiguous, M-grouped range of the
// tile grid, keeping A/B panels resident in that XCD's L2.
#include "fp4q_launch.hpp"

#include <hip/hip_runtime.h>

namespace fp4q {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256;
constexpr int kThreads = 256;
constexpr int kRowBytes = 64;                       // K bytes per row per stage
constexpr int kTileBytes = kBM * kRowBytes;         // 16 KB per operand per stage
constexpr int kLdsBytes = 2 * 2 * kTileBytes;       // 2 operands x 2 buffers

// Byte offset of 16-byte chunk c of row r inside a stage tile.  The xor
// spreads the 32 rows read by one MFMA operand fetch over all LDS banks.
__device__ __forceinline__ int swz(int r, int c) { return r * kRowBytes + ((c ^ ((r >> 1) & 3)) << 4); }

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

// Scale byte of (row, kb) for one operand.
template <int FMT, bool ST>
__device__ __forceinline__ uint32_t scale_at(const uint8_t* s, int64_t lds, int row, int kb)
{
    if (FMT == 2)
        return s[(int64_t)row * lds + kb];
    if (ST)
        return s[(int64_t)kb * lds + (row >> 5)];
    return s[(int64_t)(row >> 5) * lds + kb];
}

template <int FMT, bool A_ST, bool B_ST>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, const Problem& P)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = P.tm * kBM, n0 = P.tn * kBN;
    const int kbytes = FMT == 1 ? P.K / 2 : P.K;    // K bytes per row
    const int nstages = (kbytes + kRowBytes - 1) / kRowBytes;
    const int kblocks = P.K / 32;

    // global -> register loader: thread owns rows (tid>>2) + 64p, chunk tid&3
    const int lrow = tid >> 2, lchk = tid & 3;
    uint4 ra[4], rb[4];
    auto gload = [&](int s) {
        const int kb0 = s * kRowBytes + lchk * 16;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int r = lrow + 64 * p;
            const int ar = m0 + r, brr = n0 + r;
            uint4 va = {0, 0, 0, 0}, vb = {0, 0, 0, 0};
            if (ar < P.a_rows && kb0 < kbytes)
                va = *reinterpret_cast<const uint4*>(P.a + (int64_t)ar * g.lda + kb0);
            if (brr < P.b_rows && kb0 < kbytes)
                vb = *reinterpret_cast<const uint4*>(P.b + (int64_t)brr * g.ldb + kb0);
            ra[p] = va;
            rb[p] = vb;
        }
    };
    auto sstore = [&](int buf) {
        uint8_t* la = lds + buf * 2 * kTileBytes;
        uint8_t* lb = la + kTileBytes;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int r = lrow + 64 * p;
            *reinterpret_cast<uint4*>(la + swz(r, lchk)) = ra[p];
            *reinterpret_cast<uint4*>(lb + swz(r, lchk)) = rb[p];
        }
    };

    // per-lane scale operands: byte j = scale of this lane's row for the
    // K-block used by MFMA step j of the stage
    const int lrow32 = lane & 31, khalf = lane >> 5;
    uint32_t sA[4], sB[4], sAn[4], sBn[4];
    auto sload = [&](int s, uint32_t* oa, uint32_t* ob) {
        const int steps = FMT == 1 ? 2 : 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ar = m0 + wm * 128 + i * 32 + lrow32;
            const int br_ = n0 + wn * 128 + i * 32 + lrow32;
            uint32_t va = 0, vb = 0;
#pragma unroll
            for (int j = 0; j < steps; ++j) {
                const int kb = s * (2 * steps) + 2 * j + khalf;
                if (kb < kblocks) {
                    if (ar < P.a_rows)
                        va |= scale_at<FMT, A_ST>(P.sa, g.lds_a, ar, kb) << (8 * j);
                    if (br_ < P.b_rows)
                        vb |= scale_at<FMT, B_ST>(P.sb, g.lds_b, br_, kb) << (8 * j);
                }
            }
            oa[i] = va;
            ob[i] = vb;
        }
    };

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;

    gload(0);
    sload(0, sA, sB);
    sstore(0);
    __syncthreads();

    for (int s = 0; s < nstages; ++s) {
        const bool more = s + 1 < nstages;
        if (more) {
            gload(s + 1);
            sload(s + 1, sAn, sBn);
        }
        const uint8_t* la = lds + (s & 1) * 2 * kTileBytes;
        const uint8_t* lb = la + kTileBytes;
        if (FMT == 1) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                v8i fa[4], fb[4];
                const int chk = 2 * j + khalf;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ar = wm * 128 + i * 32 + lrow32;
                    const int br_ = wn * 128 + i * 32 + lrow32;
                    const uint4 xa = *reinterpret_cast<const uint4*>(la + swz(ar, chk));
                    const uint4 xb = *reinterpret_cast<const uint4*>(lb + swz(br_, chk));
                    fa[i] = v8i{(int)xa.x, (int)xa.y, (int)xa.z, (int)xa.w, 0, 0, 0, 0};
                    fb[i] = v8i{(int)xb.x, (int)xb.y, (int)xb.z, (int)xb.w, 0, 0, 0, 0};
                }
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
                        if (j == 0)
                            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                fa[mi], fb[ni], acc[mi][ni], 4, 4, 0, (int)sA[mi], 0, (int)sB[ni]);
                        else
                            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                fa[mi], fb[ni], acc[mi][ni], 4, 4, 1, (int)sA[mi], 1, (int)sB[ni]);
                    }
            }
        } else {
            v8i fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ar = wm * 128 + i * 32 + lrow32;
                const int br_ = wn * 128 + i * 32 + lrow32;
                const uint4 xa0 = *reinterpret_cast<const uint4*>(la + swz(ar, 2 * khalf));
                const uint4 xa1 = *reinterpret_cast<const uint4*>(la + swz(ar, 2 * khalf + 1));
                const uint4 xb0 = *reinterpret_cast<const uint4*>(lb + swz(br_, 2 * khalf));
                const uint4 xb1 = *reinterpret_cast<const uint4*>(lb + swz(br_, 2 * khalf + 1));
                fa[i] = v8i{(int)xa0.x, (int)xa0.y, (int)xa0.z, (int)xa0.w,
                            (int)xa1.x, (int)xa1.y, (int)xa1.z, (int)xa1.w};
                fb[i] = v8i{(int)xb0.x, (int)xb0.y, (int)xb0.z, (int)xb0.w,
                            (int)xb1.x, (int)xb1.y, (int)xb1.z, (int)xb1.w};
            }
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fa[mi], fb[ni], acc[mi][ni], 0, 0, 0, (int)sA[mi], 0, (int)sB[ni]);
        }
        if (more)
            sstore((s + 1) & 1);
        __syncthreads();
        if (more) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sA[i] = sAn[i];
                sB[i] = sBn[i];
            }
        }
    }

    // epilogue: lane holds C[8(r/4) + 4(lane/32) + r%4][lane%32] of each 32x32 tile
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
                if (row < P.M)
                    P.c[(int64_t)row * g.ldc + col] = acc[mi][ni][r];
            }
        }
    }
}

// Tile order: each XCD (dispatch id mod 8) receives a contiguous range of
// tile ids; inside it tiles are M-grouped in bands of 8 tile rows.
__device__ __forceinline__ void tile_of(int pid, int ntm, int ntn, int& tm, int& tn)
{
    const int nt = ntm * ntn;
    if ((nt & 7) == 0)
        pid = (pid & 7) * (nt >> 3) + (pid >> 3);
    const int band = 8 * ntn;
    const int first = (pid / band) * 8;
    const int rows = min(ntm - first, 8);
    const int in = pid - (pid / band) * band;
    tm = first + in % rows;
    tn = in / rows;
}

template <int FMT, bool A_ST, bool B_ST>
__global__ __launch_bounds__(kThreads, 1) void gemm_dense_kernel(GemmArgs g)
{
    const int bz = blockIdx.y;
    Problem P;
    P.a = g.a + bz * g.bs_a;
    P.b = g.b + bz * g.bs_b;
    P.sa = g.sa + bz * g.bs_sa;
    P.sb = g.sb + bz * g.bs_sb;
    P.c = g.c + bz * g.bs_c;
    P.M = g.M;
    P.N = g.N;
    P.K = g.K;
    P.a_rows = g.a_rows;
    P.b_rows = g.b_rows;
    const int ntm = (g.M + kBM - 1) / kBM, ntn = (g.N + kBN - 1) / kBN;
    tile_of(blockIdx.x, ntm, ntn, P.tm, P.tn);
    gemm_tile<FMT, A_ST, B_ST>(g, P);
}

// Grouped (expert) products.  Group g owns token rows [row_off[g], row_off[g+1]).
//   FWD:   A = X rows of g,  B = W rows [g*gn, (g+1)*gn),       C rows of g
//   DGRAD: A = dY rows of g, B = W^T plane, K range of expert g, C rows of g
//   WGRAD: A = dY^T, B = X^T planes over the token range of g,  C rows [g*gn, ..)
template <int OP, bool A_ST, bool B_ST>
__global__ __launch_bounds__(kThreads, 1) void gemm_grouped_kernel(GemmArgs g)
{
    const int pid = blockIdx.x;
    int lo = 0, hi = g.n_groups;  // find grp with tile_start[grp] <= pid < tile_start[grp+1]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (g.tile_start[mid] <= pid)
            lo = mid;
        else
            hi = mid;
    }
    const int grp = lo;
    const int r0 = g.row_off[grp], r1 = g.row_off[grp + 1];
    const int gn = g.group_n;
    Problem P;
    if (OP == kGemmFwd || OP == kGemmDgrad) {
        P.M = r1 - r0;
        P.a = g.a + (int64_t)r0 * g.lda;
        P.sa = g.sa + (int64_t)(r0 >> 5) * g.lds_a;
        P.a_rows = g.a_rows - r0;
        P.c = g.c + (int64_t)r0 * g.ldc;
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
        P.c = g.c + (int64_t)grp * gn * g.ldc;
    }
    const int ntn = (P.N + kBN - 1) / kBN;
    const int local = pid - g.tile_start[grp];
    P.tm = local / ntn;
    P.tn = local - P.tm * ntn;
    gemm_tile<1, A_ST, B_ST>(g, P);
}

template <int FMT, bool A_ST, bool B_ST>
hipError_t launch_dense(const GemmArgs& g, int batch, hipStream_t s)
{
    const int ntm = (g.M + kBM - 1) / kBM, ntn = (g.N + kBN - 1) / kBN;
    hipLaunchKernelGGL((gemm_dense_kernel<FMT, A_ST, B_ST>), dim3(ntm * ntn, batch), dim3(kThreads),
                       kLdsBytes, s, g);
    return hipGetLastError();
}

template <int OP, bool A_ST, bool B_ST>
hipError_t launch_grouped(const GemmArgs& g, hipStream_t s)
{
    const int ntiles = g.tile_start[g.n_groups];
    if (ntiles == 0)
        return hipSuccess;
    hipLaunchKernelGGL((gemm_grouped_kernel<OP, A_ST, B_ST>), dim3(ntiles), dim3(kThreads), kLdsBytes,
                       s, g);
    return hipGetLastError();
}

} // namespace

hipError_t launch_gemm(const GemmArgs& g, int fmt, bool a_st, bool b_st, int grouped_op, int batch,
                       hipStream_t s)
{
    if (grouped_op == kGemmFwd)
        return launch_grouped<kGemmFwd, false, false>(g, s);
    if (grouped_op == kGemmDgrad)
        return launch_grouped<kGemmDgrad, false, true>(g, s);
    if (grouped_op == kGemmWgrad)
        return launch_grouped<kGemmWgrad, true, true>(g, s);
    if (fmt == 2)
        return launch_dense<2, false, false>(g, batch, s);
    if (!a_st && !b_st)
        return launch_dense<1, false, false>(g, batch, s);
    if (!a_st && b_st)
        return launch_dense<1, false, true>(g, batch, s);
    if (a_st && b_st)
        return launch_dense<1, true, true>(g, batch, s);
    return launch_dense<1, true, false>(g, batch, s);
}

int gemm_tile_m() { return kBM; }
int gemm_tile_n() { return kBN; }

} // namespace fp4q
