// Internal launch interface between the C ABI layer (api.hip) and the kernel
// translation units.  Host code validates every argument before filling
// these structs; the kernels trust them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

struct Quant2dArgs {
    const void* x;
    int64_t ldx;       // elements
    int rows, cols;    // logical shape
    int rows_pad, cols_pad;
    uint8_t* codes;    // [rows_pad x ld]
    int64_t ld;
    uint8_t* codes_t;  // [cols_pad x ld_t] or null
    int64_t ld_t;
    uint8_t* scales;   // 2D: [rows_pad/b x ld_s]; 1D: [rows_pad x ld_s], ld_s % 4 == 0
    int64_t ld_s;
    uint8_t* scales_t; // 1D only: [cols_pad x ld_st] scales of the transposed plane, ld_st % 4 == 0
    int64_t ld_st;
    uint32_t key0, key1, stream;
};

// Up to kQuant2dBatchMax matrices in one launch: item i owns workgroups
// [first[i], first[i+1]), one per 128x128 region of its padded matrix.
constexpr int kQuant2dBatchMax = 8;
struct Quant2dBatch {
    Quant2dArgs item[kQuant2dBatchMax];
    int first[kQuant2dBatchMax + 1];
    int n;
    // Optional device-resident seed: when set, the Philox key of every item
    // is (key1:key0) + *seed_dev, read when the kernel runs.
    const uint64_t* seed_dev;
};

// Regions (workgroups) of one padded matrix.
int64_t quant2d_regions(int64_t rows_pad, int64_t cols_pad);

// Scale layouts: square 32x32, 64x64, 16x16 or 8x8 blocks, or the 1D
// activation layout (1x32 blocks along the rows of each plane).
enum QuantLayout { kLayout2D32 = 0, kLayout2D64 = 1, kLayout1D = 2, kLayout2D16 = 3, kLayout2D8 = 4 };
hipError_t launch_quant2d(const Quant2dBatch& b, bool f32, bool rne, bool aligned, int layout, hipStream_t s);

struct Mxfp8Args {
    const void* x;
    int64_t ldx;
    int64_t rows;
    int cols, cols_pad;
    uint8_t* codes;    // [rows x ld]
    int64_t ld;
    uint8_t* scales;   // [rows x ld_s]
    int64_t ld_s;
};

hipError_t launch_quant1d_mxfp8(const Mxfp8Args& p, bool f32, bool aligned, hipStream_t s);

struct DequantArgs {
    const uint8_t* codes;
    int64_t ld;
    const uint8_t* scales;
    int64_t ld_s;
    int scale_transposed;  // FP4: 1 -- scale of (r, c) at (c/b)*ld_s + r/b; 2 -- the 1D layout's tiled grid
    int block_shift;       // FP4: log2 of the square block side b (5 or 6)
    int rows, cols;        // output shape
    void* y;
    int64_t ldy;
};

hipError_t launch_dequant(const DequantArgs& p, int fmt, bool out_bf16, hipStream_t s);

// Block-scaled GEMM C[M x N] = A[M x K] . B[N x K]^T with both operands
// contraction-contiguous (one row of A or B is K codes).  Scale of A row m,
// K-block kb:  FP4 2D grid   sa[(m/32)*lds_a + kb]   (a_st = 0)
//                            sa[kb*lds_a + m/32]     (a_st = 1, transposed grid)
//              MXFP8 1D grid sa[m*lds_a + kb]
constexpr int kMaxGroups = 256;

struct GemmArgs {
    const uint8_t* a;
    const uint8_t* b;
    const uint8_t* sa;
    const uint8_t* sb;
    float* c;              // fp32 C, or bf16 C reinterpreted (out_bf16)
    int64_t lda, ldb;      // bytes per operand row
    int64_t lds_a, lds_b;  // bytes per scale-grid row
    int sh_a, sh_b;        // FP4: log2 of each operand's square scale block (5: 32x32, 6: 64x64)
    int64_t ldc;           // floats
    int M, N, K;           // K in elements, multiple of 32
    int a_rows, b_rows;    // rows allocated in the operand planes (load bound)
    // batch (blockIdx.y): per-item strides
    int64_t bs_a, bs_b, bs_sa, bs_sb, bs_c;
    // grouped mode: number of groups and row offsets (multiples of 32)
    int n_groups;
    int group_n;           // rows of B per group (FWD/DGRAD) or C rows per group (WGRAD)
    int tile_start[kMaxGroups + 1];
    int row_off[kMaxGroups + 1];
    // grouped mode with device offsets (row_off_dev non-null): n_groups + 1
    // int64 offsets in device memory, clamped by the kernel to [0, tok_rows];
    // WGRAD groups are cut to max_rows rows; the grid has tile_bound
    // workgroups (an upper bound on the tiles).
    const int64_t* row_off_dev;
    int tok_rows, max_rows, tile_bound;
    // quantize-in-epilogue (launch_gemm_quant): instead of C, the 2D 32x32
    // FP4 planes of C -- row plane [q_rows_pad x q_ld], transposed plane
    // [q_cols_pad x q_ld_t] (or null), scale grid [q_rows_pad/32 x q_ld_s] --
    // with the Philox key (q_key1:q_key0) (+ *q_seed_dev when set) and stream
    // q_stream; q_rne selects round-to-nearest-even.
    uint8_t* q_codes;
    int64_t q_ld;
    uint8_t* q_codes_t;
    int64_t q_ld_t;
    uint8_t* q_scales;
    int64_t q_ld_s;
    int q_rows_pad, q_cols_pad;
    uint32_t q_key0, q_key1, q_stream;
    int q_rne;
    const uint64_t* q_seed_dev;
};

enum GemmKind { kGemmFwd = 0, kGemmDgrad = 1, kGemmWgrad = 2 };

// fmt: 1 FP4, 2 FP8.  a_st / b_st: transposed scale grids (FP4 only).
// oned: bit 0 / bit 1 -- A / B carry the 1D layout's tiled scale grid
// (chunk (g, q) of rows 128g.., K-blocks 4q.. at g*lds + q*512; FP4, dense).
// grouped_op: -1 dense/batched, else the op whose grouped wiring applies.
// accumulate: C += A B^T (FP4, dense; oned 0 or 2 only).
// out_bf16: C is bf16, ldc and the batch stride in bf16 elements (FP4 with
// oned 0, dense or grouped, or MXFP8).
// Dense FP4 products (no bf16 output, A with a square-block grid) with K
// above kDenseKChunk run as accumulating chunks of kDenseKChunk.
constexpr int kDenseKChunk = 65024;
hipError_t launch_gemm(const GemmArgs& p, int fmt, bool a_st, bool b_st, int oned, int grouped_op, int batch,
                       bool accumulate, bool out_bf16, hipStream_t s);

// Fused attention with MXFP8 Q and K (head dimension 128).  Rows of every
// tensor are head-major: row (head, i) at head * L + i.
struct AttnArgs {
    const uint8_t* qc;   // Q E4M3 codes [bh*L x ldq]
    int64_t ldq;
    const uint8_t* qs;   // Q E8M0 scales [bh*L x ldqs] (4 per row)
    int64_t ldqs;
    const uint8_t* kc;   // K codes / scales likewise
    int64_t ldk;
    const uint8_t* ks;
    int64_t ldks;
    const uint16_t* v;   // V bf16 [bh*L x ldv]
    int64_t ldv;
    void* o;             // O fp32 or bf16 [bh*L x ldo] (forward output, backward input)
    int64_t ldo;
    float* lse;          // [bh*L] natural-log log-sum-exp of every query row
    const uint16_t* dout;  // backward: dO bf16 [bh*L x lddo]
    int64_t lddo;
    float* dq;           // backward outputs fp32 [bh*L x ldg]
    float* dk;
    float* dv;
    int64_t ldg;
    float* delta;        // backward workspace [bh*L]: D_i = sum_d dO_id O_id
    int bh, L;
    float scale;
    int causal, o_bf16;
};

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_bwd(const AttnArgs& a, hipStream_t s);
// The allocation-free backward's scratch: a file-scope device array of
// kAttnScratchRows floats; *p gets its address on the current device.
constexpr int64_t kAttnScratchRows = (int64_t)1 << 20;
hipError_t attn_noalloc_scratch(float** p);

// Sustained FP4 MFMA loop (measured-peak probe): `workgroups` workgroups of
// 256 threads, each wave issuing 8 * iters 32x32x64 MFMAs on hashed operand
// words or on words taken from `codes` (n_words >= 8); sink gets one float
// per thread.
hipError_t launch_mfma_probe(int64_t iters, int workgroups, float* sink, const uint32_t* codes, int64_t n_words,
                             hipStream_t s);
// Streaming copy (measured-peak probe) of `bytes` (a multiple of 16).
hipError_t launch_copy_probe(const void* src, void* dst, int64_t bytes, int workgroups, hipStream_t s);
hipError_t launch_stream_probe(const void* src, void* dst, int64_t bytes, int nread, int workgroups, hipStream_t s);
hipError_t launch_mfma_fp8_block(const uint8_t* a, const uint8_t* b, const uint8_t* sa, const uint8_t* sb, float* c,
                                 hipStream_t s);

// Dense FP4 product (square-block operands, batch 1) whose epilogue
// quantizes the fp32 result into 2D 32x32 FP4 planes (the q_* fields)
// instead of writing it: bit for bit the planes launch_quant2d gives for
// that fp32 result.
hipError_t launch_gemm_quant(const GemmArgs& p, bool a_st, bool b_st, hipStream_t s);

// Dense FP4 product (batch 1) of operands that both take 16x16 (block 16)
// or 8x8 (block 8) scale blocks; the scale grid of an operand is
// [rows_pad/b x lds] (or its transpose for a_st / b_st).  accumulate: C +=.
hipError_t launch_gemm_subblock(const GemmArgs& p, int block, bool a_st, bool b_st, bool accumulate, hipStream_t s);

// Output tile of the GEMM kernel (grouped launches size their grids with it).
int gemm_tile_m();
int gemm_tile_n();
// Dynamic LDS bytes one GEMM workgroup needs for contraction length K.
size_t gemm_lds_bytes(int fmt, int K);

} // namespace fp4q
