/*
 * fp4q.h -- C ABI of the MI355X (gfx950) library for transposition-invariant
 * 2D-block FP4 quantization and the block-scaled MXFP4 / MXFP8 GEMMs of a
 * linear layer.
 *
 * Method: "Stable FP4 Training via Transposition-Invariant Block
 * Quantization" (Rahimifar et al., arXiv 2607.24953).
 *
 * Conventions shared by every entry point
 *  - Pointers named x, y, c and every pointer inside fp4q_qtensor are DEVICE
 *    pointers owned by the caller; fp4q_groups.row_off is a host array
 *    unless its flags say device.
 *    The library never allocates, frees or synchronizes; work is enqueued on
 *    the caller's stream (a hipStream_t passed as void*, NULL = default
 *    stream) and descriptors are read only during the call.
 *  - Return value: FP4Q_OK (0) or a negative fp4q_status.  Argument errors are
 *    detected on the host before anything is enqueued (outputs untouched);
 *    fp4q_last_error() then returns a message (thread-local).  Faults inside a
 *    kernel surface at the caller's next synchronization.
 *  - Matrices are row-major.  Leading dimensions count elements for x/y/c and
 *    bytes for code planes and scale grids.
 *  - Inputs must be finite (no NaN/Inf); this is a documented precondition,
 *    not checked on the device.
 *
 * Formats
 *  - E2M1 nibble: bit 3 sign, bits 2..0 code of the magnitudes
 *    {0, 0.5, 1, 1.5, 2, 3, 4, 6}; two nibbles per byte, the LOW nibble holds
 *    the element with the EVEN column index.
 *  - E8M0 scale byte b: scale 2^(b - 127), b in [0, 254].
 *  - E4M3FN byte: sign, 4 exponent bits (bias 7), 3 mantissa bits; max 448.
 */
#ifndef FP4Q_H
#define FP4Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4Q_ABI_VERSION 3

typedef enum {
    FP4Q_OK = 0,
    FP4Q_EINVAL = -1,       /* bad argument: null pointer, shape, alignment, leading dim */
    FP4Q_EUNSUPPORTED = -2, /* valid request the library does not implement */
    FP4Q_EHIP = -3          /* the HIP runtime rejected a launch */
} fp4q_status;

typedef enum { FP4Q_DT_BF16 = 1, FP4Q_DT_F32 = 2 } fp4q_dtype;
typedef enum { FP4Q_ROUND_SR = 0, FP4Q_ROUND_RNE = 1 } fp4q_round;
typedef enum { FP4Q_OP_FWD = 0, FP4Q_OP_DGRAD = 1, FP4Q_OP_WGRAD = 2 } fp4q_op;
typedef enum {
    FP4Q_FMT_FP4_2D32 = 1,   /* E2M1 codes, one E8M0 scale per 32x32 tile */
    FP4Q_FMT_MXFP8_1D32 = 2, /* E4M3FN bytes, one E8M0 scale per 1x32 row group */
    FP4Q_FMT_FP4_2D64 = 3,   /* E2M1 codes, one E8M0 scale per 64x64 tile; code planes as 2D32,
                                scale grid ceil(rows/64) x ceil(cols/64) (ld_s >= ceil(cols/64)) */
    FP4Q_FMT_FP4_1D32 = 4,   /* E2M1 codes, activation layout: one E8M0 scale per 1x32 block of
                                each plane's rows (layout below) */
    FP4Q_FMT_FP4_2D16 = 5,   /* E2M1 codes, one E8M0 scale per 16x16 tile; code planes as 2D32,
                                scale grid R/16 x C/16 over the 32-padded planes */
    FP4Q_FMT_FP4_2D8 = 6     /* E2M1 codes, one E8M0 scale per 8x8 tile; scale grid R/8 x C/8 */
} fp4q_fmt;

/*
 * A quantized matrix of logical shape rows x cols (caller-owned host struct
 * holding device pointers).
 *
 * FP4_2D32 (written by fp4q_quant2d), with R = rows and C = cols rounded up
 * to multiples of 32:
 *   codes   [R x ld]    row plane: nibble (r, c) in byte r*ld + c/2
 *   codes_t [C x ld_t]  transposed plane: nibble (r, c) in byte c*ld_t + r/2
 *   scales  [R/32 x ld_s] E8M0 byte of tile (r/32, c/32) at (r/32)*ld_s + c/32
 *   Requires ld >= C/2, ld_t >= R/2, ld_s >= C/32; ld and ld_t multiples of 16
 *   and the planes 16-byte aligned.  Padding nibbles (r >= rows or c >= cols)
 *   are written as 0.
 * FP4_1D32 (written by fp4q_quant2d; appendix "Activations" of the page
 * below: activations take 1D blocks along the hidden channels), with R, C
 * as for FP4_2D32:
 *   codes    [R x ld]     row plane, x in 1x32 blocks along its rows (the
 *                         forward product contracts over the columns)
 *   codes_t  [C x ld_t]   transposed plane: x^T in 1x32 blocks along its
 *                         rows, i.e. 32 rows of one column of x (the
 *                         weight-gradient product contracts over the rows)
 *   scales   [ceil(R/128) x ld_s]   tiled E8M0 grid of the row plane
 *   scales_t [ceil(C/128) x ld_st]  tiled E8M0 grid of the transposed plane
 *   A tiled grid of a plane with n rows of w codes holds one 512-byte chunk
 *   per 128 rows x 128 codes: the byte of plane row r, 1x32 block kb sits at
 *     (r/128)*ld + (kb/4)*512 + (kb%2)*256 + (r%32)*8 + ((r/32)%4)*2 + (kb/2)%2
 *   (the order in which the GEMM's matrix-core lanes consume them).  Requires
 *   ld_s >= 512*ceil(C/128) and ld_st >= 512*ceil(R/128), multiples of 16,
 *   and 16-byte aligned grids; every chunk byte past the matrix is written
 *   as 0.  Code planes as for FP4_2D32.  codes_t and scales_t may both be
 *   NULL.  batch must be 1.
 * FP4_2D64 / FP4_2D16 / FP4_2D8: the code planes of FP4_2D32 with b x b scale
 *   blocks, b = 64, 16 or 8: scales [ceil(R/b) x ld_s], byte of tile
 *   (r/b, c/b) at (r/b)*ld_s + c/b, ld_s >= ceil(C/b); a tile with no valid
 *   entry (wholly in the padding) holds byte 0.
 * MXFP8_1D32 (written by fp4q_quant1d_mxfp8), with C = cols rounded up to 32:
 *   codes   [rows x ld]   one E4M3FN byte per element (padding bytes 0)
 *   scales  [rows x ld_s] E8M0 byte of group (r, c/32)
 *   codes_t unused.  Requires ld >= C (multiple of 16), ld_s >= C/32.
 * batch >= 1 stacks matrices of the same shape; item i starts at
 * codes + i*bstride, codes_t + i*bstride_t, scales + i*bstride_s (bytes).
 */
typedef struct fp4q_qtensor {
    int32_t fmt;
    int32_t reserved;
    int64_t rows, cols;
    uint8_t* codes;
    int64_t ld;
    uint8_t* codes_t;
    int64_t ld_t;
    uint8_t* scales;
    int64_t ld_s;
    int64_t batch;
    int64_t bstride, bstride_t, bstride_s;
    uint8_t* scales_t;  /* FP4_1D32 only: scale grid of the transposed plane */
    int64_t ld_st;
} fp4q_qtensor;

/*
 * Token groups of a grouped (mixture-of-experts) GEMM: group g owns token
 * rows [row_off[g], row_off[g+1]).  1 <= n <= FP4Q_MAX_GROUPS.
 *   flags 0: row_off is a HOST array of n+1 non-decreasing offsets, each a
 *     multiple of 32, row_off[0] = 0 and row_off[n] <= the token rows of a
 *     (validated; FP4Q_EINVAL otherwise).
 *   flags FP4Q_GROUPS_DEVICE: row_off is a DEVICE array of n+1 int64
 *     offsets, read by the kernels when they run (for routing computed on
 *     the GPU; no host synchronization).  They should satisfy the same
 *     rules; the kernels make any values memory-safe by clamping each
 *     offset into [0, T32] (T32 = the token rows of a rounded down to 32),
 *     rounding it down to a multiple of 32 and treating a decreasing pair as
 *     an empty group.  WGRAD needs max_rows: a bound, a multiple of 32, on
 *     any group's rows (its LDS is sized for it); a group's rows past it
 *     are ignored.  max_rows is unused otherwise.
 */
#define FP4Q_MAX_GROUPS 256
#define FP4Q_GROUPS_DEVICE 1
typedef struct fp4q_groups {
    int32_t n;
    int32_t flags;
    const int64_t* row_off;
    int64_t max_rows;
} fp4q_groups;

/* ABI version of the loaded library (FP4Q_ABI_VERSION). */
int fp4q_version(void);

/* Message describing the last non-zero return on this thread ("" if none). */
const char* fp4q_last_error(void);

/*
 * Bytes needed by fp4q_quant2d's outputs for a rows x cols matrix with the
 * tightest leading dimensions (ld = C/2, ld_t = R/2, ld_s = C/32 with R, C
 * rounded up to 32).  Any out-pointer may be NULL.
 * Following the size accounting of the pages' Table 1, each code plane is a
 * quarter of the bf16 bytes; scales add one byte per 32x32 tile.  (With
 * 64x64 blocks the planes are the same and the grid is
 * ceil(rows/64) x ceil(cols/64) bytes.)
 */
int fp4q_quant2d_sizes(int64_t rows, int64_t cols, int64_t* codes_bytes,
                       int64_t* codes_t_bytes, int64_t* scales_bytes);

/*
 * 2D-block FP4 quantization ("Stable FP4 Training via Transposition-Invariant
 * Block Quantization": Sec. 3 square blocks with S(B) = S(B^T); Sec. 3.1
 * truncation-free scale S = 2^ceil(log2(2M/(Qp-Qn))) with Qp = 6, Qn = -6
 * and stochastic rounding; Sec. 2.1 P = round_FP4(X/S); appendix "Boundary
 * blocks": the amax M covers valid entries only).
 *
 *   x        device, rows x cols, leading dim ldx elements, dtype bf16 or f32;
 *            16-byte aligned rows (ldx*elemsize % 16 == 0) take the fast path.
 *   round_mode FP4Q_ROUND_SR (stochastic) or FP4Q_ROUND_RNE (nearest-even).
 *   seed, stream_id  key and fourth counter word of the Philox4x32-10 stream.
 *            Element (r, c) draws 16 bits from the counter
 *            ((a%32)*4 + (b%32)/8, a/32, b/32, stream_id), a = min(r,c),
 *            b = max(r,c), taking half (b%8) of the 128-bit output; rounding
 *            goes up iff floor(frac * 2^16) + draw >= 2^16.  Hence
 *            quant(x^T) equals quant(x)^T bit for bit.
 *   out      fmt = FP4Q_FMT_FP4_2D32 (32x32 blocks), FP4Q_FMT_FP4_2D64,
 *            FP4Q_FMT_FP4_2D16 or FP4Q_FMT_FP4_2D8 (64x64, 16x16 or 8x8
 *            blocks, the other block sides compared in the page's Table 4:
 *            same rule per block, same per-element random fields)
 *            or FP4Q_FMT_FP4_1D32 (the activation layout: each plane in
 *            1x32 blocks along its rows, each element rounded once per
 *            plane with its one random field; the pages' appendix
 *            "Activations"),
 *            rows/cols equal to the arguments,
 *            codes, codes_t (may be NULL to skip the transposed plane) and
 *            scales set (FP4_1D32: scales_t with codes_t); batch must be 1.
 * One read of x writes the row plane, the transposed plane and the scales.
 * A matrix of 2^24 or more 128x128 regions (one workgroup each) returns
 * FP4Q_EUNSUPPORTED; that is over 2^38 elements, beyond device memory.
 */
int fp4q_quant2d(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                 int round_mode, uint64_t seed, uint32_t stream_id,
                 const fp4q_qtensor* out, void* hip_stream);

/*
 * Several fp4q_quant2d calls in one launch (same dtype, rounding mode and
 * seed): the quantization of each item is exactly that of fp4q_quant2d with
 * the item's arguments, bit for bit, and the launch overlaps the items' ramp
 * and tail.  For example the activations and the weights of one linear
 * layer.
 *   n      1 .. FP4Q_QUANT2D_BATCH_MAX items.
 *   items  host array of n item descriptors; x and out as for fp4q_quant2d,
 *          stream_id is the item's fourth Philox counter word.  Items must
 *          not overlap in memory.
 * Every item is validated before anything is launched; an error in any of
 * them launches nothing and returns as fp4q_quant2d would.  2^24 or more
 * 128x128 regions in total return FP4Q_EUNSUPPORTED.
 */
#define FP4Q_QUANT2D_BATCH_MAX 8
typedef struct fp4q_quant2d_item {
    const void* x;
    int64_t rows, cols, ldx;
    uint32_t stream_id;
    const fp4q_qtensor* out;
} fp4q_quant2d_item;

int fp4q_quant2d_batch(int n, const fp4q_quant2d_item* items, int dtype, int round_mode,
                       uint64_t seed, void* hip_stream);

/*
 * fp4q_quant2d_batch with a device-resident seed, for stochastic rounding
 * inside captured HIP graphs (the abstract and Sec. 3.1 of the same page use
 * SR to keep gradients unbiased, which needs fresh random bits every step;
 * a seed passed by value would be frozen into the graph).
 *   seed_dev  NULL: exactly fp4q_quant2d_batch.  Else a DEVICE pointer to one
 *             uint64 (8-byte aligned) read by the kernel when it runs; the
 *             Philox key is seed + *seed_dev (mod 2^64).  A caller bumps
 *             *seed_dev between replays (for example with a small kernel
 *             captured in the same graph).
 * Otherwise as fp4q_quant2d_batch; a misaligned seed_dev returns FP4Q_EINVAL.
 */
int fp4q_quant2d_batch_ex(int n, const fp4q_quant2d_item* items, int dtype, int round_mode,
                          uint64_t seed, const uint64_t* seed_dev, void* hip_stream);

/*
 * MXFP8 quantization of the query/key projections (Sec. 3.2 of the same
 * page): E4M3FN elements, one E8M0 scale per 1x32 group along each row,
 * truncation-free (the Sec. 3.1 rule with Qp = 448), round-to-nearest-even.
 *   x    device, rows x cols, leading dim ldx elements (bf16 or f32).
 *   out  fmt = FP4Q_FMT_MXFP8_1D32, codes and scales set, batch 1.
 * One launch handles fewer than 2^32 / 4 (bf16) or 2^32 / 8 (f32) groups of
 * 32; more returns FP4Q_EINVAL.
 */
int fp4q_quant1d_mxfp8(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                       const fp4q_qtensor* out, void* hip_stream);

/*
 * GEMMs of a linear layer on quantized operands (Sec. 3 "Application to
 * linear layers": Y = X W^T, dX = dY W, dW = dY^T X), fp32 accumulation and
 * fp32 output C (row-major, leading dim ldc floats).
 *   op FWD:   a = X  [T x K], b = W [N x K]  ->  C = X W^T   [T x N]
 *   op DGRAD: a = dY [T x N], b = W [N x K]  ->  C = dY W    [T x K]
 *   op WGRAD: a = dY [T x N], b = X [T x K]  ->  C = dY^T X  [N x K]
 * FP4 operands may each have 32x32 or 64x64 scale blocks (a 64x64 block's
 * byte is used for both of its 32-row slabs and both of its 32-wide K
 * blocks); operands with 16x16 or 8x8 blocks must both take the same side
 * (dense products, batch 1, fp32 C; else FP4Q_EUNSUPPORTED): the MX MFMA
 * takes one scale per 32 K values, so each 32-K step runs as 2 (16x16) or
 * 4 (8x8) MFMAs whose A operand keeps one sub-block of its codes (the rest
 * zero) with that sub-block's scales -- every product exact, at 1/2 or 1/4
 * of the matrix-core rate (contractions past 3840 for 8x8 run as chunks
 * that accumulate in C) or the 1D activation layout (each plane read with its own tiled
 * grid: FWD reads X's row plane, WGRAD X's transposed plane; dense products
 * with batch 1 only, else FP4Q_EUNSUPPORTED); grouped products take 32x32
 * blocks only (FP4Q_EUNSUPPORTED).
 * FP4 operands must carry both planes; DGRAD reads W's transposed plane and
 * WGRAD reads the transposed planes of dY and X, so each tensor is quantized
 * once.  MXFP8 operands support FWD only (S = Q K^T); every product
 * a_i*b_j*scale_a*scale_b is formed exactly, so C differs from the exact
 * sum only by fp32 accumulation rounding, as for FP4.
 *   K      the tile keeps the scale bytes of its whole K range on chip:
 *          K (per group for grouped DGRAD / WGRAD) is at most 65152 for
 *          FP4 and 1664 for MXFP8, else FP4Q_EUNSUPPORTED -- except for
 *          dense FP4 products whose A has a square-block grid and whose C
 *          is fp32 (every op with 2D operands, and WGRAD with X in the 1D
 *          layout): a longer K runs as chunks of 65024 contraction values,
 *          every chunk after the first adding into C (so C is summed in
 *          fp32 once per chunk).
 *   size   each operand plane read (rows padded to 32, plus 256 rows of
 *          reach) times its leading dimension must stay below 2 GiB, else
 *          FP4Q_EUNSUPPORTED.
 *   batch  a->batch == b->batch = B runs B independent products; product i
 *          writes C + i*c_bstride (floats).
 *   groups NULL for a dense product; else a grouped (expert) product with
 *          batch 1: FWD  b = stacked W [n*N x K], C [T x N], group g maps
 *          rows row_off[g].. of X to expert g's rows of W; DGRAD likewise
 *          with C [T x K]; WGRAD C = stacked dW [n*N x K], each expert
 *          contracting over its own token rows.  The offsets are host or
 *          device memory (fp4q_groups.flags); with device offsets the
 *          kernels clamp them and WGRAD's K is bounded by max_rows.
 */
int fp4q_gemm(int op, const fp4q_qtensor* a, const fp4q_qtensor* b, float* c, int64_t ldc,
              int64_t c_bstride, const fp4q_groups* groups, void* hip_stream);

/*
 * fp4q_gemm with flags.  FP4Q_GEMM_ACCUMULATE: C += op(a, b) instead of
 * C = op(a, b) -- gradient accumulation over micro-batches (the weight
 * gradient dW = dY^T X of Sec. 3 "Application to linear layers", summed
 * into a resident fp32 dW).  C must hold the values to add to; each element
 * is read once and written once, the sum rounded once to fp32.  Dense FP4
 * products only, and A must have a square-block grid (FWD/DGRAD/WGRAD with
 * 32x32 or 64x64 blocks, and WGRAD with X in the 1D layout); anything else
 * returns FP4Q_EUNSUPPORTED.  flags 0 is fp4q_gemm.  Unknown flag bits
 * return FP4Q_EINVAL.
 */
#define FP4Q_GEMM_ACCUMULATE 1
/*
 * FP4Q_GEMM_OUT_BF16: C is bf16 (each fp32 result rounded to nearest even;
 * c points to bf16, ldc and c_bstride count bf16 elements), halving the
 * output bytes that bound the store phase.  Products without accumulation
 * (dense, batched or grouped) of FP4 operands with square-block grids, or of
 * MXFP8 operands (S = Q K^T); anything else returns FP4Q_EUNSUPPORTED.
 */
#define FP4Q_GEMM_OUT_BF16 2
int fp4q_gemm_ex(int op, const fp4q_qtensor* a, const fp4q_qtensor* b, void* c, int64_t ldc,
                 int64_t c_bstride, const fp4q_groups* groups, int flags, void* hip_stream);

/*
 * A GEMM whose epilogue quantizes its own result (Sec. 3 "Application to
 * linear layers" of the same page: the output of one product -- a layer's
 * dX, or its Y -- is an operand of the next product, and every operand is
 * quantized once, in 32x32 blocks with the Sec. 3.1 scale and stochastic
 * rounding).  C = op(a, b) is formed exactly as fp4q_gemm forms it, in fp32,
 * and is never written: the epilogue writes its 2D 32x32 FP4 planes into
 * `out` instead, bit for bit those fp4q_quant2d writes for that fp32 C
 * (rows x cols = M x N, dtype FP4Q_DT_F32, the same round_mode, seed and
 * stream_id).  It saves C's 4-byte store and the quantizer's 4-byte read per
 * element.
 *   op, a, b   as fp4q_gemm; dense FP4 products of 32x32- or 64x64-block
 *              operands with batch 1 (else FP4Q_EUNSUPPORTED).
 *   out        fmt FP4Q_FMT_FP4_2D32, rows = M, cols = N, batch 1; codes and
 *              scales required, codes_t optional (NULL: row plane only);
 *              leading dims as fp4q_quant2d requires.
 *   round_mode, seed, stream_id   as fp4q_quant2d.
 *   seed_dev   NULL, or a DEVICE pointer to a uint64 (8-byte aligned) added
 *              to the Philox key when the kernel runs (as in
 *              fp4q_quant2d_batch_ex).
 */
int fp4q_gemm_quant(int op, const fp4q_qtensor* a, const fp4q_qtensor* b, const fp4q_qtensor* out,
                    int round_mode, uint64_t seed, uint32_t stream_id, const uint64_t* seed_dev,
                    void* hip_stream);

/*
 * Fused attention forward with MXFP8 queries and keys (Sec. 3.2 "MXFP8
 * Attention" and Fig. 3 of the same page: Q and K enter the score product in
 * MXFP8; the attention around it is standard scaled dot-product attention):
 *   O = softmax(scale * Q K^T [+ causal mask]) V,   lse_i = ln sum_j exp(s_ij)
 * computed in one pass without writing the scores: every product q_d k_d is
 * formed exactly (E4M3 x E8M0 is exact in bf16) and summed in fp32, the
 * softmax is online in fp32, and P is rounded to bf16 to multiply V.
 *   q, k     FP4Q_FMT_MXFP8_1D32 from fp4q_quant1d_mxfp8, bh*seq_len rows of
 *            128 (head dimension 128 only, else FP4Q_EUNSUPPORTED), rows
 *            head-major (row h*seq_len + i), batch 1; scale grids with 4-byte
 *            aligned rows (ld_s % 4 == 0).
 *   v        device bf16 [bh*seq_len x ldv], ldv >= 128 and a multiple of 8,
 *            16-byte aligned.
 *   o        device [bh*seq_len x ldo] in o_dtype (FP4Q_DT_BF16 or
 *            FP4Q_DT_F32), ldo >= 128 and a multiple of 8, 16-byte aligned.
 *   lse      device fp32 [bh*seq_len]: natural-log log-sum-exp of each row's
 *            scaled scores (needed by fp4q_attn_bwd).
 *   bh, seq_len  heads (1..65535) and rows per head (1..2^21); every
 *            head's slice of every tensor, seq_len x its leading dimension,
 *            stays below 2^31 elements (else FP4Q_EINVAL).
 *   scale    the score factor (1/sqrt(128) for standard attention), > 0.
 *   causal   1: key j is visible to query i iff j <= i; 0: all keys.
 */
int fp4q_attn_fwd(const fp4q_qtensor* q, const fp4q_qtensor* k, const void* v, int64_t ldv, void* o, int64_t ldo,
                  int o_dtype, float* lse, int64_t bh, int64_t seq_len, float scale, int causal, void* hip_stream);

/*
 * Fused attention backward for the forward above: the gradients of Q, K, V
 * for dL/dO = dout, with the scores and probabilities recomputed from the
 * MXFP8 Q and K and lse, never stored:
 *   dV = P^T dO,  dP = dO V^T,  D_i = sum_d dO_id O_id,  dS = P (dP - D),
 *   dQ = scale dS K,  dK = scale dS^T Q
 * (P, dS rounded to bf16 to multiply; products of bf16 values exact; fp32
 * accumulation).  dQ comes from one kernel over query blocks and dK, dV from
 * one over key blocks, so no partial sums cross workgroups.
 *   q, k, v, o, ldo, o_dtype, lse, bh, seq_len, scale, causal  as given to
 *            and returned by fp4q_attn_fwd.
 *   dout     device bf16 [bh*seq_len x lddo], lddo >= 128, a multiple of 8,
 *            16-byte aligned.
 *   dq, dk, dv  device fp32 [bh*seq_len x ldg] outputs, ldg >= 128 and a
 *            multiple of 4, 16-byte aligned.
 *   workspace device fp32 scratch of bh*seq_len floats (D), caller-owned;
 *            overwritten.
 */
int fp4q_attn_bwd(const fp4q_qtensor* q, const fp4q_qtensor* k, const void* v, int64_t ldv, const void* o,
                  int64_t ldo, int o_dtype, const float* lse, const void* dout, int64_t lddo, float* dq, float* dk,
                  float* dv, int64_t ldg, float* workspace, int64_t bh, int64_t seq_len, float scale, int causal,
                  void* hip_stream);

/*
 * fp4q_attn_bwd without the workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): D lives in a static device array of
 * FP4Q_ATTN_NOALLOC_MAX_ROWS floats (4 MiB) that each GPU holds for the life
 * of the process.  bh*seq_len above that limit returns FP4Q_EINVAL.  The
 * call allocates and frees nothing.  Every call on one GPU shares that GPU's
 * array (D is fully rewritten by each call before it is read), so calls that
 * overlap on one GPU -- on different streams, unordered -- race.  Otherwise
 * exactly fp4q_attn_bwd.
 */
#define FP4Q_ATTN_NOALLOC_MAX_ROWS (1 << 20)
int fp4q_attn_bwd_noalloc(const fp4q_qtensor* q, const fp4q_qtensor* k, const void* v, int64_t ldv, const void* o,
                          int64_t ldo, int o_dtype, const float* lse, const void* dout, int64_t lddo, float* dq,
                          float* dk, float* dv, int64_t ldg, int64_t bh, int64_t seq_len, float scale, int causal,
                          void* hip_stream);

/*
 * Dequantization X ~ P * S (Sec. 2.1 of the same page) to fp32 or bf16, for
 * every format (each plane of the 1D layout with its own grid).
 *   transposed  0: the row plane, y is rows x cols; 1 (FP4 only): the
 *               transposed plane, y is cols x rows.
 *   out_dtype   FP4Q_DT_F32 or FP4Q_DT_BF16; ldy in elements.
 */
int fp4q_dequant(const fp4q_qtensor* q, int transposed, int out_dtype, void* y, int64_t ldy,
                 void* hip_stream);

/*
 * Diagnostics, not part of the method: the measured peaks that benchmarks
 * report beside the nominal ones.
 *
 * fp4q_probe_mfma_fp4: a sustained loop of block-scaled FP4 MFMAs
 * (v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands, the instruction of
 * every FP4 product above).  Launches `workgroups` workgroups of 4 waves;
 * each wave issues 8 * iters MFMAs of 2*32*32*64 flops.  The matrix cores'
 * rate depends on the codes they multiply: codes NULL takes operand words
 * hashed per lane; else codes (device, 4-byte aligned, code_bytes >= 32) is
 * a code plane whose words the lanes take, so the loop runs on a
 * workload's own codes.  sink: device array of workgroups*256 floats,
 * written (keeps the loop alive).
 *   iters in [1, 2^32], workgroups in [1, 2^20], else FP4Q_EINVAL.
 *
 * fp4q_probe_copy: a streaming device-to-device copy of `bytes` (a positive
 * multiple of 16, both buffers 16-byte aligned, device) with 16-byte loads
 * and stores over `workgroups` workgroups of 256 threads; its rate (read +
 * written bytes over time) is the practical HBM ceiling of a read-once,
 * write-once kernel.
 *
 * fp4q_probe_stream: a streaming kernel with `nread` (1..4) read streams and
 * one write stream: dst (bytes, device, 16-byte aligned) receives, word by
 * word, the xor of the words at the same index of nread consecutive source
 * streams of `bytes` each (src holds nread*bytes).  A grid-stride loop of
 * one 16-byte word per thread over `workgroups` workgroups of 256 threads.
 * nread = 2 is the quantizer's traffic mix (two bytes read per byte
 * written): its rate is that kernel's practical HBM ceiling.
 *
 * fp4q_probe_mfma_fp8: ONE block-scaled FP8 MFMA (the same instruction with
 * E4M3 operands), C = A B^T for a [32 x 64] and b [32 x 64] E4M3 bytes
 * (row-major, device, 4-byte aligned), sa / sb [32 x 2] E8M0 bytes (one per
 * row and 32 K values, device) and c [32 x 32] fp32 (row-major, device).  It
 * exposes the instruction's own arithmetic, which rounds inside its dot
 * product, so callers can compare it with the exact product; the MXFP8
 * products above (Sec. 3.2 of the same page) form every product exactly
 * instead.  Null or misaligned buffers: FP4Q_EINVAL.
 */
int fp4q_probe_mfma_fp4(int64_t iters, int workgroups, float* sink, const uint8_t* codes, int64_t code_bytes,
                        void* hip_stream);
int fp4q_probe_copy(const void* src, void* dst, int64_t bytes, int workgroups, void* hip_stream);
int fp4q_probe_stream(const void* src, void* dst, int64_t bytes, int nread, int workgroups, void* hip_stream);
int fp4q_probe_mfma_fp8(const uint8_t* a, const uint8_t* b, const uint8_t* sa, const uint8_t* sb, float* c,
                        void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* FP4Q_H */
