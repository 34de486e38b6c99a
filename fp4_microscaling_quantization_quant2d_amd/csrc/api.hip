// C ABI of libfp4q: host-side validation and dispatch to the gfx950 kernels.
// Every argument is checked before anything is enqueued; nothing here
// allocates device memory or synchronizes.
#include "fp4q.h"
#include "fp4q_launch.hpp"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <string>

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok()
{
    g_err.clear();
    return FP4Q_OK;
}

int hip_status(hipError_t e, const char* what)
{
    if (e != hipSuccess)
        return fail(FP4Q_EHIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
    return ok();
}

inline int64_t pad32(int64_t n) { return (n + 31) / 32 * 32; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// LDS of one compute unit on gfx950.
constexpr size_t kMaxLdsBytes = 160 * 1024;

// Largest K (a multiple of 32) whose tile fits in LDS.
int max_k(int fmt)
{
    int k = 32;
    while (fp4q::gemm_lds_bytes(fmt, k + 32) <= kMaxLdsBytes)
        k += 32;
    return k;
}
constexpr int64_t kMaxDim = (int64_t)1 << 30;

// 1D layout: a plane with `width` codes per row has a tiled scale grid of
// one 512-byte chunk per 128 rows x 128 codes, ld bytes per 128-row group.
inline int64_t act1d_grid_ld(int64_t width) { return 512 * ((width + 127) / 128); }

int check_1d_grid(const uint8_t* s, int64_t ld, int64_t width, const char* name, const char* what)
{
    if (!s)
        return fail(FP4Q_EINVAL, "%s: null %s", name, what);
    if (ld < act1d_grid_ld(width) || ld % 16 || !aligned16(s))
        return fail(FP4Q_EINVAL, "%s: %s needs a leading dim >= %lld, a multiple of 16, and 16-byte alignment",
                    name, what, (long long)act1d_grid_ld(width));
    return FP4Q_OK;
}

// Side of a square-block FP4 format's scale blocks (0 for the 1D layout).
int square_block(int fmt)
{
    switch (fmt) {
    case FP4Q_FMT_FP4_2D32: return 32;
    case FP4Q_FMT_FP4_2D64: return 64;
    case FP4Q_FMT_FP4_2D16: return 16;
    case FP4Q_FMT_FP4_2D8: return 8;
    default: return 0;
    }
}

inline int log2_block(int b) { return b == 64 ? 6 : b == 16 ? 4 : b == 8 ? 3 : 5; }

int check_fp4_tensor(const fp4q_qtensor* t, const char* name, bool need_t)
{
    if (!t)
        return fail(FP4Q_EINVAL, "%s: null descriptor", name);
    if (t->fmt != FP4Q_FMT_FP4_2D32 && t->fmt != FP4Q_FMT_FP4_2D64 && t->fmt != FP4Q_FMT_FP4_1D32 &&
        t->fmt != FP4Q_FMT_FP4_2D16 && t->fmt != FP4Q_FMT_FP4_2D8)
        return fail(FP4Q_EINVAL, "%s: fmt %d is not an FP4 format", name, t->fmt);
    if (t->rows <= 0 || t->cols <= 0 || t->rows > kMaxDim || t->cols > kMaxDim)
        return fail(FP4Q_EINVAL, "%s: bad shape %lld x %lld", name, (long long)t->rows, (long long)t->cols);
    const int64_t R = pad32(t->rows), C = pad32(t->cols);
    if (!t->codes || !t->scales)
        return fail(FP4Q_EINVAL, "%s: null codes or scales", name);
    if (t->ld < C / 2 || t->ld % 16 || !aligned16(t->codes))
        return fail(FP4Q_EINVAL, "%s: row plane needs ld >= %lld, ld %% 16 == 0 and 16-byte alignment", name,
                    (long long)(C / 2));
    const bool is1d = t->fmt == FP4Q_FMT_FP4_1D32;
    if (is1d) {
        int rc = check_1d_grid(t->scales, t->ld_s, C, name, "scales");
        if (rc)
            return rc;
    } else {
        // the grid covers the 32-padded planes: ceil(C / b) columns
        const int64_t blk = square_block(t->fmt);
        if (t->ld_s < (C + blk - 1) / blk)
            return fail(FP4Q_EINVAL, "%s: ld_s %lld < %lld", name, (long long)t->ld_s, (long long)((C + blk - 1) / blk));
    }
    if (need_t || (is1d && t->codes_t)) {
        if (!t->codes_t)
            return fail(FP4Q_EINVAL, "%s: the transposed plane is required", name);
        if (t->ld_t < R / 2 || t->ld_t % 16 || !aligned16(t->codes_t))
            return fail(FP4Q_EINVAL, "%s: transposed plane needs ld_t >= %lld, ld_t %% 16 == 0, 16-byte alignment",
                        name, (long long)(R / 2));
        if (is1d) {
            int rc = check_1d_grid(t->scales_t, t->ld_st, R, name, "scales_t");
            if (rc)
                return rc;
        }
    }
    if (t->batch < 1)
        return fail(FP4Q_EINVAL, "%s: batch must be >= 1", name);
    return FP4Q_OK;
}

int check_fp8_tensor(const fp4q_qtensor* t, const char* name)
{
    if (!t)
        return fail(FP4Q_EINVAL, "%s: null descriptor", name);
    if (t->fmt != FP4Q_FMT_MXFP8_1D32)
        return fail(FP4Q_EINVAL, "%s: fmt %d is not FP4Q_FMT_MXFP8_1D32", name, t->fmt);
    if (t->rows <= 0 || t->cols <= 0 || t->rows > ((int64_t)1 << 40) || t->cols > kMaxDim)
        return fail(FP4Q_EINVAL, "%s: bad shape", name);
    const int64_t C = pad32(t->cols);
    if (!t->codes || !t->scales)
        return fail(FP4Q_EINVAL, "%s: null codes or scales", name);
    if (t->ld < C || t->ld % 16 || !aligned16(t->codes))
        return fail(FP4Q_EINVAL, "%s: codes need ld >= %lld, ld %% 16 == 0 and 16-byte alignment", name, (long long)C);
    if (t->ld_s < C / 32)
        return fail(FP4Q_EINVAL, "%s: ld_s too small", name);
    if (t->batch < 1)
        return fail(FP4Q_EINVAL, "%s: batch must be >= 1", name);
    return FP4Q_OK;
}

// Validates every item, then quantizes all of them in one launch.
int quant2d_launch(const char* fn, int n, const fp4q_quant2d_item* items, int dtype, int round_mode,
                   uint64_t seed, const uint64_t* seed_dev, void* hip_stream)
{
    if (seed_dev && (reinterpret_cast<uintptr_t>(seed_dev) & 7u))
        return fail(FP4Q_EINVAL, "%s: seed_dev must be 8-byte aligned", fn);
    static_assert(FP4Q_QUANT2D_BATCH_MAX == fp4q::kQuant2dBatchMax, "batch limit");
    if (dtype != FP4Q_DT_BF16 && dtype != FP4Q_DT_F32)
        return fail(FP4Q_EINVAL, "%s: dtype %d", fn, dtype);
    if (round_mode != FP4Q_ROUND_SR && round_mode != FP4Q_ROUND_RNE)
        return fail(FP4Q_EINVAL, "%s: round_mode %d", fn, round_mode);
    const int esz = dtype == FP4Q_DT_F32 ? 4 : 2;
    fp4q::Quant2dBatch b;
    b.n = n;
    b.seed_dev = seed_dev;
    b.first[0] = 0;
    bool aligned = true;
    int fmt = 0;
    int64_t regions = 0;
    for (int i = 0; i < n; ++i) {
        const fp4q_quant2d_item& it = items[i];
        if (!it.x)
            return fail(FP4Q_EINVAL, "%s: item %d: x is null", fn, i);
        if (it.rows <= 0 || it.cols <= 0 || it.rows > kMaxDim || it.cols > kMaxDim || it.ldx < it.cols)
            return fail(FP4Q_EINVAL, "%s: item %d: bad shape %lld x %lld (ldx %lld)", fn, i, (long long)it.rows,
                        (long long)it.cols, (long long)it.ldx);
        const fp4q_qtensor* out = it.out;
        int rc = check_fp4_tensor(out, fn, false);
        if (rc)
            return rc;
        if (out->rows != it.rows || out->cols != it.cols)
            return fail(FP4Q_EINVAL, "%s: item %d: out shape %lld x %lld != input", fn, i, (long long)out->rows,
                        (long long)out->cols);
        if (i > 0 && out->fmt != fmt)
            return fail(FP4Q_EINVAL, "%s: item %d: format differs from item 0", fn, i);
        fmt = out->fmt;
        if (out->batch != 1)
            return fail(FP4Q_EINVAL, "%s: item %d: out batch must be 1", fn, i);
        const int64_t R = pad32(it.rows), C = pad32(it.cols);
        if (out->codes_t && (out->ld_t < R / 2 || out->ld_t % 16 || !aligned16(out->codes_t)))
            return fail(FP4Q_EINVAL, "%s: item %d: transposed plane needs ld_t >= %lld, multiple of 16, aligned", fn,
                        i, (long long)(R / 2));
        // One 256-thread workgroup per 128x128 region; a launch holds fewer than 2^32 work-items.
        regions += fp4q::quant2d_regions(R, C);
        if (regions >= ((int64_t)1 << 24))
            return fail(FP4Q_EUNSUPPORTED, "%s: 2^24 or more 128x128 regions in one launch", fn);
        fp4q::Quant2dArgs& p = b.item[i];
        p.x = it.x;
        p.ldx = it.ldx;
        p.rows = (int)it.rows;
        p.cols = (int)it.cols;
        p.rows_pad = (int)R;
        p.cols_pad = (int)C;
        p.codes = out->codes;
        p.ld = out->ld;
        p.codes_t = out->codes_t;
        p.ld_t = out->ld_t;
        p.scales = out->scales;
        p.ld_s = out->ld_s;
        p.scales_t = out->fmt == FP4Q_FMT_FP4_1D32 ? out->scales_t : nullptr;
        p.ld_st = out->ld_st;
        p.key0 = (uint32_t)seed;
        p.key1 = (uint32_t)(seed >> 32);
        p.stream = it.stream_id;
        b.first[i + 1] = (int)regions;
        aligned = aligned && aligned16(it.x) && (it.ldx * esz) % 16 == 0;
    }
    return hip_status(fp4q::launch_quant2d(b, dtype == FP4Q_DT_F32, round_mode == FP4Q_ROUND_RNE, aligned,
                                           fmt == FP4Q_FMT_FP4_1D32   ? fp4q::kLayout1D
                                           : fmt == FP4Q_FMT_FP4_2D64 ? fp4q::kLayout2D64
                                           : fmt == FP4Q_FMT_FP4_2D16 ? fp4q::kLayout2D16
                                           : fmt == FP4Q_FMT_FP4_2D8  ? fp4q::kLayout2D8
                                                                      : fp4q::kLayout2D32,
                                           static_cast<hipStream_t>(hip_stream)),
                      fn);
}

} // namespace

extern "C" {

int fp4q_version(void) { return FP4Q_ABI_VERSION; }

const char* fp4q_last_error(void) { return g_err.c_str(); }

int fp4q_quant2d_sizes(int64_t rows, int64_t cols, int64_t* codes_bytes, int64_t* codes_t_bytes,
                       int64_t* scales_bytes)
{
    if (rows <= 0 || cols <= 0 || rows > kMaxDim || cols > kMaxDim)
        return fail(FP4Q_EINVAL, "fp4q_quant2d_sizes: bad shape %lld x %lld", (long long)rows, (long long)cols);
    const int64_t R = pad32(rows), C = pad32(cols);
    if (codes_bytes)
        *codes_bytes = R * C / 2;
    if (codes_t_bytes)
        *codes_t_bytes = C * R / 2;
    if (scales_bytes)
        *scales_bytes = (R / 32) * (C / 32);
    return ok();
}

int fp4q_quant2d(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int round_mode,
                 uint64_t seed, uint32_t stream_id, const fp4q_qtensor* out, void* hip_stream)
{
    fp4q_quant2d_item it;
    it.x = x;
    it.rows = rows;
    it.cols = cols;
    it.ldx = ldx;
    it.stream_id = stream_id;
    it.out = out;
    return quant2d_launch("fp4q_quant2d", 1, &it, dtype, round_mode, seed, nullptr, hip_stream);
}

int fp4q_quant2d_batch(int n, const fp4q_quant2d_item* items, int dtype, int round_mode, uint64_t seed,
                       void* hip_stream)
{
    if (n < 1 || n > FP4Q_QUANT2D_BATCH_MAX)
        return fail(FP4Q_EINVAL, "fp4q_quant2d_batch: n %d outside 1..%d", n, FP4Q_QUANT2D_BATCH_MAX);
    if (!items)
        return fail(FP4Q_EINVAL, "fp4q_quant2d_batch: items is null");
    return quant2d_launch("fp4q_quant2d_batch", n, items, dtype, round_mode, seed, nullptr, hip_stream);
}

int fp4q_quant2d_batch_ex(int n, const fp4q_quant2d_item* items, int dtype, int round_mode, uint64_t seed,
                          const uint64_t* seed_dev, void* hip_stream)
{
    if (n < 1 || n > FP4Q_QUANT2D_BATCH_MAX)
        return fail(FP4Q_EINVAL, "fp4q_quant2d_batch_ex: n %d outside 1..%d", n, FP4Q_QUANT2D_BATCH_MAX);
    if (!items)
        return fail(FP4Q_EINVAL, "fp4q_quant2d_batch_ex: items is null");
    return quant2d_launch("fp4q_quant2d_batch_ex", n, items, dtype, round_mode, seed, seed_dev, hip_stream);
}

int fp4q_quant1d_mxfp8(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                       const fp4q_qtensor* out, void* hip_stream)
{
    if (!x)
        return fail(FP4Q_EINVAL, "fp4q_quant1d_mxfp8: x is null");
    if (dtype != FP4Q_DT_BF16 && dtype != FP4Q_DT_F32)
        return fail(FP4Q_EINVAL, "fp4q_quant1d_mxfp8: dtype %d", dtype);
    if (rows <= 0 || cols <= 0 || cols > kMaxDim || ldx < cols || rows > ((int64_t)1 << 40))
        return fail(FP4Q_EINVAL, "fp4q_quant1d_mxfp8: bad shape");
    int rc = check_fp8_tensor(out, "fp4q_quant1d_mxfp8 out");
    if (rc)
        return rc;
    if (out->rows != rows || out->cols != cols || out->batch != 1)
        return fail(FP4Q_EINVAL, "fp4q_quant1d_mxfp8: out shape/batch mismatch");
    const int esz = dtype == FP4Q_DT_F32 ? 4 : 2;
    // 4 (bf16) or 8 (fp32) work-items per 1x32 group; a launch holds fewer than 2^32.
    if (rows * (pad32(cols) / 32) * (esz == 4 ? 8 : 4) >= ((int64_t)1 << 32))
        return fail(FP4Q_EINVAL, "fp4q_quant1d_mxfp8: too many groups for one launch");
    fp4q::Mxfp8Args p;
    p.x = x;
    p.ldx = ldx;
    p.rows = rows;
    p.cols = (int)cols;
    p.cols_pad = (int)pad32(cols);
    p.codes = out->codes;
    p.ld = out->ld;
    p.scales = out->scales;
    p.ld_s = out->ld_s;
    const bool aligned = aligned16(x) && ((ldx * esz) % 16 == 0);
    return hip_status(fp4q::launch_quant1d_mxfp8(p, dtype == FP4Q_DT_F32, aligned,
                                                 static_cast<hipStream_t>(hip_stream)),
                      "fp4q_quant1d_mxfp8");
}

int fp4q_gemm(int op, const fp4q_qtensor* a, const fp4q_qtensor* b, float* c, int64_t ldc, int64_t c_bstride,
              const fp4q_groups* groups, void* hip_stream)
{
    return fp4q_gemm_ex(op, a, b, c, ldc, c_bstride, groups, 0, hip_stream);
}

}  // extern "C"

namespace {

// The quantized output of fp4q_gemm_quant, validated against the product's
// shape before anything is launched.
struct QuantOut {
    const fp4q_qtensor* out;
    int round_mode;
    uint64_t seed;
    uint32_t stream_id;
    const uint64_t* seed_dev;
};

int gemm_common(int op, const fp4q_qtensor* a, const fp4q_qtensor* b, void* c, int64_t ldc, int64_t c_bstride,
                const fp4q_groups* groups, int flags, const QuantOut* qo, void* hip_stream)
{
    if (op != FP4Q_OP_FWD && op != FP4Q_OP_DGRAD && op != FP4Q_OP_WGRAD)
        return fail(FP4Q_EINVAL, "fp4q_gemm: op %d", op);
    if (flags & ~(FP4Q_GEMM_ACCUMULATE | FP4Q_GEMM_OUT_BF16))
        return fail(FP4Q_EINVAL, "fp4q_gemm_ex: unknown flags 0x%x", flags);
    const bool accumulate = (flags & FP4Q_GEMM_ACCUMULATE) != 0;
    const bool out_bf16 = (flags & FP4Q_GEMM_OUT_BF16) != 0;
    if (!a || !b || (!c && !qo))
        return fail(FP4Q_EINVAL, "fp4q_gemm: null a, b or c");
    const bool fp8 = a->fmt == FP4Q_FMT_MXFP8_1D32;
    if (fp8 != (b->fmt == FP4Q_FMT_MXFP8_1D32))
        return fail(FP4Q_EINVAL, "fp4q_gemm: operand formats differ (%d, %d)", a->fmt, b->fmt);
    int rc;
    if (fp8) {
        if (op != FP4Q_OP_FWD)
            return fail(FP4Q_EUNSUPPORTED, "fp4q_gemm: MXFP8 operands support FWD only");
        if ((rc = check_fp8_tensor(a, "fp4q_gemm a")) || (rc = check_fp8_tensor(b, "fp4q_gemm b")))
            return rc;
    } else {
        const bool at = op == FP4Q_OP_WGRAD, bt = op != FP4Q_OP_FWD;
        if ((rc = check_fp4_tensor(a, "fp4q_gemm a", at)) || (rc = check_fp4_tensor(b, "fp4q_gemm b", bt)))
            return rc;
    }
    if (a->batch != b->batch)
        return fail(FP4Q_EINVAL, "fp4q_gemm: batch mismatch %lld vs %lld", (long long)a->batch,
                    (long long)b->batch);
    if (a->batch > 65535)
        return fail(FP4Q_EINVAL, "fp4q_gemm: batch above 65535");
    if (groups && (fp8 || a->batch != 1))
        return fail(FP4Q_EINVAL, "fp4q_gemm: grouped products take FP4 operands with batch 1");
    if (groups && (a->fmt != FP4Q_FMT_FP4_2D32 || b->fmt != FP4Q_FMT_FP4_2D32))
        return fail(FP4Q_EUNSUPPORTED, "fp4q_gemm: grouped products take 32x32-block operands");

    fp4q::GemmArgs g = {};
    int64_t M, N, K;
    bool a_st = false, b_st = false;
    switch (op) {
    case FP4Q_OP_FWD:  // X [T x K], W [N x K]
        if (a->cols != b->cols)
            return fail(FP4Q_EINVAL, "fp4q_gemm FWD: K mismatch (%lld vs %lld)", (long long)a->cols,
                        (long long)b->cols);
        M = a->rows; N = b->rows; K = pad32(a->cols);
        g.a = a->codes; g.lda = a->ld; g.sa = a->scales; g.lds_a = a->ld_s;
        g.b = b->codes; g.ldb = b->ld; g.sb = b->scales; g.lds_b = b->ld_s;
        g.a_rows = (int)(fp8 ? a->rows : pad32(a->rows));
        g.b_rows = (int)(fp8 ? b->rows : pad32(b->rows));
        g.bs_a = a->bstride; g.bs_b = b->bstride;
        break;
    case FP4Q_OP_DGRAD:  // dY [T x N], W [N x K] -> [T x K]
        if (a->cols != b->rows && !groups)
            return fail(FP4Q_EINVAL, "fp4q_gemm DGRAD: dY cols %lld != W rows %lld", (long long)a->cols,
                        (long long)b->rows);
        M = a->rows; N = b->cols; K = pad32(a->cols);
        g.a = a->codes; g.lda = a->ld; g.sa = a->scales; g.lds_a = a->ld_s;
        g.b = b->codes_t; g.ldb = b->ld_t; g.sb = b->scales; g.lds_b = b->ld_s;
        b_st = true;
        g.a_rows = (int)pad32(a->rows);
        g.b_rows = (int)pad32(b->cols);
        g.bs_a = a->bstride; g.bs_b = b->bstride_t;
        break;
    default:  // WGRAD: dY [T x N], X [T x K] -> [N x K]
        if (a->rows != b->rows)
            return fail(FP4Q_EINVAL, "fp4q_gemm WGRAD: dY rows %lld != X rows %lld", (long long)a->rows,
                        (long long)b->rows);
        M = a->cols; N = b->cols; K = pad32(a->rows);
        g.a = a->codes_t; g.lda = a->ld_t; g.sa = a->scales; g.lds_a = a->ld_s;
        g.b = b->codes_t; g.ldb = b->ld_t; g.sb = b->scales; g.lds_b = b->ld_s;
        a_st = b_st = true;
        g.a_rows = (int)pad32(a->cols);
        g.b_rows = (int)pad32(b->cols);
        g.bs_a = a->bstride_t; g.bs_b = b->bstride_t;
        break;
    }
    g.bs_sa = a->bstride_s;
    g.bs_sb = b->bstride_s;
    g.sh_a = log2_block(square_block(a->fmt));
    g.sh_b = log2_block(square_block(b->fmt));
    // 16x16 / 8x8 blocks: both operands take the same block side
    const int sub_a = fp8 ? 0 : square_block(a->fmt), sub_b = fp8 ? 0 : square_block(b->fmt);
    const bool subblock = (sub_a > 0 && sub_a < 32) || (sub_b > 0 && sub_b < 32);
    if (subblock) {
        if (sub_a != sub_b)
            return fail(FP4Q_EUNSUPPORTED, "fp4q_gemm: 16x16 and 8x8 scale blocks need both operands in the same "
                                           "block side (got %d and %d)", sub_a, sub_b);
        if (groups || a->batch != 1 || qo || (flags & FP4Q_GEMM_OUT_BF16))
            return fail(FP4Q_EUNSUPPORTED, "fp4q_gemm: 16x16 and 8x8 scale blocks take dense products with batch 1 "
                                           "and fp32 C (plain or accumulating)");
    }
    // 1D-layout operands: the plane read takes its own tiled grid (scales for
    // the row plane, scales_t for the transposed plane).
    int oned = 0;
    {
        const bool a1 = a->fmt == FP4Q_FMT_FP4_1D32, b1 = b->fmt == FP4Q_FMT_FP4_1D32;
        if ((a1 || b1) && a->batch != 1)
            return fail(FP4Q_EUNSUPPORTED, "fp4q_gemm: 1D-layout operands take batch 1");
        if (a1) {
            oned |= 1;
            if (a_st) {
                g.sa = a->scales_t;
                g.lds_a = a->ld_st;
            }
            a_st = false;
        }
        if (b1) {
            oned |= 2;
            if (b_st) {
                g.sb = b->scales_t;
                g.lds_b = b->ld_st;
            }
            b_st = false;
        }
        if (((oned & 1) && ((int64_t)g.a_rows + 127) / 128 * g.lds_a > INT_MAX) ||
            ((oned & 2) && ((int64_t)g.b_rows + 127) / 128 * g.lds_b > INT_MAX))
            return fail(FP4Q_EUNSUPPORTED, "fp4q_gemm: a 1D scale grid exceeds 2 GiB");
    }
    // The kernels address each operand plane through a buffer descriptor with
    // a 32-bit byte range; a tile may reach one tile height past the last row.
    {
        const int64_t reach = fp4q::gemm_tile_m();
        if ((g.a_rows + reach) * g.lda > INT_MAX || (g.b_rows + reach) * g.ldb > INT_MAX)
            return fail(FP4Q_EUNSUPPORTED, "fp4q_gemm: an operand plane exceeds 2 GiB");
    }
    g.c = static_cast<float*>(c);
    g.ldc = ldc;
    g.bs_c = c_bstride;
    g.M = (int)M;
    g.N = (int)N;
    g.K = (int)K;
    if (fp8 && (a->cols % 32))
        return fail(FP4Q_EUNSUPPORTED, "fp4q_gemm: MXFP8 K must be a multiple of 32");

    if (qo) {
        // quantize-in-epilogue: dense FP4 products of square-block operands
        if (fp8 || groups || a->batch != 1 || oned || flags)
            return fail(FP4Q_EUNSUPPORTED, "fp4q_gemm_quant: dense FP4 products of square-block operands "
                                           "with batch 1 only");
        const fp4q_qtensor* o = qo->out;
        if ((rc = check_fp4_tensor(o, "fp4q_gemm_quant out", false)))
            return rc;
        if (o->fmt != FP4Q_FMT_FP4_2D32)
            return fail(FP4Q_EUNSUPPORTED, "fp4q_gemm_quant: out must be FP4Q_FMT_FP4_2D32");
        if (o->rows != M || o->cols != N || o->batch != 1)
            return fail(FP4Q_EINVAL, "fp4q_gemm_quant: out is %lld x %lld (batch %lld), the product %lld x %lld",
                        (long long)o->rows, (long long)o->cols, (long long)o->batch, (long long)M, (long long)N);
        if (o->codes_t && (o->ld_t < pad32(M) / 2 || o->ld_t % 16 || !aligned16(o->codes_t)))
            return fail(FP4Q_EINVAL, "fp4q_gemm_quant: transposed plane needs ld_t >= %lld, a multiple of 16, "
                                     "16-byte alignment", (long long)(pad32(M) / 2));
        if (qo->round_mode != FP4Q_ROUND_SR && qo->round_mode != FP4Q_ROUND_RNE)
            return fail(FP4Q_EINVAL, "fp4q_gemm_quant: round_mode %d", qo->round_mode);
        if (qo->seed_dev && (reinterpret_cast<uintptr_t>(qo->seed_dev) & 7u))
            return fail(FP4Q_EINVAL, "fp4q_gemm_quant: seed_dev must be 8-byte aligned");
        if (fp4q::gemm_lds_bytes(1, (int)K) > kMaxLdsBytes)
            return fail(FP4Q_EUNSUPPORTED, "fp4q_gemm_quant: K %lld too large (max %d)", (long long)K, max_k(1));
        g.q_codes = o->codes;
        g.q_ld = o->ld;
        g.q_codes_t = o->codes_t;
        g.q_ld_t = o->ld_t;
        g.q_scales = o->scales;
        g.q_ld_s = o->ld_s;
        g.q_rows_pad = (int)pad32(M);
        g.q_cols_pad = (int)pad32(N);
        g.q_key0 = (uint32_t)qo->seed;
        g.q_key1 = (uint32_t)(qo->seed >> 32);
        g.q_stream = qo->stream_id;
        g.q_rne = qo->round_mode == FP4Q_ROUND_RNE;
        g.q_seed_dev = qo->seed_dev;
        return hip_status(fp4q::launch_gemm_quant(g, a_st, b_st, static_cast<hipStream_t>(hip_stream)),
                          "fp4q_gemm_quant");
    }
    int grouped_op = -1;
    if (!groups) {
        if (ldc < N)
            return fail(FP4Q_EINVAL, "fp4q_gemm: ldc %lld < N %lld", (long long)ldc, (long long)N);
        if (a->batch > 1 && c_bstride < M * ldc)
            return fail(FP4Q_EINVAL, "fp4q_gemm: c_bstride %lld < M*ldc", (long long)c_bstride);
    } else {
        const int n = groups->n;
        if (n < 1 || n > FP4Q_MAX_GROUPS || !groups->row_off)
            return fail(FP4Q_EINVAL, "fp4q_gemm: groups->n %d out of [1, %d] or null row_off", n, FP4Q_MAX_GROUPS);
        if (groups->flags & ~FP4Q_GROUPS_DEVICE)
            return fail(FP4Q_EINVAL, "fp4q_gemm: unknown groups->flags 0x%x", groups->flags);
        const bool dev = (groups->flags & FP4Q_GROUPS_DEVICE) != 0;
        const int64_t* off = groups->row_off;
        // Group rows index C's rows (FWD, DGRAD) and the token range of the
        // planes; they end at or before the last whole 32 rows of a.
        const int64_t tok = a->rows / 32 * 32;
        if (dev) {
            if (op == FP4Q_OP_WGRAD && (groups->max_rows < 32 || groups->max_rows % 32 || groups->max_rows > tok))
                return fail(FP4Q_EINVAL, "fp4q_gemm: device-offset WGRAD needs max_rows, a multiple of 32 in "
                                         "[32, %lld]", (long long)tok);
        } else {
            if (off[0] != 0)
                return fail(FP4Q_EINVAL, "fp4q_gemm: row_off[0] must be 0");
            for (int i = 0; i < n; ++i)
                if (off[i + 1] < off[i] || off[i + 1] % 32)
                    return fail(FP4Q_EINVAL, "fp4q_gemm: row_off must be non-decreasing multiples of 32");
            if (off[n] > tok)
                return fail(FP4Q_EINVAL, "fp4q_gemm: row_off[n] %lld beyond %lld token rows", (long long)off[n],
                            (long long)tok);
        }
        int64_t gn;
        if (op == FP4Q_OP_FWD) {
            if (b->rows % n || (b->rows / n) % 32)
                return fail(FP4Q_EINVAL, "fp4q_gemm grouped FWD: W rows %lld not n x (multiple of 32)",
                            (long long)b->rows);
            gn = b->rows / n;
        } else {
            gn = a->cols;
            if (gn % 32)
                return fail(FP4Q_EINVAL, "fp4q_gemm grouped: per-expert width %lld not a multiple of 32",
                            (long long)gn);
            if (op == FP4Q_OP_DGRAD && b->rows != gn * n)
                return fail(FP4Q_EINVAL, "fp4q_gemm grouped DGRAD: W rows %lld != n x %lld", (long long)b->rows,
                            (long long)gn);
        }
        const int64_t nout = op == FP4Q_OP_FWD ? gn : N;
        if (ldc < nout)
            return fail(FP4Q_EINVAL, "fp4q_gemm grouped: ldc %lld < %lld", (long long)ldc, (long long)nout);
        g.n_groups = n;
        g.group_n = (int)gn;
        int64_t tiles = 0;
        const int tm = fp4q::gemm_tile_m(), tn = fp4q::gemm_tile_n();
        if (dev) {
            // the kernel builds the tile table; the grid is an upper bound:
            // sum_g ceil(rows_g / tm) <= ceil(tok / tm) + n
            const int64_t ntn = (nout + tn - 1) / tn;
            tiles = op == FP4Q_OP_WGRAD ? n * ((gn + tm - 1) / tm) * ntn : ((tok + tm - 1) / tm + n) * ntn;
            if (tiles > INT_MAX)
                return fail(FP4Q_EINVAL, "fp4q_gemm grouped: too many tiles");
            g.row_off_dev = off;
            g.tok_rows = (int)tok;
            g.max_rows = op == FP4Q_OP_WGRAD ? (int)groups->max_rows : 0;
            g.tile_bound = (int)tiles;
        }
        for (int i = 0; i <= n && !dev; ++i) {
            g.row_off[i] = (int)off[i];
            g.tile_start[i] = (int)tiles;
            if (i == n)
                break;
            const int64_t mg = op == FP4Q_OP_WGRAD ? gn : off[i + 1] - off[i];
            const int64_t ng = nout;
            tiles += ((mg + tm - 1) / tm) * ((ng + tn - 1) / tn);
        }
        if (tiles > INT_MAX)
            return fail(FP4Q_EINVAL, "fp4q_gemm grouped: too many tiles");
        grouped_op = op;
    }
    // The tile keeps the scale bytes of its whole K range in LDS.  K of a
    // group: FWD the full K, DGRAD the expert width, WGRAD its token count.
    int64_t kmax = K;
    if (grouped_op == FP4Q_OP_DGRAD)
        kmax = g.group_n;
    if (grouped_op == FP4Q_OP_WGRAD) {
        kmax = 32;
        if (g.row_off_dev)
            kmax = g.max_rows;
        else
            for (int i = 0; i < g.n_groups; ++i)
                kmax = std::max<int64_t>(kmax, g.row_off[i + 1] - g.row_off[i]);
    }
    if (subblock) {
        if (ldc < N)
            return fail(FP4Q_EINVAL, "fp4q_gemm: ldc %lld < N %lld", (long long)ldc, (long long)N);
        return hip_status(fp4q::launch_gemm_subblock(g, sub_a, a_st, b_st, accumulate,
                                                     static_cast<hipStream_t>(hip_stream)),
                          "fp4q_gemm");
    }
    if (accumulate && (fp8 || groups || (oned & 1)))
        return fail(FP4Q_EUNSUPPORTED, "fp4q_gemm_ex: accumulation takes dense FP4 products whose A operand "
                                       "has a square-block grid");
    if (out_bf16 && (accumulate || oned))
        return fail(FP4Q_EUNSUPPORTED, "fp4q_gemm_ex: bf16 output takes products (no accumulation) of "
                                       "square-block FP4 or MXFP8 operands");
    // Dense FP4 products with a square-block A (and no bf16 output) take any
    // K: the launcher splits a long contraction into accumulating chunks.
    const bool chunked = !fp8 && grouped_op < 0 && !out_bf16 && (oned & 1) == 0 && K > fp4q::kDenseKChunk;
    if (chunked && fp4q::gemm_lds_bytes(1, fp4q::kDenseKChunk) > kMaxLdsBytes)
        return fail(FP4Q_EUNSUPPORTED, "fp4q_gemm: K chunk does not fit the FP4 tile");
    if (!chunked && fp4q::gemm_lds_bytes(fp8 ? 2 : 1, (int)kmax) > kMaxLdsBytes)
        return fail(FP4Q_EUNSUPPORTED, "fp4q_gemm: K %lld too large for the %s tile (max %d)", (long long)kmax,
                    fp8 ? "MXFP8" : "FP4", fp8 ? max_k(2) : max_k(1));
    return hip_status(fp4q::launch_gemm(g, fp8 ? 2 : 1, a_st, b_st, oned, grouped_op, (int)a->batch, accumulate, out_bf16,
                                        static_cast<hipStream_t>(hip_stream)),
                      "fp4q_gemm");
}

} // namespace

extern "C" {

int fp4q_gemm_ex(int op, const fp4q_qtensor* a, const fp4q_qtensor* b, void* c, int64_t ldc, int64_t c_bstride,
                 const fp4q_groups* groups, int flags, void* hip_stream)
{
    return gemm_common(op, a, b, c, ldc, c_bstride, groups, flags, nullptr, hip_stream);
}

int fp4q_gemm_quant(int op, const fp4q_qtensor* a, const fp4q_qtensor* b, const fp4q_qtensor* out, int round_mode,
                    uint64_t seed, uint32_t stream_id, const uint64_t* seed_dev, void* hip_stream)
{
    if (!out)
        return fail(FP4Q_EINVAL, "fp4q_gemm_quant: null out");
    QuantOut qo = {out, round_mode, seed, stream_id, seed_dev};
    return gemm_common(op, a, b, nullptr, 0, 0, nullptr, 0, &qo, hip_stream);
}

int fp4q_dequant(const fp4q_qtensor* q, int transposed, int out_dtype, void* y, int64_t ldy, void* hip_stream)
{
    if (!q || !y)
        return fail(FP4Q_EINVAL, "fp4q_dequant: null q or y");
    if (out_dtype != FP4Q_DT_F32 && out_dtype != FP4Q_DT_BF16)
        return fail(FP4Q_EINVAL, "fp4q_dequant: out_dtype %d", out_dtype);
    int rc;
    fp4q::DequantArgs p;
    int fmt;
    const uint8_t* scales = q->scales;
    int64_t ld_s = q->ld_s;
    if (q->fmt == FP4Q_FMT_FP4_2D32 || q->fmt == FP4Q_FMT_FP4_2D64 || q->fmt == FP4Q_FMT_FP4_1D32 ||
        q->fmt == FP4Q_FMT_FP4_2D16 || q->fmt == FP4Q_FMT_FP4_2D8) {
        if ((rc = check_fp4_tensor(q, "fp4q_dequant q", transposed != 0)))
            return rc;
        fmt = 1;
        p.block_shift = log2_block(square_block(q->fmt));
        p.codes = transposed ? q->codes_t : q->codes;
        p.ld = transposed ? q->ld_t : q->ld;
        p.scale_transposed = transposed ? 1 : 0;
        if (q->fmt == FP4Q_FMT_FP4_1D32) {
            p.scale_transposed = 2;
            if (transposed) {
                scales = q->scales_t;
                ld_s = q->ld_st;
            }
        }
        p.rows = (int)(transposed ? q->cols : q->rows);
        p.cols = (int)(transposed ? q->rows : q->cols);
    } else if (q->fmt == FP4Q_FMT_MXFP8_1D32) {
        if ((rc = check_fp8_tensor(q, "fp4q_dequant q")))
            return rc;
        if (transposed)
            return fail(FP4Q_EUNSUPPORTED, "fp4q_dequant: MXFP8 has no transposed plane");
        if (q->rows > INT_MAX)
            return fail(FP4Q_EINVAL, "fp4q_dequant: too many rows");
        fmt = 2;
        p.block_shift = 5;
        p.codes = q->codes;
        p.ld = q->ld;
        p.scale_transposed = 0;
        p.rows = (int)q->rows;
        p.cols = (int)q->cols;
    } else {
        return fail(FP4Q_EINVAL, "fp4q_dequant: fmt %d", q->fmt);
    }
    if (q->batch != 1)
        return fail(FP4Q_EINVAL, "fp4q_dequant: batch must be 1");
    if (ldy < p.cols)
        return fail(FP4Q_EINVAL, "fp4q_dequant: ldy %lld < %d", (long long)ldy, p.cols);
    p.scales = scales;
    p.ld_s = ld_s;
    p.y = y;
    p.ldy = ldy;
    return hip_status(fp4q::launch_dequant(p, fmt, out_dtype == FP4Q_DT_BF16, static_cast<hipStream_t>(hip_stream)),
                      "fp4q_dequant");
}

}  // extern "C"

namespace {

// Validation shared by the attention entry points: MXFP8 Q and K of
// bh*seq_len rows and 128 columns, aligned for the kernels' vector accesses.
int check_attn(const char* fn, const fp4q_qtensor* q, const fp4q_qtensor* k, const void* v, int64_t ldv,
               const void* o, int64_t ldo, int o_dtype, const float* lse, int64_t bh, int64_t seq_len, float scale,
               int causal, fp4q::AttnArgs& a)
{
    int rc;
    if ((rc = check_fp8_tensor(q, fn)) || (rc = check_fp8_tensor(k, fn)))
        return rc;
    // grids: heads along x, 64-row blocks along y (at most 65535)
    if (bh < 1 || seq_len < 1 || bh > 65535 || seq_len > (1 << 21) || bh * seq_len > ((int64_t)1 << 31))
        return fail(FP4Q_EINVAL, "%s: bh %lld and seq_len %lld out of range", fn, (long long)bh, (long long)seq_len);
    if (q->cols != 128 || k->cols != 128)
        return fail(FP4Q_EUNSUPPORTED, "%s: head dimension 128 only (got %lld, %lld)", fn, (long long)q->cols,
                    (long long)k->cols);
    if (q->rows != bh * seq_len || k->rows != bh * seq_len || q->batch != 1 || k->batch != 1)
        return fail(FP4Q_EINVAL, "%s: q and k need bh*seq_len rows and batch 1", fn);
    if (q->ld_s % 4 || k->ld_s % 4 || (reinterpret_cast<uintptr_t>(q->scales) & 3u) ||
        (reinterpret_cast<uintptr_t>(k->scales) & 3u))
        return fail(FP4Q_EINVAL, "%s: scale grids need 4-byte aligned rows", fn);
    if (!v || !o || !lse)
        return fail(FP4Q_EINVAL, "%s: null v, o or lse", fn);
    if (ldv < 128 || ldv % 8 || !aligned16(v))
        return fail(FP4Q_EINVAL, "%s: v needs ldv >= 128, a multiple of 8, and 16-byte alignment", fn);
    if (o_dtype != FP4Q_DT_BF16 && o_dtype != FP4Q_DT_F32)
        return fail(FP4Q_EINVAL, "%s: o_dtype %d", fn, o_dtype);
    if (ldo < 128 || ldo % 8 || !aligned16(o))
        return fail(FP4Q_EINVAL, "%s: o needs ldo >= 128, a multiple of 8, and 16-byte alignment", fn);
    if (!(scale > 0.0f) || !(scale < 1e30f))
        return fail(FP4Q_EINVAL, "%s: scale must be positive and finite", fn);
    if (causal != 0 && causal != 1)
        return fail(FP4Q_EINVAL, "%s: causal must be 0 or 1", fn);
    // the kernels address a head's rows with 32-bit element offsets
    const int64_t kHeadSlice = (int64_t)1 << 31;
    if (seq_len * q->ld >= kHeadSlice || seq_len * k->ld >= kHeadSlice || seq_len * q->ld_s >= kHeadSlice ||
        seq_len * k->ld_s >= kHeadSlice || seq_len * ldv >= kHeadSlice || seq_len * ldo >= kHeadSlice)
        return fail(FP4Q_EINVAL, "%s: seq_len x leading dimension must stay below 2^31 elements per head", fn);
    a = fp4q::AttnArgs{};
    a.qc = q->codes;
    a.ldq = q->ld;
    a.qs = q->scales;
    a.ldqs = q->ld_s;
    a.kc = k->codes;
    a.ldk = k->ld;
    a.ks = k->scales;
    a.ldks = k->ld_s;
    a.v = static_cast<const uint16_t*>(v);
    a.ldv = ldv;
    a.o = const_cast<void*>(o);
    a.ldo = ldo;
    a.lse = const_cast<float*>(lse);
    a.bh = (int)bh;
    a.L = (int)seq_len;
    a.scale = scale;
    a.causal = causal;
    a.o_bf16 = o_dtype == FP4Q_DT_BF16;
    return FP4Q_OK;
}

} // namespace

extern "C" {

int fp4q_attn_fwd(const fp4q_qtensor* q, const fp4q_qtensor* k, const void* v, int64_t ldv, void* o, int64_t ldo,
                  int o_dtype, float* lse, int64_t bh, int64_t seq_len, float scale, int causal, void* hip_stream)
{
    fp4q::AttnArgs a;
    int rc = check_attn("fp4q_attn_fwd", q, k, v, ldv, o, ldo, o_dtype, lse, bh, seq_len, scale, causal, a);
    if (rc)
        return rc;
    return hip_status(fp4q::launch_attn_fwd(a, static_cast<hipStream_t>(hip_stream)), "fp4q_attn_fwd");
}

int fp4q_attn_bwd(const fp4q_qtensor* q, const fp4q_qtensor* k, const void* v, int64_t ldv, const void* o,
                  int64_t ldo, int o_dtype, const float* lse, const void* dout, int64_t lddo, float* dq, float* dk,
                  float* dv, int64_t ldg, float* workspace, int64_t bh, int64_t seq_len, float scale, int causal,
                  void* hip_stream)
{
    fp4q::AttnArgs a;
    int rc = check_attn("fp4q_attn_bwd", q, k, v, ldv, o, ldo, o_dtype, lse, bh, seq_len, scale, causal, a);
    if (rc)
        return rc;
    if (!dout || lddo < 128 || lddo % 8 || !aligned16(dout))
        return fail(FP4Q_EINVAL, "fp4q_attn_bwd: dout needs lddo >= 128, a multiple of 8, and 16-byte alignment");
    if (!dq || !dk || !dv || ldg < 128 || ldg % 4 || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
        return fail(FP4Q_EINVAL, "fp4q_attn_bwd: dq, dk, dv need ldg >= 128, a multiple of 4, 16-byte alignment");
    if (seq_len * lddo >= ((int64_t)1 << 31) || seq_len * ldg >= ((int64_t)1 << 31))
        return fail(FP4Q_EINVAL, "fp4q_attn_bwd: seq_len x leading dimension must stay below 2^31 elements per head");
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 3u))
        return fail(FP4Q_EINVAL, "fp4q_attn_bwd: workspace of bh*seq_len floats required");
    a.dout = static_cast<const uint16_t*>(dout);
    a.lddo = lddo;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.ldg = ldg;
    a.delta = workspace;
    return hip_status(fp4q::launch_attn_bwd(a, static_cast<hipStream_t>(hip_stream)), "fp4q_attn_bwd");
}

static_assert(FP4Q_ATTN_NOALLOC_MAX_ROWS == fp4q::kAttnScratchRows, "static scratch size");

int fp4q_attn_bwd_noalloc(const fp4q_qtensor* q, const fp4q_qtensor* k, const void* v, int64_t ldv, const void* o,
                          int64_t ldo, int o_dtype, const float* lse, const void* dout, int64_t lddo, float* dq,
                          float* dk, float* dv, int64_t ldg, int64_t bh, int64_t seq_len, float scale, int causal,
                          void* hip_stream)
{
    // bh * seq_len is formed only once both factors are known small enough
    if (bh < 1 || seq_len < 1 || bh > fp4q::kAttnScratchRows || seq_len > fp4q::kAttnScratchRows / bh)
        return fail(FP4Q_EINVAL, "fp4q_attn_bwd_noalloc: bh %lld x seq_len %lld rows exceed the static scratch of "
                    "%lld rows", (long long)bh, (long long)seq_len, (long long)fp4q::kAttnScratchRows);
    float* ws = nullptr;
    hipError_t e = fp4q::attn_noalloc_scratch(&ws);
    if (e != hipSuccess)
        return hip_status(e, "fp4q_attn_bwd_noalloc: address of the static scratch");
    return fp4q_attn_bwd(q, k, v, ldv, o, ldo, o_dtype, lse, dout, lddo, dq, dk, dv, ldg, ws, bh, seq_len, scale,
                         causal, hip_stream);
}

int fp4q_probe_mfma_fp4(int64_t iters, int workgroups, float* sink, const uint8_t* codes, int64_t code_bytes,
                        void* hip_stream)
{
    if (iters < 1 || iters > ((int64_t)1 << 32) || workgroups < 1 || workgroups > (1 << 20) || !sink)
        return fail(FP4Q_EINVAL, "fp4q_probe_mfma_fp4: iters in [1, 2^32], workgroups in [1, 2^20] and a sink");
    if (codes && (code_bytes < 32 || (reinterpret_cast<uintptr_t>(codes) & 3u)))
        return fail(FP4Q_EINVAL, "fp4q_probe_mfma_fp4: codes need >= 32 bytes and 4-byte alignment");
    return hip_status(fp4q::launch_mfma_probe(iters, workgroups, sink, reinterpret_cast<const uint32_t*>(codes),
                                              codes ? code_bytes / 4 : 0, static_cast<hipStream_t>(hip_stream)),
                      "fp4q_probe_mfma_fp4");
}

int fp4q_probe_copy(const void* src, void* dst, int64_t bytes, int workgroups, void* hip_stream)
{
    if (!src || !dst || bytes < 16 || bytes % 16 || workgroups < 1 || workgroups > (1 << 20) ||
        !aligned16(src) || !aligned16(dst))
        return fail(FP4Q_EINVAL, "fp4q_probe_copy: 16-byte aligned buffers, bytes a positive multiple of 16, "
                                 "workgroups in [1, 2^20]");
    return hip_status(fp4q::launch_copy_probe(src, dst, bytes, workgroups, static_cast<hipStream_t>(hip_stream)),
                      "fp4q_probe_copy");
}

int fp4q_probe_stream(const void* src, void* dst, int64_t bytes, int nread, int workgroups, void* hip_stream)
{
    if (!src || !dst || bytes < 16 || bytes % 16 || nread < 1 || nread > 4 || workgroups < 1 ||
        workgroups > (1 << 20) || !aligned16(src) || !aligned16(dst))
        return fail(FP4Q_EINVAL, "fp4q_probe_stream: 16-byte aligned buffers, bytes a positive multiple of 16, "
                                 "nread in [1, 4], workgroups in [1, 2^20]");
    return hip_status(fp4q::launch_stream_probe(src, dst, bytes, nread, workgroups,
                                                static_cast<hipStream_t>(hip_stream)),
                      "fp4q_probe_stream");
}

int fp4q_probe_mfma_fp8(const uint8_t* a, const uint8_t* b, const uint8_t* sa, const uint8_t* sb, float* c,
                        void* hip_stream)
{
    if (!a || !b || !sa || !sb || !c || (reinterpret_cast<uintptr_t>(a) & 3u) ||
        (reinterpret_cast<uintptr_t>(b) & 3u))
        return fail(FP4Q_EINVAL, "fp4q_probe_mfma_fp8: non-null buffers, a and b 4-byte aligned");
    return hip_status(fp4q::launch_mfma_fp8_block(a, b, sa, sb, c, static_cast<hipStream_t>(hip_stream)),
                      "fp4q_probe_mfma_fp8");
}

}  // extern "C"
