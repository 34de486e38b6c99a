/*
 * fp4q_oracle.c -- plain, slow CPU oracle.  TEST INFRASTRUCTURE ONLY (see
 * fp4q_oracle.h for who may use it and which parts are parity-unpinned).
 *
 * Every step follows the definition on "Stable FP4 Training via
 * Transposition-Invariant Block Quantization" in the order the page gives
 * it; arithmetic is fp64, in which every value below is exact (E2M1, E4M3
 * and power-of-two scales have few significant bits).  No blocking, fusion or
 * reordering beyond the definitions.
 */
#include "fp4q_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <stddef.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Element formats                                                          */
/* ------------------------------------------------------------------------ */

/* E2M1 (Sec. 2: MXFP4 stores each value as E2M1, four bits): one sign bit,
 * two exponent bits with bias 1, one mantissa bit, subnormals when the
 * exponent field is 0. */
static double e2m1_magnitude(int code)
{
    int e = (code >> 1) & 3;
    int m = code & 1;
    if (e == 0)
        return 0.5 * m;
    return ldexp(1.0 + 0.5 * m, e - 1);
}

double orc_e2m1_value(int nibble)
{
    double mag = e2m1_magnitude(nibble & 7);
    return (nibble & 8) ? -mag : mag;
}

/* E4M3FN (Sec. 3.2 MXFP8): sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, subnormals at exponent 0, no infinities, S.1111.111 is NaN. */
static double e4m3_magnitude(int code)
{
    int e = (code >> 3) & 15;
    int m = code & 7;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        return ldexp((double)m, -9);
    return ldexp(1.0 + m / 8.0, e - 7);
}

double orc_e4m3_value(int byte)
{
    double mag = e4m3_magnitude(byte & 0x7f);
    return (byte & 0x80) ? -mag : mag;
}

/* Shared power-of-two scale byte: value 2^(byte - 127). */
double orc_e8m0_value(int byte)
{
    if (byte == 255)
        return NAN;
    return ldexp(1.0, byte - 127);
}

/* Sec. 3.1: S = 2^ceil(log2(2M/(Qp - Qn))).  With Qp = qmax, Qn = -qmax this
 * is 2^ceil(log2(M/qmax)): the smallest power of two that keeps M/S <= qmax,
 * i.e. nothing in the block is clipped.  The exponent is found by exact
 * comparison of M with qmax * 2^k (both exact in fp64). */
int orc_truncfree_exponent(double M, double qmax)
{
    int k;
    if (!(M > 0.0))
        return -127;
    k = ilogb(M) - ilogb(qmax);
    while (ldexp(qmax, k) < M)
        k++;
    while (ldexp(qmax, k - 1) >= M)
        k--;
    if (k < -127)
        k = -127;
    if (k > 127)
        k = 127;
    return k;
}

/* round_FP4 of Sec. 2.1 for a non-negative scaled value v.  The two
 * neighbouring grid points g_lo <= v < g_hi are found by scanning the eight
 * magnitudes.  Stochastic rounding (abstract; Sec. 3.1): the fraction
 * t = (v - g_lo)/(g_hi - g_lo) is truncated to 16 bits, F = floor(t * 2^16),
 * and v rounds up iff F + r16 >= 2^16 for the element's uniform 16-bit draw
 * r16, so P(up) = F / 2^16.  RNE: nearest, ties to the even code. */
int orc_e2m1_round(double v, int mode, uint32_t r16)
{
    int lo = -1;
    int c;
    double glo, ghi, t;
    if (!(v >= 0.0) || v > 6.0)
        return -1;
    for (c = 7; c >= 0; c--) {
        if (e2m1_magnitude(c) <= v) {
            lo = c;
            break;
        }
    }
    if (lo == 7)
        return 7; /* v == 6 exactly */
    glo = e2m1_magnitude(lo);
    ghi = e2m1_magnitude(lo + 1);
    t = (v - glo) / (ghi - glo);
    if (mode == ORC_ROUND_SR) {
        uint32_t F = (uint32_t)floor(t * 65536.0);
        return lo + ((F + (r16 & 0xffffu)) >= 65536u ? 1 : 0);
    }
    if (t > 0.5)
        return lo + 1;
    if (t < 0.5)
        return lo;
    return (lo & 1) ? lo + 1 : lo;
}

/* Round v in [0, 448] to the nearest E4M3FN magnitude, ties to even mantissa. */
int orc_e4m3_round(double v)
{
    int lo = -1;
    int c;
    double dlo, dhi;
    if (!(v >= 0.0) || v > 448.0)
        return -1;
    for (c = 126; c >= 0; c--) {
        if (e4m3_magnitude(c) <= v) {
            lo = c;
            break;
        }
    }
    if (lo == 126 || e4m3_magnitude(lo) == v)
        return lo;
    dlo = v - e4m3_magnitude(lo);
    dhi = e4m3_magnitude(lo + 1) - v;
    if (dlo < dhi)
        return lo;
    if (dhi < dlo)
        return lo + 1;
    return (lo & 1) ? lo + 1 : lo;
}

/* ------------------------------------------------------------------------ */
/* Random stream                                                            */
/* ------------------------------------------------------------------------ */

/* Philox4x32-10 as published by Salmon, Moraes, Dror and Shaw, "Parallel
 * Random Numbers: As Easy as 1, 2, 3" (SC'11): ten rounds of two 32x32->64
 * multiplications with multipliers 0xD2511F53 and 0xCD9E8D57, the high halves
 * xored with the other counter words and the round key, and a Weyl key
 * schedule with increments 0x9E3779B9 and 0xBB67AE85. */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    int round;
    for (round = 0; round < 10; round++) {
        uint64_t p0 = (uint64_t)0xD2511F53u * x0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * x2;
        uint32_t y0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0;
        uint32_t y1 = (uint32_t)p1;
        uint32_t y2 = (uint32_t)(p0 >> 32) ^ x3 ^ k1;
        uint32_t y3 = (uint32_t)p0;
        x0 = y0;
        x1 = y1;
        x2 = y2;
        x3 = y3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = x0;
    out[1] = x1;
    out[2] = x2;
    out[3] = x3;
}

/* The draw of element (r, c) is keyed by the unordered pair a = min(r, c),
 * b = max(r, c), so element (r, c) of X and element (c, r) of X^T round with
 * the same bits and quant(X^T) = quant(X)^T holds bit for bit under SR.
 * Counter = ((a mod 32)*4 + (b mod 32)/8, a/32, b/32, stream); the 16-bit
 * field is half (b mod 8) of the 128-bit output. */
void orc_sr_counter(int64_t r, int64_t c, uint32_t stream, uint32_t ctr[4], int* lane)
{
    int64_t a = r < c ? r : c;
    int64_t b = r < c ? c : r;
    ctr[0] = (uint32_t)((a % 32) * 4 + (b % 32) / 8);
    ctr[1] = (uint32_t)(a / 32);
    ctr[2] = (uint32_t)(b / 32);
    ctr[3] = stream;
    *lane = (int)(b % 8);
}

uint32_t orc_sr_bits(uint64_t seed, uint32_t stream, int64_t r, int64_t c)
{
    uint32_t ctr[4], key[2], out[4];
    int lane;
    orc_sr_counter(r, c, stream, ctr, &lane);
    key[0] = (uint32_t)seed;
    key[1] = (uint32_t)(seed >> 32);
    orc_philox4x32_10(ctr, key, out);
    return (out[lane / 2] >> (16 * (lane % 2))) & 0xffffu;
}

/* ------------------------------------------------------------------------ */
/* Quantizers                                                               */
/* ------------------------------------------------------------------------ */

static double load_elem(const void* x, int dtype, int64_t r, int64_t c, int64_t ldx)
{
    if (dtype == ORC_DT_F32)
        return (double)((const float*)x)[r * ldx + c];
    {
        uint32_t bits = (uint32_t)((const uint16_t*)x)[r * ldx + c] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
}

static int elem_sign(const void* x, int dtype, int64_t r, int64_t c, int64_t ldx)
{
    if (dtype == ORC_DT_F32) {
        float f = ((const float*)x)[r * ldx + c];
        return signbit(f) ? 1 : 0;
    }
    return (((const uint16_t*)x)[r * ldx + c] >> 15) & 1;
}

static void put_nibble(uint8_t* plane, int64_t ld, int64_t row, int64_t col, int nib)
{
    uint8_t* p = plane + row * ld + col / 2;
    int sh = (int)(col % 2) * 4;
    *p = (uint8_t)((*p & ~(0xf << sh)) | ((nib & 0xf) << sh));
}

static int64_t pad32(int64_t n) { return (n + 31) / 32 * 32; }

/* Quantize one element x with block exponent k: P = round_FP4(x / S),
 * S = 2^k (Sec. 2.1), sign carried in bit 3. */
static int quant_elem(double x, int sign, int k, int mode, uint32_t r16)
{
    double v = ldexp(fabs(x), -k);
    int code = orc_e2m1_round(v, mode, r16);
    if (code < 0)
        return -1;
    return (sign << 3) | code;
}

int orc_quant2d(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                int round_mode, uint64_t seed, uint32_t stream,
                uint8_t* codes, int64_t ld, uint8_t* codes_t, int64_t ld_t,
                uint8_t* scales, int64_t ld_s,
                int64_t tile_row_begin, int64_t tile_row_end)
{
    int64_t rows_pad = pad32(rows), cols_pad = pad32(cols);
    int64_t tr, tc, i, j;
    if (!x || rows <= 0 || cols <= 0 || ldx < cols)
        return -1;
    if ((dtype != ORC_DT_BF16 && dtype != ORC_DT_F32) ||
        (round_mode != ORC_ROUND_SR && round_mode != ORC_ROUND_RNE))
        return -1;
    if (ld < cols_pad / 2 || ld_t < rows_pad / 2 || ld_s < cols_pad / 32)
        return -1;
    if (tile_row_begin < 0) {
        tile_row_begin = 0;
        tile_row_end = rows_pad / 32;
    }
    for (tr = tile_row_begin; tr < tile_row_end; tr++) {
        for (tc = 0; tc < cols_pad / 32; tc++) {
            /* Block amax over valid entries only (appendix "Boundary blocks"). */
            double M = 0.0;
            int k;
            for (i = 32 * tr; i < 32 * tr + 32 && i < rows; i++) {
                for (j = 32 * tc; j < 32 * tc + 32 && j < cols; j++) {
                    double a = fabs(load_elem(x, dtype, i, j, ldx));
                    if (!isfinite(a))
                        return -2;
                    if (a > M)
                        M = a;
                }
            }
            k = orc_truncfree_exponent(M, 6.0);
            if (scales)
                scales[tr * ld_s + tc] = (uint8_t)(k + 127);
            for (i = 32 * tr; i < 32 * tr + 32; i++) {
                for (j = 32 * tc; j < 32 * tc + 32; j++) {
                    int nib = 0;
                    if (i < rows && j < cols) {
                        uint32_t r16 = round_mode == ORC_ROUND_SR ? orc_sr_bits(seed, stream, i, j) : 0;
                        nib = quant_elem(load_elem(x, dtype, i, j, ldx),
                                         elem_sign(x, dtype, i, j, ldx), k, round_mode, r16);
                        if (nib < 0)
                            return -3;
                    }
                    if (codes)
                        put_nibble(codes, ld, i, j, nib);
                    if (codes_t)
                        put_nibble(codes_t, ld_t, j, i, nib);
                }
            }
        }
    }
    return 0;
}

/* Square b x b blocks for b in {8, 16, 32, 64} (Sec. 3 defines the scheme
 * for any square block; Table 4 compares b = 8, 16, 32, 64).  The same
 * definition as orc_quant2d with the block side as a parameter: one scale per
 * b x b block from the amax of its valid entries, every element rounded with
 * its own random field, so the element-to-random mapping does not depend on
 * b.  The code planes keep the 32-padded shapes of orc_quant2d, and the
 * scale grid covers them: [ceil(rows_pad/b) x ld_s]; a block with no valid
 * entry has amax 0 and byte 0. */
int orc_quant2d_block(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                      int round_mode, uint64_t seed, uint32_t stream, int block,
                      uint8_t* codes, int64_t ld, uint8_t* codes_t, int64_t ld_t,
                      uint8_t* scales, int64_t ld_s)
{
    int64_t rows_pad = pad32(rows), cols_pad = pad32(cols);
    int64_t br, bc, i, j;
    if (!x || rows <= 0 || cols <= 0 || ldx < cols || (block != 8 && block != 16 && block != 32 && block != 64))
        return -1;
    if ((dtype != ORC_DT_BF16 && dtype != ORC_DT_F32) ||
        (round_mode != ORC_ROUND_SR && round_mode != ORC_ROUND_RNE))
        return -1;
    if (ld < cols_pad / 2 || ld_t < rows_pad / 2 || ld_s < (cols_pad + block - 1) / block)
        return -1;
    for (br = 0; br * block < rows_pad; br++) {
        for (bc = 0; bc * block < cols_pad; bc++) {
            double M = 0.0;
            int k;
            for (i = block * br; i < block * br + block && i < rows; i++) {
                for (j = block * bc; j < block * bc + block && j < cols; j++) {
                    double a = fabs(load_elem(x, dtype, i, j, ldx));
                    if (!isfinite(a))
                        return -2;
                    if (a > M)
                        M = a;
                }
            }
            k = orc_truncfree_exponent(M, 6.0);
            if (scales)
                scales[br * ld_s + bc] = (uint8_t)(k + 127);
            for (i = block * br; i < block * br + block && i < rows_pad; i++) {
                for (j = block * bc; j < block * bc + block && j < cols_pad; j++) {
                    int nib = 0;
                    if (i < rows && j < cols) {
                        uint32_t r16 = round_mode == ORC_ROUND_SR ? orc_sr_bits(seed, stream, i, j) : 0;
                        nib = quant_elem(load_elem(x, dtype, i, j, ldx),
                                         elem_sign(x, dtype, i, j, ldx), k, round_mode, r16);
                        if (nib < 0)
                            return -3;
                    }
                    if (codes)
                        put_nibble(codes, ld, i, j, nib);
                    if (codes_t)
                        put_nibble(codes_t, ld_t, j, i, nib);
                }
            }
        }
    }
    return 0;
}

int orc_quant1x32_fp4(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                      int round_mode, uint64_t seed, uint32_t stream,
                      uint8_t* codes, int64_t ld, uint8_t* scales, int64_t ld_s)
{
    int64_t cols_pad = pad32(cols);
    int64_t r, g, j;
    if (!x || rows <= 0 || cols <= 0 || ldx < cols || ld < cols_pad / 2 || ld_s < cols_pad / 32)
        return -1;
    for (r = 0; r < rows; r++) {
        for (g = 0; g < cols_pad / 32; g++) {
            double M = 0.0;
            int k;
            for (j = 32 * g; j < 32 * g + 32 && j < cols; j++) {
                double a = fabs(load_elem(x, dtype, r, j, ldx));
                if (!isfinite(a))
                    return -2;
                if (a > M)
                    M = a;
            }
            k = orc_truncfree_exponent(M, 6.0);
            scales[r * ld_s + g] = (uint8_t)(k + 127);
            for (j = 32 * g; j < 32 * g + 32; j++) {
                int nib = 0;
                if (j < cols) {
                    uint32_t r16 = round_mode == ORC_ROUND_SR ? orc_sr_bits(seed, stream, r, j) : 0;
                    nib = quant_elem(load_elem(x, dtype, r, j, ldx), elem_sign(x, dtype, r, j, ldx),
                                     k, round_mode, r16);
                    if (nib < 0)
                        return -3;
                }
                put_nibble(codes, ld, r, j, nib);
            }
        }
    }
    return 0;
}

int orc_quant1d_mxfp8(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                      uint8_t* codes, int64_t ld, uint8_t* scales, int64_t ld_s)
{
    int64_t cols_pad = pad32(cols);
    int64_t r, g, j;
    if (!x || rows <= 0 || cols <= 0 || ldx < cols || ld < cols_pad || ld_s < cols_pad / 32)
        return -1;
    for (r = 0; r < rows; r++) {
        for (g = 0; g < cols_pad / 32; g++) {
            double M = 0.0;
            int k;
            for (j = 32 * g; j < 32 * g + 32 && j < cols; j++) {
                double a = fabs(load_elem(x, dtype, r, j, ldx));
                if (!isfinite(a))
                    return -2;
                if (a > M)
                    M = a;
            }
            /* Sec. 3.1's rule with the E4M3 extremes Qp = 448, Qn = -448. */
            k = orc_truncfree_exponent(M, 448.0);
            scales[r * ld_s + g] = (uint8_t)(k + 127);
            for (j = 32 * g; j < 32 * g + 32; j++) {
                int byte = 0;
                if (j < cols) {
                    double v = ldexp(fabs(load_elem(x, dtype, r, j, ldx)), -k);
                    int code = orc_e4m3_round(v);
                    if (code < 0)
                        return -3;
                    byte = (elem_sign(x, dtype, r, j, ldx) << 7) | code;
                }
                codes[r * ld + j] = (uint8_t)byte;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dequantization: X_i ~ P_i * S (Sec. 2.1)                                 */
/* ------------------------------------------------------------------------ */

int orc_dequant_fp4(const uint8_t* codes, int64_t ld, const uint8_t* scales, int64_t ld_s,
                    int block_rows, int64_t rows, int64_t cols, double* out)
{
    int64_t r, c;
    if (!codes || !scales || !out || rows <= 0 || cols <= 0 || block_rows <= 0)
        return -1;
    for (r = 0; r < rows; r++) {
        for (c = 0; c < cols; c++) {
            int nib = (codes[r * ld + c / 2] >> ((c % 2) * 4)) & 0xf;
            int sb = scales[(r / block_rows) * ld_s + c / 32];
            out[r * cols + c] = orc_e2m1_value(nib) * orc_e8m0_value(sb);
        }
    }
    return 0;
}

/* Dequantization with a block_rows x block_cols scale grid (32 x 32 or
 * 64 x 64 for the square layouts, 1 x 32 for the row layout). */
int orc_dequant_fp4_blocks(const uint8_t* codes, int64_t ld, const uint8_t* scales, int64_t ld_s,
                           int block_rows, int block_cols, int64_t rows, int64_t cols, double* out)
{
    int64_t r, c;
    if (!codes || !scales || !out || rows <= 0 || cols <= 0 || block_rows <= 0 || block_cols <= 0)
        return -1;
    for (r = 0; r < rows; r++) {
        for (c = 0; c < cols; c++) {
            int nib = (codes[r * ld + c / 2] >> ((c % 2) * 4)) & 0xf;
            int sb = scales[(r / block_rows) * ld_s + c / block_cols];
            out[r * cols + c] = orc_e2m1_value(nib) * orc_e8m0_value(sb);
        }
    }
    return 0;
}

int orc_dequant_mxfp8(const uint8_t* codes, int64_t ld, const uint8_t* scales, int64_t ld_s,
                      int64_t rows, int64_t cols, double* out)
{
    int64_t r, c;
    if (!codes || !scales || !out || rows <= 0 || cols <= 0)
        return -1;
    for (r = 0; r < rows; r++)
        for (c = 0; c < cols; c++)
            out[r * cols + c] = orc_e4m3_value(codes[r * ld + c]) * orc_e8m0_value(scales[r * ld_s + c / 32]);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Linear-layer GEMMs, Sec. 3 "Application to linear layers":               */
/*   Y = X W^T,  dX = dY W,  dW = dY^T X                                    */
/* ------------------------------------------------------------------------ */

static int gemm_shape(int op, int64_t a_rows, int64_t a_cols, int64_t b_rows, int64_t b_cols,
                      int64_t* m, int64_t* n, int64_t* kk)
{
    if (a_rows <= 0 || a_cols <= 0 || b_rows <= 0 || b_cols <= 0)
        return -1;
    switch (op) {
    case ORC_OP_FWD: /* X [T x K], W [N x K] -> [T x N] */
        if (a_cols != b_cols)
            return -1;
        *m = a_rows; *n = b_rows; *kk = a_cols;
        return 0;
    case ORC_OP_DGRAD: /* dY [T x N], W [N x K] -> [T x K] */
        if (a_cols != b_rows)
            return -1;
        *m = a_rows; *n = b_cols; *kk = a_cols;
        return 0;
    case ORC_OP_WGRAD: /* dY [T x N], X [T x K] -> [N x K] */
        if (a_rows != b_rows)
            return -1;
        *m = a_cols; *n = b_cols; *kk = a_rows;
        return 0;
    }
    return -1;
}

static void gemm_one(int op, const double* A, int64_t a_cols, const double* B, int64_t b_cols,
                     int64_t kk, int64_t i, int64_t j, double* c_out, double* b_out)
{
    double acc = 0.0, bnd = 0.0;
    int64_t t;
    for (t = 0; t < kk; t++) {
        double a, b;
        if (op == ORC_OP_FWD) {        /* sum_k X[i,k] W[j,k] */
            a = A[i * a_cols + t];
            b = B[j * b_cols + t];
        } else if (op == ORC_OP_DGRAD) { /* sum_n dY[i,n] W[n,j] */
            a = A[i * a_cols + t];
            b = B[t * b_cols + j];
        } else {                       /* sum_t dY[t,i] X[t,j] */
            a = A[t * a_cols + i];
            b = B[t * b_cols + j];
        }
        acc += a * b;
        bnd += fabs(a) * fabs(b);
    }
    *c_out = acc;
    if (b_out)
        *b_out = bnd;
}

int orc_gemm(int op, const double* A, int64_t a_rows, int64_t a_cols,
             const double* B, int64_t b_rows, int64_t b_cols,
             double* C, double* bound)
{
    int64_t m, n, kk, i, j;
    if (!A || !B || !C || gemm_shape(op, a_rows, a_cols, b_rows, b_cols, &m, &n, &kk))
        return -1;
    for (i = 0; i < m; i++)
        for (j = 0; j < n; j++)
            gemm_one(op, A, a_cols, B, b_cols, kk, i, j, &C[i * n + j], bound ? &bound[i * n + j] : NULL);
    return 0;
}

int orc_gemm_sampled(int op, const double* A, int64_t a_rows, int64_t a_cols,
                     const double* B, int64_t b_rows, int64_t b_cols,
                     int64_t n, const int64_t* ci, const int64_t* cj,
                     double* C, double* bound)
{
    int64_t m, nn, kk, s;
    if (!A || !B || !C || !ci || !cj || gemm_shape(op, a_rows, a_cols, b_rows, b_cols, &m, &nn, &kk))
        return -1;
    for (s = 0; s < n; s++) {
        if (ci[s] < 0 || ci[s] >= m || cj[s] < 0 || cj[s] >= nn)
            return -1;
        gemm_one(op, A, a_cols, B, b_cols, kk, ci[s], cj[s], &C[s], bound ? &bound[s] : NULL);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention with MXFP8 queries and keys (Sec. 3.2 "MXFP8 Attention" and    */
/* Fig. 3: Q and K enter the score product in MXFP8; the appendix           */
/* "Attention").  One head at a time; Q, K are the dequantized MXFP8 values */
/* (exact in fp64), V and dO as given.  Standard scaled dot-product          */
/* attention, written out:                                                   */
/*   s_ij = scale * sum_d Q_id K_jd          (j <= i when causal)            */
/*   P_ij = exp(s_ij - m_i) / l_i,  m_i = max_j s_ij,  l_i = sum_j exp(...)  */
/*   O_i  = sum_j P_ij V_j,         lse_i = m_i + log(l_i)                   */
/* and its gradient for a loss with dL/dO = dO:                              */
/*   dV_j = sum_i P_ij dO_i,  dP_ij = sum_d dO_id V_jd,                      */
/*   D_i = sum_d dO_id O_id,  dS_ij = P_ij (dP_ij - D_i),                    */
/*   dQ_i = scale sum_j dS_ij K_j,  dK_j = scale sum_i dS_ij Q_i.            */
/* ------------------------------------------------------------------------ */

static double attn_score(const double* Q, const double* K, int64_t d, int64_t i, int64_t j, double scale)
{
    double acc = 0.0;
    int64_t t;
    for (t = 0; t < d; t++)
        acc += Q[i * d + t] * K[j * d + t];
    return scale * acc;
}

/* Softmax statistics of query row i: m_i and l_i over its visible keys. */
static void attn_row_stats(const double* Q, const double* K, int64_t L, int64_t d, double scale, int causal,
                           int64_t i, double* m_out, double* l_out)
{
    int64_t j, jend = causal ? i + 1 : L;
    double m = -INFINITY, l = 0.0;
    for (j = 0; j < jend; j++) {
        double sv = attn_score(Q, K, d, i, j, scale);
        if (sv > m)
            m = sv;
    }
    for (j = 0; j < jend; j++)
        l += exp(attn_score(Q, K, d, i, j, scale) - m);
    *m_out = m;
    *l_out = l;
}

/* O_i = sum_j P_ij V_j and oa_i = sum_j P_ij |V_j| over keys [0, jend). */
static void attn_row_out(const double* Q, const double* K, const double* V, int64_t d, double scale, int64_t i,
                         int64_t jend, double m, double l, double* o, double* oa)
{
    int64_t j, t;
    for (t = 0; t < d; t++) {
        o[t] = 0.0;
        oa[t] = 0.0;
    }
    for (j = 0; j < jend; j++) {
        double pij = exp(attn_score(Q, K, d, i, j, scale) - m) / l;
        for (t = 0; t < d; t++) {
            o[t] += pij * V[j * d + t];
            oa[t] += pij * fabs(V[j * d + t]);
        }
    }
}

int orc_attn_fwd_rows(const double* Q, const double* K, const double* V, int64_t L, int64_t d, double scale,
                      int causal, int64_t nrows, const int64_t* rows, double* O, double* lse, double* pv_abs)
{
    int64_t r, j, t;
    if (!Q || !K || !V || !rows || !O || L <= 0 || d <= 0 || nrows < 0)
        return -1;
    for (r = 0; r < nrows; r++) {
        int64_t i = rows[r], jend;
        double m, l;
        if (i < 0 || i >= L)
            return -1;
        attn_row_stats(Q, K, L, d, scale, causal, i, &m, &l);
        for (t = 0; t < d; t++) {
            O[r * d + t] = 0.0;
            if (pv_abs)
                pv_abs[r * d + t] = 0.0;
        }
        jend = causal ? i + 1 : L;
        for (j = 0; j < jend; j++) {
            double pij = exp(attn_score(Q, K, d, i, j, scale) - m) / l;
            for (t = 0; t < d; t++) {
                O[r * d + t] += pij * V[j * d + t];
                if (pv_abs)
                    pv_abs[r * d + t] += pij * fabs(V[j * d + t]);
            }
        }
        if (lse)
            lse[r] = m + log(l);
    }
    return 0;
}

/* dQ of selected query rows (self-contained per row: P_i, dP_i and D_i are
 * formed from the row's own softmax).  Also returns, per row and feature,
 * the magnitudes the GPU's rounding acts on:
 *   ds_abs_k[r][t] = scale * sum_j |dS_ij| |K_jt|
 *   p_abs_k[r][t]  = scale * sum_j P_ij (|dP_ij| + |D_i|) |K_jt|
 *   p_k[r][t]      = scale * sum_j P_ij |K_jt|
 * and dvo[r] = sum_t |dO_it| * sum_j P_ij |V_jt| (the size of D's error). */
int orc_attn_bwd_dq_rows(const double* Q, const double* K, const double* V, const double* dO, int64_t L, int64_t d,
                         double scale, int causal, int64_t nrows, const int64_t* rows, double* dQ,
                         double* ds_abs_k, double* p_abs_k, double* p_k, double* dvo)
{
    int64_t r, j, t;
    double *orow, *oarow;
    int rc = 0;
    if (!Q || !K || !V || !dO || !rows || !dQ || L <= 0 || d <= 0 || nrows < 0)
        return -1;
    orow = (double*)malloc(2 * (size_t)d * sizeof(double));
    if (!orow)
        return -4;
    oarow = orow + d;
    for (r = 0; r < nrows; r++) {
        int64_t i = rows[r], jend;
        double m, l, D = 0.0, pvo = 0.0;
        if (i < 0 || i >= L) {
            rc = -1;
            break;
        }
        attn_row_stats(Q, K, L, d, scale, causal, i, &m, &l);
        jend = causal ? i + 1 : L;
        /* D_i = sum_t dO_it O_it, O_i = sum_j P_ij V_j */
        attn_row_out(Q, K, V, d, scale, i, jend, m, l, orow, oarow);
        for (t = 0; t < d; t++) {
            D += dO[i * d + t] * orow[t];
            pvo += fabs(dO[i * d + t]) * oarow[t];
        }
        for (t = 0; t < d; t++) {
            dQ[r * d + t] = 0.0;
            if (ds_abs_k) {
                ds_abs_k[r * d + t] = 0.0;
                p_abs_k[r * d + t] = 0.0;
                p_k[r * d + t] = 0.0;
            }
        }
        for (j = 0; j < jend; j++) {
            double pij = exp(attn_score(Q, K, d, i, j, scale) - m) / l;
            double dp = 0.0, dsij;
            for (t = 0; t < d; t++)
                dp += dO[i * d + t] * V[j * d + t];
            dsij = pij * (dp - D);
            for (t = 0; t < d; t++) {
                dQ[r * d + t] += scale * dsij * K[j * d + t];
                if (ds_abs_k) {
                    ds_abs_k[r * d + t] += scale * fabs(dsij) * fabs(K[j * d + t]);
                    p_abs_k[r * d + t] += scale * pij * (fabs(dp) + fabs(D)) * fabs(K[j * d + t]);
                    p_k[r * d + t] += scale * pij * fabs(K[j * d + t]);
                }
            }
        }
        if (dvo)
            dvo[r] = pvo;
    }
    free(orow);
    return rc;
}

/* Softmax statistics m_i, l_i of query rows [i0, i1), and, when dO is
 * given, D_i = sum_t dO_it O_it and dvo_i = sum_t |dO_it| sum_j P_ij |V_jt|. */
int orc_attn_stats(const double* Q, const double* K, const double* V, const double* dO, int64_t L, int64_t d,
                   double scale, int causal, int64_t i0, int64_t i1, double* mv, double* lv, double* Dv, double* dvo)
{
    int64_t i, t;
    double *orow, *oarow;
    if (!Q || !K || !V || !mv || !lv || L <= 0 || d <= 0 || i0 < 0 || i1 > L || i0 > i1)
        return -1;
    orow = (double*)malloc(2 * (size_t)d * sizeof(double));
    if (!orow)
        return -4;
    oarow = orow + d;
    for (i = i0; i < i1; i++) {
        int64_t jend = causal ? i + 1 : L;
        attn_row_stats(Q, K, L, d, scale, causal, i, &mv[i], &lv[i]);
        if (!dO)
            continue;
        attn_row_out(Q, K, V, d, scale, i, jend, mv[i], lv[i], orow, oarow);
        Dv[i] = 0.0;
        dvo[i] = 0.0;
        for (t = 0; t < d; t++) {
            Dv[i] += dO[i * d + t] * orow[t];
            dvo[i] += fabs(dO[i * d + t]) * oarow[t];
        }
    }
    free(orow);
    return 0;
}

/* dK and dV of selected key rows, from every query's statistics (m, l, D and
 * dvo of orc_attn_stats): the sums run over the queries that see key j.
 * Magnitudes for the tolerances:
 *   ds_abs_q[r][t] = scale * sum_i |dS_ij| |Q_it|
 *   p_abs_q[r][t]  = scale * sum_i P_ij (|dP_ij| + |D_i|) |Q_it|
 *   pd_q[r][t]     = scale * sum_i P_ij dvo_i |Q_it|
 *   p_q[r][t]      = scale * sum_i P_ij |Q_it|
 *   p_do[r][t]     = sum_i P_ij |dO_it|                 (dV's) */
int orc_attn_bwd_dkdv_rows(const double* Q, const double* K, const double* V, const double* dO, int64_t L, int64_t d,
                           double scale, int causal, const double* mv, const double* lv, const double* Dv,
                           const double* dvo, int64_t nrows, const int64_t* rows, double* dK, double* dV,
                           double* ds_abs_q, double* p_abs_q, double* pd_q, double* p_q, double* p_do)
{
    int64_t r, i, j, t;
    if (!Q || !K || !V || !dO || !rows || !dK || !dV || !mv || !lv || !Dv || !dvo || L <= 0 || d <= 0 || nrows < 0)
        return -1;
    for (r = 0; r < nrows; r++) {
        j = rows[r];
        if (j < 0 || j >= L)
            return -1;
        for (t = 0; t < d; t++) {
            dK[r * d + t] = 0.0;
            dV[r * d + t] = 0.0;
            if (ds_abs_q) {
                ds_abs_q[r * d + t] = 0.0;
                p_abs_q[r * d + t] = 0.0;
                pd_q[r * d + t] = 0.0;
                p_q[r * d + t] = 0.0;
                p_do[r * d + t] = 0.0;
            }
        }
        for (i = causal ? j : 0; i < L; i++) {
            double pij = exp(attn_score(Q, K, d, i, j, scale) - mv[i]) / lv[i];
            double dp = 0.0, dsij;
            for (t = 0; t < d; t++)
                dp += dO[i * d + t] * V[j * d + t];
            dsij = pij * (dp - Dv[i]);
            for (t = 0; t < d; t++) {
                dK[r * d + t] += scale * dsij * Q[i * d + t];
                dV[r * d + t] += pij * dO[i * d + t];
                if (ds_abs_q) {
                    ds_abs_q[r * d + t] += scale * fabs(dsij) * fabs(Q[i * d + t]);
                    p_abs_q[r * d + t] += scale * pij * (fabs(dp) + fabs(Dv[i])) * fabs(Q[i * d + t]);
                    pd_q[r * d + t] += scale * pij * dvo[i] * fabs(Q[i * d + t]);
                    p_q[r * d + t] += scale * pij * fabs(Q[i * d + t]);
                    p_do[r * d + t] += pij * fabs(dO[i * d + t]);
                }
            }
        }
    }
    return 0;
}
