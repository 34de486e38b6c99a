"""ctypes binding of the CPU oracle (oracle/fp4q_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library does not.

Arrays are numpy: bf16 tensors travel as uint16 bit patterns, fp32 as
float32.  Plane shapes follow the library convention:
    codes   [rows_pad, cols_pad // 2]  (row plane, low nibble = even column)
    codes_t [cols_pad, rows_pad // 2]  (transposed plane)
    scales  [rows_pad // 32, cols_pad // 32]  E8M0 bytes
with rows_pad / cols_pad rounded up to multiples of 32.
"""
import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import build as _build

DT_BF16, DT_F32 = 1, 2
ROUND_SR, ROUND_RNE = 0, 1
OP_FWD, OP_DGRAD, OP_WGRAD = 0, 1, 2
OPS = {"fwd": OP_FWD, "dgrad": OP_DGRAD, "wgrad": OP_WGRAD}

_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def lib():
    """Load the oracle library, building it first if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e2m1_value.argtypes = [ctypes.c_int]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_int]
        L.orc_e8m0_value.restype = ctypes.c_double
        L.orc_e8m0_value.argtypes = [ctypes.c_int]
        L.orc_truncfree_exponent.restype = ctypes.c_int
        L.orc_truncfree_exponent.argtypes = [ctypes.c_double, ctypes.c_double]
        L.orc_e2m1_round.restype = ctypes.c_int
        L.orc_e2m1_round.argtypes = [ctypes.c_double, ctypes.c_int, ctypes.c_uint32]
        L.orc_e4m3_round.restype = ctypes.c_int
        L.orc_e4m3_round.argtypes = [ctypes.c_double]
        L.orc_philox4x32_10.restype = None
        L.orc_philox4x32_10.argtypes = [_P, _P, _P]
        L.orc_sr_counter.restype = None
        L.orc_sr_counter.argtypes = [_I64, _I64, ctypes.c_uint32, _P, _P]
        L.orc_sr_bits.restype = ctypes.c_uint32
        L.orc_sr_bits.argtypes = [ctypes.c_uint64, ctypes.c_uint32, _I64, _I64]
        L.orc_quant2d.restype = ctypes.c_int
        L.orc_quant2d.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, ctypes.c_int, ctypes.c_uint64,
                                  ctypes.c_uint32, _P, _I64, _P, _I64, _P, _I64, _I64, _I64]
        L.orc_quant2d_block.restype = ctypes.c_int
        L.orc_quant2d_block.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, ctypes.c_int,
                                        ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, _P, _I64, _P,
                                        _I64, _P, _I64]
        L.orc_dequant_fp4_blocks.restype = ctypes.c_int
        L.orc_dequant_fp4_blocks.argtypes = [_P, _I64, _P, _I64, ctypes.c_int, ctypes.c_int, _I64, _I64,
                                             _P]
        L.orc_quant1x32_fp4.restype = ctypes.c_int
        L.orc_quant1x32_fp4.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, ctypes.c_int,
                                        ctypes.c_uint64, ctypes.c_uint32, _P, _I64, _P, _I64]
        L.orc_quant1d_mxfp8.restype = ctypes.c_int
        L.orc_quant1d_mxfp8.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, _P, _I64, _P, _I64]
        L.orc_dequant_fp4.restype = ctypes.c_int
        L.orc_dequant_fp4.argtypes = [_P, _I64, _P, _I64, ctypes.c_int, _I64, _I64, _P]
        L.orc_dequant_mxfp8.restype = ctypes.c_int
        L.orc_dequant_mxfp8.argtypes = [_P, _I64, _P, _I64, _I64, _I64, _P]
        L.orc_gemm.restype = ctypes.c_int
        L.orc_gemm.argtypes = [ctypes.c_int, _P, _I64, _I64, _P, _I64, _I64, _P, _P]
        L.orc_gemm_sampled.restype = ctypes.c_int
        L.orc_gemm_sampled.argtypes = [ctypes.c_int, _P, _I64, _I64, _P, _I64, _I64, _I64, _P, _P,
                                       _P, _P]
        D = ctypes.c_double
        L.orc_attn_fwd_rows.restype = ctypes.c_int
        L.orc_attn_fwd_rows.argtypes = [_P, _P, _P, _I64, _I64, D, ctypes.c_int, _I64, _P, _P, _P, _P]
        L.orc_attn_stats.restype = ctypes.c_int
        L.orc_attn_stats.argtypes = [_P, _P, _P, _P, _I64, _I64, D, ctypes.c_int, _I64, _I64, _P, _P, _P, _P]
        L.orc_attn_bwd_dq_rows.restype = ctypes.c_int
        L.orc_attn_bwd_dq_rows.argtypes = [_P, _P, _P, _P, _I64, _I64, D, ctypes.c_int, _I64, _P, _P, _P, _P,
                                           _P, _P]
        L.orc_attn_bwd_dkdv_rows.restype = ctypes.c_int
        L.orc_attn_bwd_dkdv_rows.argtypes = [_P, _P, _P, _P, _I64, _I64, D, ctypes.c_int, _P, _P, _P, _P, _I64,
                                             _P, _P, _P, _P, _P, _P, _P, _P]
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def pad32(n):
    return (n + 31) // 32 * 32


def _dtype_of(x):
    if x.dtype == np.uint16:
        return DT_BF16
    if x.dtype == np.float32:
        return DT_F32
    raise TypeError("oracle inputs are uint16 (bf16 bits) or float32, got %s" % x.dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s failed with code %d" % (what, rc))


# -- element-level entry points -------------------------------------------------

def e2m1_value(nibble):
    return lib().orc_e2m1_value(int(nibble))


def e4m3_value(byte):
    return lib().orc_e4m3_value(int(byte))


def e8m0_value(byte):
    return lib().orc_e8m0_value(int(byte))


def truncfree_exponent(M, qmax=6.0):
    return lib().orc_truncfree_exponent(float(M), float(qmax))


def e2m1_round(v, mode=ROUND_SR, r16=0):
    return lib().orc_e2m1_round(float(v), int(mode), int(r16))


def e4m3_round(v):
    return lib().orc_e4m3_round(float(v))


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_counter(r, c, stream):
    ctr = np.zeros(4, dtype=np.uint32)
    lane = ctypes.c_int(0)
    lib().orc_sr_counter(int(r), int(c), int(stream), _ptr(ctr), ctypes.byref(lane))
    return ctr, lane.value


def sr_bits(seed, stream, r, c):
    return lib().orc_sr_bits(int(seed), int(stream), int(r), int(c))


# -- quantizers ------------------------------------------------------------------

def quant2d(x, round_mode=ROUND_SR, seed=0, stream=0, threads=None, tile_rows=None):
    """2D 32x32-block FP4 quantization; returns (codes, codes_t, scales).

    tile_rows=(lo, hi) restricts the work to tile rows [lo, hi) (rows
    32*lo .. 32*hi-1 of the row plane, bytes 16*lo .. 16*hi-1 of every
    transposed-plane row); the rest of the outputs stays zero."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    rp, cp = pad32(rows), pad32(cols)
    codes = np.zeros((rp, cp // 2), dtype=np.uint8)
    codes_t = np.zeros((cp, rp // 2), dtype=np.uint8)
    scales = np.zeros((rp // 32, cp // 32), dtype=np.uint8)
    dt = _dtype_of(x)
    t0, t1 = (0, rp // 32) if tile_rows is None else tile_rows
    ntr = t1 - t0
    nthreads = threads or min(16, os.cpu_count() or 1)
    nthreads = max(1, min(nthreads, ntr))

    def run(lo, hi):
        return lib().orc_quant2d(_ptr(x), dt, rows, cols, cols, int(round_mode), int(seed),
                                 int(stream), _ptr(codes), cp // 2, _ptr(codes_t), rp // 2,
                                 _ptr(scales), cp // 32, lo, hi)

    if nthreads == 1:
        _check(run(t0, t1), "quant2d")
    else:
        bounds = [(t0 + ntr * i // nthreads, t0 + ntr * (i + 1) // nthreads)
                  for i in range(nthreads)]
        with ThreadPoolExecutor(nthreads) as ex:
            for rc in ex.map(lambda b: run(*b), bounds):
                _check(rc, "quant2d")
    return codes, codes_t, scales


def quant2d_block(x, block, round_mode=ROUND_SR, seed=0, stream=0):
    """Square block x block FP4 quantization (block 8, 16, 32 or 64); returns
    (codes, codes_t, scales) with the scale grid [ceil(R/b) x ceil(C/b)], R
    and C the shape rounded up to 32 (blocks with no valid entry: byte 0)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    rp, cp = pad32(rows), pad32(cols)
    nbr, nbc = -(-rp // block), -(-cp // block)
    codes = np.zeros((rp, cp // 2), dtype=np.uint8)
    codes_t = np.zeros((cp, rp // 2), dtype=np.uint8)
    scales = np.zeros((nbr, nbc), dtype=np.uint8)
    _check(lib().orc_quant2d_block(_ptr(x), _dtype_of(x), rows, cols, cols, int(round_mode), int(seed),
                                   int(stream), int(block), _ptr(codes), cp // 2, _ptr(codes_t), rp // 2,
                                   _ptr(scales), nbc), "quant2d_block")
    return codes, codes_t, scales


def dequant_fp4_blocks(codes, scales, rows, cols, block_rows, block_cols):
    """A code plane times its block_rows x block_cols scale grid, in fp64."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.empty((rows, cols), dtype=np.float64)
    _check(lib().orc_dequant_fp4_blocks(_ptr(codes), codes.shape[1], _ptr(scales), scales.shape[1],
                                        int(block_rows), int(block_cols), rows, cols, _ptr(out)),
           "dequant_fp4_blocks")
    return out


def quant1x32_fp4(x, round_mode=ROUND_SR, seed=0, stream=0):
    """Conventional 1x32 FP4 quantization along rows; returns (codes, scales)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    cp = pad32(cols)
    codes = np.zeros((rows, cp // 2), dtype=np.uint8)
    scales = np.zeros((rows, cp // 32), dtype=np.uint8)
    _check(lib().orc_quant1x32_fp4(_ptr(x), _dtype_of(x), rows, cols, cols, int(round_mode),
                                   int(seed), int(stream), _ptr(codes), cp // 2, _ptr(scales),
                                   cp // 32), "quant1x32_fp4")
    return codes, scales


def quant_act1d(x, round_mode=ROUND_SR, seed=0, stream=0):
    """1D (1x32) FP4 layout of an activation matrix X [rows x cols] for the
    three products of a linear layer (appendix "Activations": activations are
    quantized in 1D blocks along the hidden channels).  The forward product
    contracts over the channels, so its plane is X quantized in 1x32 blocks
    along its rows; the weight-gradient product contracts over the tokens, so
    its plane is X^T quantized in 1x32 blocks along its rows (32 tokens of one
    channel).  Each element keeps its one random field (the field of the
    unordered pair (r, c)) in both planes.

    Returns (codes [R x C/2], codes_t [C x R/2], scales [R x C/32],
    scales_t [C x R/32]) with R, C = rows, cols rounded up to 32; rows and
    columns in the padding hold code 0 and scale byte 0."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    rp, cp = pad32(rows), pad32(cols)
    codes = np.zeros((rp, cp // 2), dtype=np.uint8)
    codes_t = np.zeros((cp, rp // 2), dtype=np.uint8)
    scales = np.zeros((rp, cp // 32), dtype=np.uint8)
    scales_t = np.zeros((cp, rp // 32), dtype=np.uint8)
    c, s = quant1x32_fp4(x, round_mode, seed, stream)
    ct, st = quant1x32_fp4(np.ascontiguousarray(x.T), round_mode, seed, stream)
    codes[:rows] = c
    scales[:rows] = s
    codes_t[:cols] = ct
    scales_t[:cols] = st
    return codes, codes_t, scales, scales_t


def quant1d_mxfp8(x):
    """MXFP8 E4M3 with 1x32 blocks along rows; returns (codes, scales)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    cp = pad32(cols)
    codes = np.zeros((rows, cp), dtype=np.uint8)
    scales = np.zeros((rows, cp // 32), dtype=np.uint8)
    _check(lib().orc_quant1d_mxfp8(_ptr(x), _dtype_of(x), rows, cols, cols, _ptr(codes), cp,
                                   _ptr(scales), cp // 32), "quant1d_mxfp8")
    return codes, scales


def dequant_fp4(codes, scales, rows, cols, block_rows=32):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.empty((rows, cols), dtype=np.float64)
    _check(lib().orc_dequant_fp4(_ptr(codes), codes.shape[1], _ptr(scales), scales.shape[1],
                                 int(block_rows), rows, cols, _ptr(out)), "dequant_fp4")
    return out


def dequant_mxfp8(codes, scales, rows, cols):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.empty((rows, cols), dtype=np.float64)
    _check(lib().orc_dequant_mxfp8(_ptr(codes), codes.shape[1], _ptr(scales), scales.shape[1],
                                   rows, cols, _ptr(out)), "dequant_mxfp8")
    return out


# -- GEMMs -----------------------------------------------------------------------

def _out_shape(op, A, B):
    if op == OP_FWD:
        return A.shape[0], B.shape[0]
    if op == OP_DGRAD:
        return A.shape[0], B.shape[1]
    return A.shape[1], B.shape[1]


def gemm(op, A, B):
    """fp64 GEMM of a linear layer on dequantized operands; returns (C, bound)."""
    op = OPS.get(op, op)
    A = np.ascontiguousarray(A, dtype=np.float64)
    B = np.ascontiguousarray(B, dtype=np.float64)
    m, n = _out_shape(op, A, B)
    C = np.empty((m, n), dtype=np.float64)
    bound = np.empty((m, n), dtype=np.float64)
    _check(lib().orc_gemm(op, _ptr(A), A.shape[0], A.shape[1], _ptr(B), B.shape[0], B.shape[1],
                          _ptr(C), _ptr(bound)), "gemm")
    return C, bound


def gemm_sampled(op, A, B, ci, cj):
    """The same products at sampled coordinates; returns (C[s], bound[s])."""
    op = OPS.get(op, op)
    A = np.ascontiguousarray(A, dtype=np.float64)
    B = np.ascontiguousarray(B, dtype=np.float64)
    ci = np.ascontiguousarray(ci, dtype=np.int64)
    cj = np.ascontiguousarray(cj, dtype=np.int64)
    C = np.empty(len(ci), dtype=np.float64)
    bound = np.empty(len(ci), dtype=np.float64)
    _check(lib().orc_gemm_sampled(op, _ptr(A), A.shape[0], A.shape[1], _ptr(B), B.shape[0],
                                  B.shape[1], len(ci), _ptr(ci), _ptr(cj), _ptr(C), _ptr(bound)),
           "gemm_sampled")
    return C, bound


# -- attention (Sec. 3.2: MXFP8 queries and keys) ----------------------------------

def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _split(n, parts):
    parts = max(1, min(parts, n))
    return [(n * i // parts, n * (i + 1) // parts) for i in range(parts)]


def _threads(threads):
    return threads or min(16, os.cpu_count() or 1)


def attn_fwd(Q, K, V, scale, causal, rows=None, threads=None):
    """One head: O [len(rows) x d], lse [len(rows)] (natural log) and
    pv_abs = sum_j P_ij |V_jt|, for the selected query rows (default all).
    Q, K are the dequantized MXFP8 values."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    L, d = Q.shape
    rows = np.arange(L, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = len(rows)
    O = np.zeros((n, d))
    lse = np.zeros(n)
    pv = np.zeros((n, d))

    def run(b):
        lo, hi = b
        if hi <= lo:
            return 0
        return lib().orc_attn_fwd_rows(_ptr(Q), _ptr(K), _ptr(V), L, d, float(scale), int(causal), hi - lo,
                                       _ptr(rows[lo:]), _ptr(O[lo:]), _ptr(lse[lo:]), _ptr(pv[lo:]))

    with ThreadPoolExecutor(_threads(threads)) as ex:
        for rc in ex.map(run, _split(n, _threads(threads))):
            _check(rc, "attn_fwd")
    return O, lse, pv


def attn_bwd_dq(Q, K, V, dO, scale, causal, rows=None, threads=None):
    """One head: dQ of the selected query rows and its tolerance magnitudes
    (ds_abs_k, p_abs_k, p_k per row and feature; dvo per row)."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    L, d = Q.shape
    rows = np.arange(L, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = len(rows)
    dQ, a, b, c = (np.zeros((n, d)) for _ in range(4))
    dvo = np.zeros(n)

    def run(bd):
        lo, hi = bd
        if hi <= lo:
            return 0
        return lib().orc_attn_bwd_dq_rows(_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), L, d, float(scale), int(causal),
                                          hi - lo, _ptr(rows[lo:]), _ptr(dQ[lo:]), _ptr(a[lo:]), _ptr(b[lo:]),
                                          _ptr(c[lo:]), _ptr(dvo[lo:]))

    with ThreadPoolExecutor(_threads(threads)) as ex:
        for rc in ex.map(run, _split(n, _threads(threads))):
            _check(rc, "attn_bwd_dq")
    return dQ, {"ds_abs_k": a, "p_abs_k": b, "p_k": c, "dvo": dvo}


def attn_bwd_dkdv(Q, K, V, dO, scale, causal, rows=None, threads=None):
    """One head: dK, dV of the selected key rows and their tolerance
    magnitudes (ds_abs_q, p_abs_q, pd_q, p_q, p_do per row and feature)."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    L, d = Q.shape
    rows = np.arange(L, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = len(rows)
    mv, lv, Dv, dvo = (np.zeros(L) for _ in range(4))
    nt = _threads(threads)

    def stats(bd):
        lo, hi = bd
        if hi <= lo:
            return 0
        return lib().orc_attn_stats(_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), L, d, float(scale), int(causal), lo, hi,
                                    _ptr(mv), _ptr(lv), _ptr(Dv), _ptr(dvo))

    dK, dV, a, b, c, f, e = (np.zeros((n, d)) for _ in range(7))

    def run(bd):
        lo, hi = bd
        if hi <= lo:
            return 0
        return lib().orc_attn_bwd_dkdv_rows(_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), L, d, float(scale), int(causal),
                                            _ptr(mv), _ptr(lv), _ptr(Dv), _ptr(dvo), hi - lo, _ptr(rows[lo:]),
                                            _ptr(dK[lo:]), _ptr(dV[lo:]), _ptr(a[lo:]), _ptr(b[lo:]), _ptr(c[lo:]),
                                            _ptr(f[lo:]), _ptr(e[lo:]))

    with ThreadPoolExecutor(nt) as ex:
        for rc in ex.map(stats, _split(L, nt)):
            _check(rc, "attn_stats")
        for rc in ex.map(run, _split(n, nt)):
            _check(rc, "attn_bwd_dkdv")
    return dK, dV, {"ds_abs_q": a, "p_abs_q": b, "pd_q": c, "p_q": f, "p_do": e}
