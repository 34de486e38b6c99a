"""Python binding of libfp4q (MI355X / gfx950).

Argument marshalling only: every step of the quantizer and the GEMMs runs in
the library's HIP kernels.  torch supplies device memory and the current
stream.  The functions carry the C entry points' names:

    fp4q_quant2d        2D 32x32-block FP4 quantization (row + transposed plane)
    fp4q_quant1d_mxfp8  MXFP8 E4M3 1x32 quantization
    fp4q_gemm           block-scaled GEMM, op "fwd" | "dgrad" | "wgrad"
    fp4q_dequant        dequantization to fp32 / bf16
    fp4q_quant2d_sizes  output sizes of fp4q_quant2d

If libfp4q.so has not been built, every call raises: there is no fallback.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

__all__ = ["QTensor", "fp4q_quant2d", "fp4q_quant1d_mxfp8", "fp4q_gemm", "fp4q_dequant",
           "fp4q_quant2d_sizes", "alloc_fp4", "alloc_mxfp8", "library_path", "Fp4qError"]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp4q.so")

FMT_FP4_2D32, FMT_MXFP8_1D32, FMT_FP4_2D64, FMT_FP4_1D32 = 1, 2, 3, 4
DT_BF16, DT_F32 = 1, 2
ROUND = {"sr": 0, "rne": 1}
OPS = {"fwd": 0, "dgrad": 1, "wgrad": 2}
GEMM_ACCUMULATE, GEMM_OUT_BF16 = 1, 2


class Fp4qError(RuntimeError):
    pass


class _QDesc(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("ld", ctypes.c_int64),
                ("codes_t", ctypes.c_void_p), ("ld_t", ctypes.c_int64),
                ("scales", ctypes.c_void_p), ("ld_s", ctypes.c_int64),
                ("batch", ctypes.c_int64), ("bstride", ctypes.c_int64),
                ("bstride_t", ctypes.c_int64), ("bstride_s", ctypes.c_int64),
                ("scales_t", ctypes.c_void_p), ("ld_st", ctypes.c_int64)]


class _QItem(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ldx", ctypes.c_int64), ("stream_id", ctypes.c_uint32),
                ("out", ctypes.POINTER(_QDesc))]


QUANT2D_BATCH_MAX = 8


class _Groups(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("row_off", ctypes.POINTER(ctypes.c_int64)), ("max_rows", ctypes.c_int64)]


GROUPS_DEVICE = 1


_lib = None


def library_path():
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise Fp4qError("libfp4q.so is not built (%s); run __graft_entry__.build() or "
                        "python fp4_microscaling_quantization_quant2d_amd/build.py" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    L.fp4q_version.restype = ctypes.c_int
    L.fp4q_last_error.restype = ctypes.c_char_p
    L.fp4q_quant2d_sizes.argtypes = [I64, I64, ctypes.POINTER(I64), ctypes.POINTER(I64),
                                     ctypes.POINTER(I64)]
    L.fp4q_quant2d.argtypes = [P, ctypes.c_int, I64, I64, I64, ctypes.c_int, ctypes.c_uint64,
                               ctypes.c_uint32, ctypes.POINTER(_QDesc), P]
    L.fp4q_quant2d_batch.argtypes = [ctypes.c_int, ctypes.POINTER(_QItem), ctypes.c_int, ctypes.c_int,
                                     ctypes.c_uint64, P]
    L.fp4q_quant1d_mxfp8.argtypes = [P, ctypes.c_int, I64, I64, I64, ctypes.POINTER(_QDesc), P]
    L.fp4q_gemm_ex.argtypes = [ctypes.c_int, ctypes.POINTER(_QDesc), ctypes.POINTER(_QDesc), P, I64,
                               I64, ctypes.POINTER(_Groups), ctypes.c_int, P]
    L.fp4q_gemm.argtypes = [ctypes.c_int, ctypes.POINTER(_QDesc), ctypes.POINTER(_QDesc), P, I64,
                            I64, ctypes.POINTER(_Groups), P]
    L.fp4q_dequant.argtypes = [ctypes.POINTER(_QDesc), ctypes.c_int, ctypes.c_int, P, I64, P]
    for fn in ("fp4q_quant2d_sizes", "fp4q_quant2d", "fp4q_quant2d_batch", "fp4q_quant1d_mxfp8",
               "fp4q_gemm", "fp4q_gemm_ex", "fp4q_dequant"):
        getattr(L, fn).restype = ctypes.c_int
    _lib = L
    return L


def lib():
    """The loaded ctypes library (raises Fp4qError if it is not built)."""
    return _load()


def _check(rc, what):
    if rc != 0:
        msg = _load().fp4q_last_error().decode()
        raise Fp4qError("%s failed (%d): %s" % (what, rc, msg))


def _pad32(n):
    return (n + 31) // 32 * 32


def _stream_ptr(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@dataclass
class QTensor:
    """A quantized matrix (or a batch of them) in device memory.

    fmt 1 (FP4, 2D 32x32 blocks): codes [R, ld] row plane, codes_t [C, ld_t]
    transposed plane (optional), scales [R/32, ld_s] E8M0 -- R, C = rows, cols
    rounded up to 32.  fmt 3 (FP4, 2D 64x64 blocks): the same planes with
    scales [ceil(rows/64), ld_s].  fmt 4 (FP4, 1D activation layout): the
    same planes, with one byte per 1x32 block of each plane row in tiled
    grids: scales [ceil(R/128), ld_s] for the row plane, scales_t
    [ceil(C/128), ld_st] for the transposed plane, one 512-byte chunk per
    128 rows x 128 codes (ld_s, ld_st multiples of 16).  fmt 2 (MXFP8, 1x32): codes [rows, ld] E4M3
    bytes, scales [rows, ld_s].  batch > 1 stacks items at the given byte
    strides.
    """
    fmt: int
    rows: int
    cols: int
    codes: torch.Tensor
    scales: torch.Tensor
    codes_t: Optional[torch.Tensor] = None
    batch: int = 1
    bstride: int = 0
    bstride_t: int = 0
    bstride_s: int = 0
    scales_t: Optional[torch.Tensor] = None

    def desc(self):
        d = _QDesc()
        d.fmt, d.rows, d.cols = self.fmt, self.rows, self.cols
        d.codes = self.codes.data_ptr()
        d.ld = self.codes.stride(-2)
        if self.codes_t is not None:
            d.codes_t = self.codes_t.data_ptr()
            d.ld_t = self.codes_t.stride(-2)
        d.scales = self.scales.data_ptr()
        d.ld_s = self.scales.stride(-2)
        if self.scales_t is not None:
            d.scales_t = self.scales_t.data_ptr()
            d.ld_st = self.scales_t.stride(-2)
        d.batch, d.bstride, d.bstride_t, d.bstride_s = (self.batch, self.bstride, self.bstride_t,
                                                        self.bstride_s)
        return d


def fp4q_quant2d_sizes(rows, cols):
    """(codes_bytes, codes_t_bytes, scales_bytes) of fp4q_quant2d's outputs."""
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(_load().fp4q_quant2d_sizes(rows, cols, ctypes.byref(a), ctypes.byref(b),
                                      ctypes.byref(c)), "fp4q_quant2d_sizes")
    return a.value, b.value, c.value


def alloc_fp4(rows, cols, device="cuda", transposed=True, block=32):
    """Output buffers for fp4q_quant2d with the tightest leading dimensions;
    block 32 or 64 picks the square scale block (FMT_FP4_2D32 / FMT_FP4_2D64),
    block "1d" the activation layout (FMT_FP4_1D32)."""
    if block not in (32, 64, "1d"):
        raise Fp4qError("block must be 32, 64 or '1d', got %r" % (block,))
    R, C = _pad32(rows), _pad32(cols)
    codes = torch.empty((R, C // 2), dtype=torch.uint8, device=device)
    codes_t = torch.empty((C, R // 2), dtype=torch.uint8, device=device) if transposed else None
    if block == "1d":
        # tiled grids: one 512-byte chunk per 128 rows x 128 codes of a plane
        g = lambda n: -(-n // 128)
        scales = torch.empty((g(R), 512 * g(C)), dtype=torch.uint8, device=device)
        scales_t = torch.empty((g(C), 512 * g(R)), dtype=torch.uint8, device=device) if transposed else None
        return QTensor(FMT_FP4_1D32, rows, cols, codes, scales, codes_t, scales_t=scales_t)
    scales = torch.empty((-(-rows // block), -(-cols // block)), dtype=torch.uint8, device=device)
    return QTensor(FMT_FP4_2D32 if block == 32 else FMT_FP4_2D64, rows, cols, codes, scales, codes_t)


def alloc_mxfp8(rows, cols, device="cuda"):
    C = _pad32(cols)
    codes = torch.empty((rows, C), dtype=torch.uint8, device=device)
    scales = torch.empty((rows, C // 32), dtype=torch.uint8, device=device)
    return QTensor(FMT_MXFP8_1D32, rows, cols, codes, scales)


def _dtype_code(x):
    if x.dtype == torch.bfloat16:
        return DT_BF16
    if x.dtype == torch.float32:
        return DT_F32
    raise Fp4qError("inputs must be bfloat16 or float32, got %s" % x.dtype)


def _check_matrix(x):
    if x.dim() != 2 or x.stride(1) != 1 or not x.is_cuda:
        raise Fp4qError("expected a row-major 2-D CUDA tensor")


def fp4q_quant2d(x, out: Optional[QTensor] = None, round_mode="sr", seed=0, stream_id=0,
                 stream=None, transposed=True):
    """2D 32x32-block FP4 quantization of x (bf16/fp32, rows x cols)."""
    _check_matrix(x)
    rows, cols = x.shape
    if out is None:
        out = alloc_fp4(rows, cols, x.device, transposed)
    d = out.desc()
    _check(_load().fp4q_quant2d(_ptr(x), _dtype_code(x), rows, cols, x.stride(0),
                                ROUND[round_mode], int(seed) & ((1 << 64) - 1),
                                int(stream_id) & 0xFFFFFFFF, ctypes.byref(d), _stream_ptr(stream)),
           "fp4q_quant2d")
    return out


def fp4q_quant2d_batch(items, round_mode="sr", seed=0, stream=None):
    """Several fp4q_quant2d calls in one launch.  items: (x, out, stream_id)
    triples (out a QTensor from alloc_fp4, or None to allocate one), all x of
    one dtype; returns the outputs in order."""
    items = list(items)
    if not 1 <= len(items) <= QUANT2D_BATCH_MAX:
        raise Fp4qError("fp4q_quant2d_batch takes 1..%d items, got %d" % (QUANT2D_BATCH_MAX, len(items)))
    outs, descs = [], []
    arr = (_QItem * len(items))()
    dtype = None
    for k, (x, out, stream_id) in enumerate(items):
        _check_matrix(x)
        dt = _dtype_code(x)
        if dtype is not None and dt != dtype:
            raise Fp4qError("fp4q_quant2d_batch: items of one dtype only")
        dtype = dt
        rows, cols = x.shape
        if out is None:
            out = alloc_fp4(rows, cols, x.device)
        d = out.desc()
        descs.append(d)
        outs.append(out)
        arr[k].x = _ptr(x)
        arr[k].rows, arr[k].cols, arr[k].ldx = rows, cols, x.stride(0)
        arr[k].stream_id = int(stream_id) & 0xFFFFFFFF
        arr[k].out = ctypes.pointer(d)
    _check(_load().fp4q_quant2d_batch(len(items), arr, dtype, ROUND[round_mode],
                                      int(seed) & ((1 << 64) - 1), _stream_ptr(stream)),
           "fp4q_quant2d_batch")
    return outs


def fp4q_quant1d_mxfp8(x, out: Optional[QTensor] = None, stream=None):
    """MXFP8 (E4M3, 1x32 along rows) quantization of x (bf16/fp32, rows x cols)."""
    _check_matrix(x)
    rows, cols = x.shape
    if out is None:
        out = alloc_mxfp8(rows, cols, x.device)
    d = out.desc()
    _check(_load().fp4q_quant1d_mxfp8(_ptr(x), _dtype_code(x), rows, cols, x.stride(0),
                                      ctypes.byref(d), _stream_ptr(stream)), "fp4q_quant1d_mxfp8")
    return out


def gemm_out_shape(op, a: QTensor, b: QTensor, groups: Optional[Sequence[int]] = None):
    op = OPS.get(op, op)
    if groups is None:
        if op == 0:
            return a.rows, b.rows
        if op == 1:
            return a.rows, b.cols
        return a.cols, b.cols
    n = len(groups) - 1
    if op == 0:
        return a.rows, b.rows // n
    if op == 1:
        return a.rows, b.cols
    return n * a.cols, b.cols


def fp4q_gemm(op, a: QTensor, b: QTensor, c: Optional[torch.Tensor] = None,
              groups=None, stream=None, accumulate=False, max_group_rows=None, out_dtype=torch.float32):
    """C = X W^T (fwd), dY W (dgrad) or dY^T X (wgrad) in fp32.  groups: row
    offsets (multiples of 32) of a grouped expert product -- a host sequence,
    or an int64 CUDA tensor read by the kernels (FP4Q_GROUPS_DEVICE; wgrad then
    needs max_group_rows, a bound on any group's rows).  accumulate: C += the
    product (fp4q_gemm_ex with FP4Q_GEMM_ACCUMULATE; c required).  A bfloat16 C
    (given, or out_dtype=torch.bfloat16) takes FP4Q_GEMM_OUT_BF16."""
    opc = OPS.get(op, op)
    M, N = gemm_out_shape(opc, a, b, groups)
    if accumulate and c is None:
        raise Fp4qError("accumulate needs the C to add to")
    if c is None:
        shape = (a.batch, M, N) if a.batch > 1 else (M, N)
        c = torch.empty(shape, dtype=out_dtype, device=a.codes.device)
    if c.dtype not in (torch.float32, torch.bfloat16) or c.stride(-1) != 1:
        raise Fp4qError("C must be a row-major float32 or bfloat16 tensor")
    flags = (GEMM_ACCUMULATE if accumulate else 0) | (GEMM_OUT_BF16 if c.dtype == torch.bfloat16 else 0)
    ldc = c.stride(-2)
    cbs = c.stride(0) if c.dim() == 3 else 0
    g = None
    if isinstance(groups, torch.Tensor):
        if not groups.is_cuda or groups.dtype != torch.int64 or groups.dim() != 1 or not groups.is_contiguous():
            raise Fp4qError("device group offsets must be a contiguous 1-D int64 CUDA tensor")
        g = _Groups(groups.numel() - 1, GROUPS_DEVICE,
                    ctypes.cast(ctypes.c_void_p(groups.data_ptr()), ctypes.POINTER(ctypes.c_int64)),
                    int(max_group_rows or 0))
    elif groups is not None:
        arr = (ctypes.c_int64 * len(groups))(*[int(v) for v in groups])
        g = _Groups(len(groups) - 1, 0, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64)), 0)
    da, db = a.desc(), b.desc()
    if flags:
        _check(_load().fp4q_gemm_ex(opc, ctypes.byref(da), ctypes.byref(db), _ptr(c), ldc, cbs,
                                    ctypes.byref(g) if g is not None else None, flags,
                                    _stream_ptr(stream)), "fp4q_gemm_ex")
        return c
    _check(_load().fp4q_gemm(opc, ctypes.byref(da), ctypes.byref(db), _ptr(c), ldc, cbs,
                             ctypes.byref(g) if g is not None else None, _stream_ptr(stream)),
           "fp4q_gemm")
    return c


def fp4q_dequant(q: QTensor, transposed=False, out_dtype=torch.float32, out=None, stream=None):
    """X ~ P * S for the row plane (rows x cols) or the transposed plane."""
    shape = (q.cols, q.rows) if transposed else (q.rows, q.cols)
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=q.codes.device)
    code = DT_F32 if out.dtype == torch.float32 else DT_BF16
    d = q.desc()
    _check(_load().fp4q_dequant(ctypes.byref(d), 1 if transposed else 0, code, _ptr(out),
                                out.stride(0), _stream_ptr(stream)), "fp4q_dequant")
    return out
