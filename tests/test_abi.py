"""The C ABI library loads, exports every entry point declared in
include/fp4q.h, and rejects bad arguments on the host before any launch
(no GPU needed: validation runs before the first HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4q.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4q_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def fp4q():
    import fp4_microscaling_quantization_quant2d_amd as m
    if not os.path.exists(m.library_path()):
        from fp4_microscaling_quantization_quant2d_amd import build
        build.build()
    m.lib()
    return m


def test_header_declares_the_entry_points():
    names = _declared()
    for fn in ("fp4q_quant2d", "fp4q_quant1d_mxfp8", "fp4q_gemm", "fp4q_gemm_ex", "fp4q_dequant",
               "fp4q_quant2d_sizes", "fp4q_last_error", "fp4q_version"):
        assert fn in names


def test_library_exports_every_declared_symbol(fp4q):
    L = fp4q.lib()
    for fn in _declared():
        assert hasattr(L, fn), fn
    out = os.popen("nm -D --defined-only %s" % fp4q.library_path()).read()
    for fn in _declared():
        assert re.search(r"\bT %s\b" % fn, out), fn


def test_version_and_sizes(fp4q):
    assert fp4q.lib().fp4q_version() == 3
    # Table 1 accounting: codes are a quarter of the bf16 bytes, plus 1 byte per tile
    assert fp4q.fp4q_quant2d_sizes(4096, 2048) == (4096 * 1024, 2048 * 2048, 128 * 64)
    assert fp4q.fp4q_quant2d_sizes(33, 65) == (64 * 48, 96 * 32, 2 * 3)
    with pytest.raises(fp4q.Fp4qError):
        fp4q.fp4q_quant2d_sizes(0, 5)


def _desc(fp4q, fmt=1, rows=64, cols=64, ld=32, ld_t=32, ld_s=2, codes=0x1000, codes_t=0x2000,
          scales=0x3000, batch=1):
    d = fp4q._QDesc()
    d.fmt, d.rows, d.cols, d.ld, d.ld_t, d.ld_s, d.batch = fmt, rows, cols, ld, ld_t, ld_s, batch
    d.codes, d.codes_t, d.scales = codes, codes_t, scales
    return d


def _err(fp4q):
    return fp4q.lib().fp4q_last_error().decode()


def test_quant2d_rejects_bad_arguments(fp4q):
    L = fp4q.lib()
    P = ctypes.c_void_p
    x = P(0x10000)
    good = _desc(fp4q)
    cases = [
        (P(0), 1, 64, 64, 64, 0, good),          # null x
        (x, 3, 64, 64, 64, 0, good),             # dtype
        (x, 1, 0, 64, 64, 0, good),              # rows
        (x, 1, 64, 64, 32, 0, good),             # ldx < cols
        (x, 1, 64, 64, 64, 7, good),             # round mode
        (x, 1, 64, 64, 64, 0, _desc(fp4q, ld=16)),       # ld too small
        (x, 1, 64, 64, 64, 0, _desc(fp4q, ld=40)),       # ld not multiple of 16
        (x, 1, 64, 64, 64, 0, _desc(fp4q, codes=0x1008)),  # misaligned plane
        (x, 1, 64, 64, 64, 0, _desc(fp4q, ld_s=1)),      # scale grid too narrow
        (x, 1, 64, 64, 64, 0, _desc(fp4q, rows=32)),     # shape mismatch
        (x, 1, 64, 64, 64, 0, _desc(fp4q, fmt=2)),       # wrong format
        (x, 1, 64, 64, 64, 0, _desc(fp4q, ld_t=16)),     # transposed plane too small
        (x, 1, 64, 200, 200, 0, _desc(fp4q, fmt=3, cols=200, ld=112, ld_s=3)),  # 64-block grid too narrow
    ]
    for xp, dt, r, c, ldx, rm, d in cases:
        rc = L.fp4q_quant2d(xp, dt, r, c, ldx, rm, 0, 0, ctypes.byref(d), None)
        assert rc == -1, (dt, r, c, ldx, rm)
        assert _err(fp4q)
    # one workgroup per 128x128 region: 2^24 regions exceed one launch
    n = 1 << 19
    big = _desc(fp4q, rows=n, cols=n, ld=n // 2, ld_t=n // 2, ld_s=n // 32)
    assert L.fp4q_quant2d(x, 1, n, n, n, 0, 0, 0, ctypes.byref(big), None) == -2
    assert "regions" in _err(fp4q)


def test_quant2d_batch_rejects_bad_arguments(fp4q):
    L = fp4q.lib()
    P = ctypes.c_void_p
    good = _desc(fp4q)

    def items(*specs):
        arr = (fp4q._QItem * max(len(specs), 1))()
        keep = []
        for k, (x, r, c, ldx, d) in enumerate(specs):
            keep.append(d)
            arr[k].x, arr[k].rows, arr[k].cols, arr[k].ldx = x, r, c, ldx
            arr[k].stream_id = k
            arr[k].out = ctypes.pointer(d)
        return arr, keep

    ok_item = (0x10000, 64, 64, 64, good)
    arr, keep = items(ok_item, ok_item)
    assert L.fp4q_quant2d_batch(0, arr, 1, 0, 0, None) == -1                  # n = 0
    assert L.fp4q_quant2d_batch(fp4q.QUANT2D_BATCH_MAX + 1, arr, 1, 0, 0, None) == -1
    assert L.fp4q_quant2d_batch(2, None, 1, 0, 0, None) == -1                 # null items
    assert L.fp4q_quant2d_batch(2, arr, 5, 0, 0, None) == -1                  # dtype
    assert L.fp4q_quant2d_batch(2, arr, 1, 9, 0, None) == -1                  # round mode
    for bad in ((0, 64, 64, 64, good),                 # null x in the second item
                (0x20000, 64, 64, 32, good),           # ldx < cols
                (0x20000, 64, 64, 64, _desc(fp4q, rows=32)),   # shape mismatch
                (0x20000, 64, 64, 64, _desc(fp4q, ld_t=16))):  # transposed plane too small
        arr, keep = items(ok_item, bad)
        assert L.fp4q_quant2d_batch(2, arr, 1, 0, 0, None) == -1
        assert _err(fp4q).startswith("fp4q_quant2d_batch")
    # the region limit counts all items together: two of 2^23 regions each
    n = 1 << 19
    half = _desc(fp4q, rows=n // 2, cols=n, ld=n // 2, ld_t=n // 4, ld_s=n // 32)
    arr, keep = items((0x10000, n // 2, n, n, half), (0x10000, n // 2, n, n, half))
    assert L.fp4q_quant2d_batch(2, arr, 1, 0, 0, None) == -2
    assert "regions" in _err(fp4q)


def test_gemm_rejects_bad_arguments(fp4q):
    L = fp4q.lib()
    c = ctypes.c_void_p(0x50000)
    a = _desc(fp4q, rows=64, cols=64)
    b = _desc(fp4q, rows=96, cols=32, ld=16, ld_t=48, ld_s=1)
    assert L.fp4q_gemm(0, ctypes.byref(a), ctypes.byref(b), c, 96, 0, None, None) == -1  # K mismatch
    assert "K mismatch" in _err(fp4q)
    assert L.fp4q_gemm(5, ctypes.byref(a), ctypes.byref(a), c, 64, 0, None, None) == -1   # op
    assert L.fp4q_gemm(0, ctypes.byref(a), ctypes.byref(a), c, 32, 0, None, None) == -1   # ldc
    nt = _desc(fp4q, codes_t=0)
    assert L.fp4q_gemm(1, ctypes.byref(a), ctypes.byref(nt), c, 64, 0, None, None) == -1  # needs W^T
    assert L.fp4q_gemm(2, ctypes.byref(nt), ctypes.byref(a), c, 64, 0, None, None) == -1  # needs dY^T
    f8 = _desc(fp4q, fmt=2, ld=64)
    assert L.fp4q_gemm(0, ctypes.byref(a), ctypes.byref(f8), c, 64, 0, None, None) == -1  # mixed fmt
    assert L.fp4q_gemm(1, ctypes.byref(f8), ctypes.byref(f8), c, 64, 0, None, None) == -2  # fp8 dgrad
    # the tile holds the scale bytes of its whole K range in LDS: MXFP8 K is bounded
    big = _desc(fp4q, fmt=2, cols=4096, ld=4096, ld_s=128)
    assert L.fp4q_gemm(0, ctypes.byref(big), ctypes.byref(big), c, 64, 0, None, None) == -2
    assert "too large" in _err(fp4q)
    # grouped: offsets must start at 0 and be multiples of 32
    for offs in ([0, 16, 64], [32, 64], [0, 64, 32], [0, 32, 96]):
        arr = (ctypes.c_int64 * len(offs))(*offs)
        g = fp4q._Groups(len(offs) - 1, 0, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64)), 0)
        w = _desc(fp4q, rows=64 * (len(offs) - 1), cols=64, ld_t=64 * (len(offs) - 1) // 2)
        assert L.fp4q_gemm(0, ctypes.byref(a), ctypes.byref(w), c, 64, 0, ctypes.byref(g), None) == -1
    # grouped products take 32x32 blocks only
    arr = (ctypes.c_int64 * 2)(0, 64)
    g = fp4q._Groups(1, 0, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64)), 0)
    a64 = _desc(fp4q, fmt=3, rows=64, cols=64)
    assert L.fp4q_gemm(0, ctypes.byref(a64), ctypes.byref(a), c, 64, 0, ctypes.byref(g), None) == -2
    assert "32x32" in _err(fp4q)


def _desc1d(fp4q, rows=64, cols=64, ld_s=512, ld_st=512, scales=0x3000, scales_t=0x4000, **kw):
    d = _desc(fp4q, fmt=4, rows=rows, cols=cols, ld_s=ld_s, scales=scales, **kw)
    d.scales_t, d.ld_st = scales_t, ld_st
    return d


def test_act1d_layout_rejects_bad_arguments(fp4q):
    """The 1D activation layout's tiled scale grids: one 512-byte chunk per
    128 rows x 128 codes, leading dims multiples of 16, 16-byte aligned; the
    transposed plane needs its own grid; dense products with batch 1 only."""
    L = fp4q.lib()
    x = ctypes.c_void_p(0x10000)
    good = _desc1d(fp4q, rows=64, cols=300, ld=160, ld_s=1536)
    assert good.ld_s == 512 * 3
    for bad in (_desc1d(fp4q, rows=64, cols=300, ld=160, ld_s=1024),            # grid too narrow
                _desc1d(fp4q, rows=64, cols=300, ld=160, ld_s=1544),            # ld_s % 16
                _desc1d(fp4q, rows=64, cols=300, ld=160, ld_s=1536, scales=0x3004),  # misaligned
                _desc1d(fp4q, rows=64, cols=300, ld=160, ld_s=1536, scales_t=0),     # no scales_t
                _desc1d(fp4q, rows=64, cols=300, ld=160, ld_s=1536, ld_st=256, ld_t=32)):  # scales_t narrow
        assert L.fp4q_quant2d(x, 1, 64, 300, 300, 0, 0, 0, ctypes.byref(bad), None) == -1
        assert "scales" in _err(fp4q)
    # batch items must share the layout
    arr = (fp4q._QItem * 2)()
    d2 = _desc(fp4q)
    for k, d in enumerate((good, d2)):
        arr[k].x, arr[k].rows, arr[k].cols, arr[k].ldx = 0x10000, d.rows, d.cols, d.cols
        arr[k].out = ctypes.pointer(d)
    assert L.fp4q_quant2d_batch(2, arr, 1, 0, 0, None) == -1
    assert "format differs" in _err(fp4q)
    c = ctypes.c_void_p(0x50000)
    a = _desc1d(fp4q)
    w = _desc(fp4q)
    ab = _desc1d(fp4q, batch=2)
    wb = _desc(fp4q, batch=2)
    assert L.fp4q_gemm(0, ctypes.byref(ab), ctypes.byref(wb), c, 64, 64 * 64, None, None) == -2
    assert "batch 1" in _err(fp4q)
    arr = (ctypes.c_int64 * 2)(0, 64)
    g = fp4q._Groups(1, 0, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64)), 0)
    assert L.fp4q_gemm(0, ctypes.byref(a), ctypes.byref(w), c, 64, 0, ctypes.byref(g), None) == -2
    nt = _desc1d(fp4q, scales_t=0)
    assert L.fp4q_gemm(2, ctypes.byref(w), ctypes.byref(nt), c, 64, 0, None, None) == -1  # X^T grid
    y = ctypes.c_void_p(0x70000)
    assert L.fp4q_dequant(ctypes.byref(nt), 1, 2, y, 64, None) == -1


def test_gemm_ex_accumulate_rejects_unsupported(fp4q):
    """fp4q_gemm_ex: unknown flags are invalid; accumulation takes dense FP4
    products whose A operand has a square-block grid."""
    L = fp4q.lib()
    c = ctypes.c_void_p(0x50000)
    a = _desc(fp4q)
    assert L.fp4q_gemm_ex(0, ctypes.byref(a), ctypes.byref(a), c, 64, 0, None, 4, None) == -1
    assert "flags" in _err(fp4q)
    f8 = _desc(fp4q, fmt=2, ld=64)
    assert L.fp4q_gemm_ex(0, ctypes.byref(f8), ctypes.byref(f8), c, 64, 0, None, 1, None) == -2
    arr = (ctypes.c_int64 * 2)(0, 64)
    g = fp4q._Groups(1, 0, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64)), 0)
    assert L.fp4q_gemm_ex(0, ctypes.byref(a), ctypes.byref(a), c, 64, 0, ctypes.byref(g), 1, None) == -2
    x1 = _desc1d(fp4q)
    assert L.fp4q_gemm_ex(0, ctypes.byref(x1), ctypes.byref(a), c, 64, 0, None, 1, None) == -2
    assert "accumulation" in _err(fp4q)
    # bf16 output: dense, no accumulation, square-block FP4 or MXFP8
    assert L.fp4q_gemm_ex(0, ctypes.byref(a), ctypes.byref(a), c, 64, 0, None, 3, None) == -2
    assert L.fp4q_gemm_ex(0, ctypes.byref(x1), ctypes.byref(a), c, 64, 0, None, 2, None) == -2
    assert L.fp4q_gemm_ex(0, ctypes.byref(x1), ctypes.byref(a), c, 64, 0, None, 2, None) == -2
    assert "bf16" in _err(fp4q)
    with pytest.raises(fp4q.Fp4qError):
        fp4q.fp4q_gemm("wgrad", fp4q.alloc_fp4(64, 64, device="cpu"), fp4q.alloc_fp4(64, 64, device="cpu"),
                       accumulate=True)


def test_device_group_offsets_validation(fp4q):
    """Device offsets cannot be checked on the host; what can be is: known
    flags, and for WGRAD a max_rows bound that is a multiple of 32 within the
    token rows (the kernels clamp the offsets themselves)."""
    L = fp4q.lib()
    c = ctypes.c_void_p(0x50000)
    a = _desc(fp4q, rows=256, cols=64, ld_t=128)
    w = _desc(fp4q, rows=128, cols=64)
    dev_off = ctypes.cast(ctypes.c_void_p(0x90000), ctypes.POINTER(ctypes.c_int64))
    for flags, max_rows in ((2, 64), (3, 64)):
        g = fp4q._Groups(2, flags, dev_off, max_rows)
        assert L.fp4q_gemm(0, ctypes.byref(a), ctypes.byref(w), c, 64, 0, ctypes.byref(g), None) == -1
        assert "flags" in _err(fp4q)
    dy = _desc(fp4q, rows=256, cols=64, ld_t=128)
    for max_rows in (0, 48, 512):
        g = fp4q._Groups(2, 1, dev_off, max_rows)
        assert L.fp4q_gemm(2, ctypes.byref(dy), ctypes.byref(a), c, 64, 0, ctypes.byref(g), None) == -1
        assert "max_rows" in _err(fp4q)
    # host offsets must end within the whole 32-row blocks of a
    arr = (ctypes.c_int64 * 2)(0, 256)
    g = fp4q._Groups(1, 0, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64)), 0)
    a250 = _desc(fp4q, rows=250, cols=64, ld_t=128)
    assert L.fp4q_gemm(0, ctypes.byref(a250), ctypes.byref(w), c, 64, 0, ctypes.byref(g), None) == -1
    assert "beyond" in _err(fp4q)


def test_dequant_and_mxfp8_reject_bad_arguments(fp4q):
    L = fp4q.lib()
    y = ctypes.c_void_p(0x70000)
    q = _desc(fp4q)
    assert L.fp4q_dequant(ctypes.byref(q), 0, 9, y, 64, None) == -1
    assert L.fp4q_dequant(ctypes.byref(q), 0, 2, y, 10, None) == -1
    f8 = _desc(fp4q, fmt=2, ld=64)
    assert L.fp4q_dequant(ctypes.byref(f8), 1, 2, y, 64, None) == -2
    assert L.fp4q_quant1d_mxfp8(ctypes.c_void_p(0x10000), 1, 64, 64, 64, ctypes.byref(q), None) == -1
    bad = _desc(fp4q, fmt=2, ld=48)
    assert L.fp4q_quant1d_mxfp8(ctypes.c_void_p(0x10000), 1, 64, 64, 64, ctypes.byref(bad), None) == -1
    # 4 (bf16) or 8 (f32) work-items per group of 32: 2^30 groups of bf16, or
    # 2^29 of f32, reach 2^32 work-items, more than one launch holds
    for dt, rows in ((1, 1 << 30), (2, 1 << 29)):
        big = _desc(fp4q, fmt=2, rows=rows, cols=32, ld=32, ld_s=1)
        assert L.fp4q_quant1d_mxfp8(ctypes.c_void_p(0x10000), dt, rows, 32, 32, ctypes.byref(big), None) == -1
        assert "too many groups" in _err(fp4q)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    import fp4_microscaling_quantization_quant2d_amd as m
    monkeypatch.setattr(m, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(m, "_lib", None)
    with pytest.raises(m.Fp4qError):
        m.lib()


def test_alloc_act1d_meets_the_grid_rules(fp4q):
    """alloc_fp4(block="1d") sizes the tiled grids as the validation requires:
    ceil(R/128) x 512*ceil(C/128) for the row plane, the transpose for the
    transposed plane (host tensors: no device needed)."""
    for rows, cols in ((1, 1), (300, 257), (128, 128), (129, 385)):
        q = fp4q.alloc_fp4(rows, cols, device="cpu", block="1d")
        R, C = -(-rows // 32) * 32, -(-cols // 32) * 32
        d = q.desc()
        assert d.fmt == 4 and q.scales.shape == (-(-R // 128), 512 * -(-C // 128))
        assert q.scales_t.shape == (-(-C // 128), 512 * -(-R // 128))
        assert d.ld_s % 16 == 0 and d.ld_st % 16 == 0 and d.ld_s >= 512 * -(-C // 128)


def test_binding_checks_outputs_before_any_launch(fp4q):
    """The binding refuses an output the C ABI could not check (it sees only a
    pointer and a leading dimension): wrong dtype, wrong shape or batch,
    another device, non-contiguous rows.  Host tensors: every refusal happens
    before anything is enqueued."""
    import torch
    a = fp4q.alloc_fp4(64, 96, device="cpu")
    b = fp4q.alloc_fp4(32, 96, device="cpu")
    cases = [
        (torch.empty(64, 32, dtype=torch.uint8), "float32 or bfloat16"),
        (torch.empty(64, 33), "shape"),
        (torch.empty(2, 64, 32), "shape"),
        (torch.empty(64, 32), "must live on"),
        (torch.empty(32, 64).t(), "contiguous rows"),
    ]
    for c, msg in cases:
        with pytest.raises(fp4q.Fp4qError, match=msg):
            fp4q.fp4q_gemm("fwd", a, b, c=c)
    with pytest.raises(fp4q.Fp4qError, match="accumulate"):
        fp4q.fp4q_gemm("wgrad", a, b, accumulate=True)
    for out, msg in ((torch.empty(64, 96, dtype=torch.uint8), "float32 or bfloat16"),
                     (torch.empty(96, 64), "shape"), (torch.empty(64, 96), "must live on")):
        with pytest.raises(fp4q.Fp4qError, match=msg):
            fp4q.fp4q_dequant(a, out=out)
    with pytest.raises(fp4q.Fp4qError, match="shape"):
        fp4q.fp4q_dequant(a, transposed=True, out=torch.empty(64, 96))


def test_device_seed_entry_validates(fp4q):
    """fp4q_quant2d_batch_ex checks what fp4q_quant2d_batch checks, plus the
    alignment of the device seed pointer."""
    L = fp4q.lib()
    d = _desc(fp4q)
    it = fp4q._QItem(ctypes.c_void_p(0x10000), 64, 64, 64, 1, ctypes.pointer(d))
    arr = (fp4q._QItem * 1)(it)
    assert L.fp4q_quant2d_batch_ex(1, arr, 1, 0, 0, ctypes.c_void_p(0x20004), None) == -1
    assert "aligned" in _err(fp4q)
    assert L.fp4q_quant2d_batch_ex(0, arr, 1, 0, 0, ctypes.c_void_p(0x20000), None) == -1
    assert L.fp4q_quant2d_batch_ex(1, arr, 7, 0, 0, ctypes.c_void_p(0x20000), None) == -1


def test_gemm_quant_validation(fp4q):
    """fp4q_gemm_quant takes dense FP4 products of square-block operands with
    batch 1 and a 32x32-block output of the product's shape."""
    L = fp4q.lib()
    a = _desc(fp4q, rows=64, cols=64)
    w = _desc(fp4q, rows=96, cols=64)
    good = _desc(fp4q, rows=64, cols=96, ld=48, ld_t=32, ld_s=3)
    seed_ok = ctypes.c_void_p(0x80000)
    call = lambda op, x, y, o, rm=0, sd=None: L.fp4q_gemm_quant(op, ctypes.byref(x), ctypes.byref(y),
                                                                   ctypes.byref(o) if o is not None else None,
                                                                   rm, 0, 0, sd, None)
    assert call(0, a, w, None) == -1
    assert call(0, a, w, _desc(fp4q, rows=64, cols=64, ld=48, ld_s=3)) == -1      # wrong shape
    assert "product" in _err(fp4q)
    assert call(0, a, w, good, rm=5) == -1
    assert call(0, a, w, good, sd=ctypes.c_void_p(0x80004)) == -1
    f8 = _desc(fp4q, fmt=2, ld=64)
    assert call(0, f8, f8, good) == -2
    ab = _desc(fp4q, rows=64, cols=64, batch=2)
    assert call(0, ab, _desc(fp4q, rows=96, cols=64, batch=2), good) == -2
    o64 = _desc(fp4q, fmt=3, rows=64, cols=96, ld=48, ld_t=32, ld_s=2)
    assert call(0, a, w, o64) == -2


def test_attention_validation(fp4q):
    """fp4q_attn_fwd / fp4q_attn_bwd check shapes, head dimension, alignment
    and arguments on the host before any launch."""
    L = fp4q.lib()
    P = ctypes.c_void_p
    rows = 2 * 64
    q = _desc(fp4q, fmt=2, rows=rows, cols=128, ld=128, ld_s=4)
    v, o, lse = P(0x100000), P(0x200000), P(0x300000)
    call = lambda qq, kk, ldv=128, ldo=128, odt=1, scale=0.088, causal=1, bh=2, n=64: L.fp4q_attn_fwd(
        ctypes.byref(qq), ctypes.byref(kk), v, ldv, o, ldo, odt, lse, bh, n, ctypes.c_float(scale), causal, None)
    assert call(q, _desc(fp4q, fmt=2, rows=rows, cols=64, ld=64, ld_s=2)) == -2   # head dimension 64
    assert "128" in _err(fp4q)
    assert call(q, q, bh=3) == -1                                                   # rows != bh*seq_len
    assert call(q, q, ldv=100) == -1
    assert call(q, q, ldo=130) == -1
    assert call(q, q, odt=7) == -1
    assert call(q, q, scale=0.0) == -1
    assert call(q, q, causal=2) == -1
    assert call(q, _desc(fp4q, fmt=2, rows=rows, cols=128, ld=128, ld_s=5)) == -1    # scale rows not 4-aligned
    g = P(0x400000)
    bwd = lambda ldg=128, ws=P(0x500000), lddo=128: L.fp4q_attn_bwd(
        ctypes.byref(q), ctypes.byref(q), v, 128, o, 128, 1, lse, g, lddo, P(0x600000), P(0x700000), P(0x800000),
        ldg, ws, 2, 64, ctypes.c_float(0.088), 1, None)
    assert bwd(ws=None) == -1 and "workspace" in _err(fp4q)
    assert bwd(ldg=130) == -1
    assert bwd(lddo=64) == -1
    # the allocation-free backward checks its static scratch bound first,
    # without forming a product that could wrap
    na = lambda bh, n: L.fp4q_attn_bwd_noalloc(
        ctypes.byref(q), ctypes.byref(q), v, 128, o, 128, 1, lse, g, 128, P(0x600000), P(0x700000), P(0x800000),
        128, bh, n, ctypes.c_float(0.088), 1, None)
    assert na(2, (1 << 19) + 1) == -1 and "static scratch" in _err(fp4q)
    assert na(1 << 40, 1 << 40) == -1 and "static scratch" in _err(fp4q)
    assert na((1 << 62) + 1, 4) == -1 and "static scratch" in _err(fp4q)
    assert na(0, 64) == -1 and na(2, 0) == -1
    # every head's slice of every tensor stays below 2^31 elements
    big = _desc(fp4q, fmt=2, rows=1 << 21, cols=128, ld=128, ld_s=4)
    assert call(big, big, bh=1, n=1 << 21, ldv=1024) == -1 and "2^31" in _err(fp4q)
    assert call(big, big, bh=1, n=1 << 21, ldo=1024) == -1 and "2^31" in _err(fp4q)


def test_fp8_mfma_probe_validation(fp4q):
    """The FP8 MFMA probe refuses null or misaligned buffers (ABI) and
    wrong shapes or host tensors (binding) before any launch."""
    import torch
    L = fp4q.lib()
    P = ctypes.c_void_p
    assert L.fp4q_probe_mfma_fp8(None, P(0x1000), P(0x2000), P(0x3000), P(0x4000), None) == -1
    assert L.fp4q_probe_mfma_fp8(P(0x1001), P(0x1000), P(0x2000), P(0x3000), P(0x4000), None) == -1
    a = torch.zeros((32, 64), dtype=torch.uint8)
    s = torch.zeros((32, 2), dtype=torch.uint8)
    with pytest.raises(fp4q.Fp4qError):
        fp4q.fp4q_probe_mfma_fp8(a, a, s, s)                  # host tensors
    with pytest.raises(fp4q.Fp4qError):
        fp4q.fp4q_probe_mfma_fp8(a[:, :32], a, s, s)          # wrong shape
