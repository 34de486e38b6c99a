"""GPU parity of the MXFP8 side path (Q/K projections): the 1x32 E4M3
quantizer bit-exact against the oracle, and the batched block-scaled FP8
GEMM S = Q K^T within 1e-5 * sum|a||b|; plus the 2D-FP4 O-projection of the
mixed-precision attention workload."""
import numpy as np
import pytest
import torch

import oracle as orc
import fp4_microscaling_quantization_quant2d_amd as fq
from fp4_microscaling_quantization_quant2d_amd import workloads as wl
from gpu_util import assert_planes_equal, check_gemm_tol, note, to_dev

pytestmark = pytest.mark.gpu


def _check_fp8(q, ref, rows):
    c, s = q.codes.cpu().numpy(), q.scales.cpu().numpy()
    rc, rs = ref
    assert np.array_equal(s[:rows], rs), "scales differ at %s" % np.argwhere(s[:rows] != rs)[:5]
    bad = np.argwhere(c[:rows] != rc)
    assert bad.size == 0, "codes differ at %s (gpu %s oracle %s)" % (bad[:5].tolist(), c[tuple(bad[0])],
                                                                      rc[tuple(bad[0])])


@pytest.mark.parametrize("shape", [(1, 1), (5, 70), (33, 100), (64, 128), (7, 32), (300, 257)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mxfp8_quant_bit_exact(shape, dtype):
    rng = np.random.default_rng(shape[0] * 1000 + shape[1])
    x = (rng.standard_normal(shape) * np.exp(rng.uniform(-20, 20, (shape[0], 1)))).astype(np.float32)
    x[0, 0] = 0.0
    if dtype == "bf16":
        x = wl.f32_to_bf16_bits(x)
    note("mxfp8 quant %s %s" % (shape, dtype))
    q = fq.fp4q_quant1d_mxfp8(to_dev(x))
    _check_fp8(q, orc.quant1d_mxfp8(x), shape[0])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("col0,cols", [(0, 96), (8, 96), (3, 77)])
def test_mxfp8_quant_strided_rows(dtype, col0, cols):
    """x a column window of a wider matrix (leading dimension 200 or 201
    elements): rows whose 16-byte lane loads stay aligned (col0 0 or 8 with
    an aligned pitch) and rows that take the element-wise path."""
    rng = np.random.default_rng(col0 * 100 + cols)
    pitch = 200 if col0 != 3 else 201
    full = (rng.standard_normal((45, pitch)) * np.exp(rng.uniform(-8, 8, (45, 1)))).astype(np.float32)
    if dtype == "bf16":
        full = wl.f32_to_bf16_bits(full)
    x = np.ascontiguousarray(full[:, col0:col0 + cols])
    dev = to_dev(full)[:, col0:col0 + cols]
    assert dev.stride(0) == pitch
    note("mxfp8 strided %s col0=%d cols=%d" % (dtype, col0, cols))
    _check_fp8(fq.fp4q_quant1d_mxfp8(dev), orc.quant1d_mxfp8(x), 45)


def test_mxfp8_special_values():
    rng = np.random.default_rng(1)
    x = np.zeros((8, 128), np.float32)
    x[0, :32] = 448.0
    x[0, 32:64] = -448.0 * rng.random(32)
    x[1, :32] = rng.integers(1, 1 << 23, 32).astype(np.uint32).view(np.float32)     # subnormals
    x[2, :] = 3e38 * rng.uniform(-1, 1, 128)
    x[3, :] = 1e-40
    x[4, :] = -0.0
    x[5, :] = np.float32(2.0) ** rng.integers(-140, 120, 128)
    x[6, :] = rng.standard_normal(128) * 1e-30
    x[7, :] = [(-1) ** i * (i + 0.5) for i in range(128)]
    for xx in (x, wl.f32_to_bf16_bits(x)):
        note("mxfp8 special %s" % xx.dtype)
        _check_fp8(fq.fp4q_quant1d_mxfp8(to_dev(xx)), orc.quant1d_mxfp8(xx), 8)


def _e4m3_values():
    """The 127 non-negative finite E4M3FN magnitudes, code order (0 .. 448)."""
    return torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_mxfp8_every_bf16_pattern_every_exponent():
    """Every finite bf16 value x at every block exponent k it can have: for
    each k (-127 .. 120) a group's first element 448 * 2^k (the largest
    bf16 value of that exponent; the largest finite bf16 for k = 120) sets
    the amax, and the other 31 elements run through every bf16 pattern of
    either sign whose magnitude is at most it.  The codes (the rounding of
    x * 2^-k to E4M3, ties to even, subnormals included) and the scale bytes
    are compared bit for bit with the oracle."""
    rows = []
    for k in range(-127, 121):
        a_bits = 0x7F7F if k == 120 else ((135 + k) << 7) | 0x60
        mags = np.arange(a_bits + 1, dtype=np.uint32)
        pats = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        n = -(-len(pats) // 31)
        body = np.zeros(n * 31, np.uint16)
        body[:len(pats)] = pats
        blk = np.empty((n, 32), np.uint16)
        blk[:, 0] = a_bits
        blk[:, 1:] = body.reshape(n, 31)
        rows.append(blk)
    x = np.ascontiguousarray(np.concatenate(rows))   # one group per row
    note("mxfp8 every bf16 pattern x every exponent: %d rows x %d" % x.shape)
    q = fq.fp4q_quant1d_mxfp8(to_dev(x))
    _check_fp8(q, orc.quant1d_mxfp8(x), x.shape[0])


def test_mxfp8_f32_ties_and_neighbours():
    """fp32 inputs at sampled block exponents: every midpoint between two
    adjacent E4M3 magnitudes (normal and subnormal), the fp32 values one ulp
    either side of it, and hashed fp32 patterns below the group's amax,
    scaled by 2^k, both signs."""
    vals = _e4m3_values()
    mid = (vals[:-1] + vals[1:]) / 2.0
    rng = np.random.default_rng(5)
    groups = []
    for k in list(range(-127, -110)) + list(range(-20, 21)) + list(range(100, 121)):
        A = np.float32(448.0 * 2.0 ** k) if k < 120 else np.float32(3.0e38)
        with np.errstate(over="ignore"):   # midpoints past the fp32 range drop out below
            m = (mid * 2.0 ** k).astype(np.float32)
        m = m[(m > 0) & (m <= A)]
        cand = np.concatenate([m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(np.inf))])
        h = (rng.integers(0, int(A.view(np.uint32)) + 1, 4 * 31, dtype=np.int64)).astype(np.uint32).view(np.float32)
        cand = np.concatenate([cand[(cand <= A) & np.isfinite(cand)], h])
        cand = np.concatenate([cand, -cand])
        n = -(-len(cand) // 31)
        body = np.zeros(n * 31, np.float32)
        body[:len(cand)] = cand
        blk = np.empty((n, 32), np.float32)
        blk[:, 0] = A
        blk[:, 1:] = body.reshape(n, 31)
        groups.append(blk)
    x = np.ascontiguousarray(np.concatenate(groups))
    note("mxfp8 f32 ties: %d rows" % x.shape[0])
    _check_fp8(fq.fp4q_quant1d_mxfp8(to_dev(x)), orc.quant1d_mxfp8(x), x.shape[0])


def _batched_fp8(q, B, L, D):
    """View a [B*L x D] MXFP8 quantization as a batch of B [L x D] matrices."""
    ld, lds = q.codes.shape[1], q.scales.shape[1]
    return fq.QTensor(fq.FMT_MXFP8_1D32, L, D, q.codes.view(B, L, ld), q.scales.view(B, L, lds),
                      batch=B, bstride=L * ld, bstride_s=L * lds)


def test_fp8_batched_gemm_small():
    rng = np.random.default_rng(3)
    B, L, D = 3, 200, 128
    Q = wl.f32_to_bf16_bits(rng.standard_normal((B * L, D)).astype(np.float32))
    K = wl.f32_to_bf16_bits((rng.standard_normal((B * L, D)) * 3).astype(np.float32))
    note("fp8 batched small")
    qq = _batched_fp8(fq.fp4q_quant1d_mxfp8(to_dev(Q)), B, L, D)
    qk = _batched_fp8(fq.fp4q_quant1d_mxfp8(to_dev(K)), B, L, D)
    S = fq.fp4q_gemm("fwd", qq, qk).cpu().numpy()
    assert S.shape == (B, L, L)
    rq, rk = orc.quant1d_mxfp8(Q), orc.quant1d_mxfp8(K)
    Qd = orc.dequant_mxfp8(rq[0], rq[1], B * L, D)
    Kd = orc.dequant_mxfp8(rk[0], rk[1], B * L, D)
    for b in range(B):
        ref, bd = orc.gemm("fwd", Qd[b * L:(b + 1) * L], Kd[b * L:(b + 1) * L])
        check_gemm_tol(S[b], ref, bd, "S batch %d" % b)


@pytest.mark.parametrize("D", [32, 96, 256, 512])
def test_fp8_head_sizes(D):
    """Contractions of one to sixteen K-blocks, including a partial last
    stage (96) and several stages (256, 512)."""
    rng = np.random.default_rng(D)
    B, L = 2, 72
    Q = wl.f32_to_bf16_bits((rng.standard_normal((B * L, D)) * 2).astype(np.float32))
    K = wl.f32_to_bf16_bits(rng.standard_normal((B * L, D)).astype(np.float32))
    note("fp8 head size %d" % D)
    S = fq.fp4q_gemm("fwd", _batched_fp8(fq.fp4q_quant1d_mxfp8(to_dev(Q)), B, L, D),
                     _batched_fp8(fq.fp4q_quant1d_mxfp8(to_dev(K)), B, L, D)).cpu().numpy()
    rq, rk = orc.quant1d_mxfp8(Q), orc.quant1d_mxfp8(K)
    Qd = orc.dequant_mxfp8(rq[0], rq[1], B * L, D)
    Kd = orc.dequant_mxfp8(rk[0], rk[1], B * L, D)
    for b in range(B):
        ref, bd = orc.gemm("fwd", Qd[b * L:(b + 1) * L], Kd[b * L:(b + 1) * L])
        check_gemm_tol(S[b], ref, bd, "D=%d batch %d" % (D, b))


def test_attention_config_sampled():
    """Q, K [4, 32, 4096, 128] -> MXFP8 -> S = Q K^T for all 128 heads
    (checked on sampled rows of the quantization and sampled S entries), and
    the 4096x4096 O-projection at 16384 tokens in 2D FP4."""
    a = wl.config_attn()
    B, Hh, L, D = a.Q.shape
    Qf = a.Q.reshape(B * Hh * L, D)
    Kf = a.K.reshape(B * Hh * L, D)
    note("attn mxfp8 quant")
    qq = fq.fp4q_quant1d_mxfp8(to_dev(Qf))
    qk = fq.fp4q_quant1d_mxfp8(to_dev(Kf))
    rng = np.random.default_rng(7)
    torch.cuda.synchronize()
    for q, x in ((qq, Qf), (qk, Kf)):
        # the first rows, the last rows and four random bands of 512 rows
        n = x.shape[0]
        starts = sorted({0, n - 512} | set(int(v) for v in rng.integers(0, n - 512, 4)))
        for r0 in starts:
            ref = orc.quant1d_mxfp8(np.ascontiguousarray(x[r0:r0 + 512]))
            c = q.codes[r0:r0 + 512].cpu().numpy()
            s = q.scales[r0:r0 + 512].cpu().numpy()
            assert np.array_equal(c, ref[0]) and np.array_equal(s, ref[1]), "MXFP8 band at row %d" % r0
    note("attn S = QK^T batched (%d heads)" % (B * Hh))
    S = fq.fp4q_gemm("fwd", _batched_fp8(qq, B * Hh, L, D), _batched_fp8(qk, B * Hh, L, D))
    torch.cuda.synchronize()
    bi = rng.integers(0, B * Hh, 1500)
    ii = rng.integers(0, L, 1500)
    jj = rng.integers(0, L, 1500)
    got = S[torch.from_numpy(bi).cuda(), torch.from_numpy(ii).cuda(), torch.from_numpy(jj).cuda()].cpu().numpy()
    del S
    ref = np.empty(len(bi))
    bnd = np.empty(len(bi))
    for t, (b, i, j) in enumerate(zip(bi, ii, jj)):
        qrow = Qf[b * L + i:b * L + i + 1]
        krow = Kf[b * L + j:b * L + j + 1]
        rq, rk = orc.quant1d_mxfp8(qrow), orc.quant1d_mxfp8(krow)
        qd = orc.dequant_mxfp8(rq[0], rq[1], 1, D)
        kd = orc.dequant_mxfp8(rk[0], rk[1], 1, D)
        c, bb = orc.gemm("fwd", qd, kd)
        ref[t], bnd[t] = c[0, 0], bb[0, 0]
    check_gemm_tol(got, ref, bnd, "attn S")

    L_o = a.o_proj
    note("attn O-projection quant + gemms")
    g = {nm: fq.fp4q_quant2d(to_dev(getattr(L_o, nm)), seed=0, stream_id=i + 1)
         for i, nm in enumerate(("X", "W", "dY"))}
    o = {nm: orc.quant2d(getattr(L_o, nm), orc.ROUND_SR, seed=0, stream=i + 1)
         for i, nm in enumerate(("X", "W", "dY"))}
    for nm in g:
        # codes, the transposed plane (read by dgrad and wgrad) and scales
        assert_planes_equal(g[nm], o[nm], "O-projection " + nm)
    deq = {nm: orc.dequant_fp4(o[nm][0], o[nm][2], *getattr(L_o, nm).shape) for nm in g}
    T, K, N = L_o.T, L_o.K, L_o.N
    for op, an, bn, (m, n) in (("fwd", "X", "W", (T, N)), ("dgrad", "dY", "W", (T, K)),
                               ("wgrad", "dY", "X", (N, K))):
        C = fq.fp4q_gemm(op, g[an], g[bn])
        i = rng.integers(0, m, 1500)
        j = rng.integers(0, n, 1500)
        gv = C[torch.from_numpy(i).cuda(), torch.from_numpy(j).cuda()].cpu().numpy()
        del C
        ref, bd = orc.gemm_sampled(op, deq[an], deq[bn], i, j)
        check_gemm_tol(gv, ref, bd, "O-proj " + op)
