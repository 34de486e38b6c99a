"""GPU parity of fp4q_gemm (MXFP4, fwd / dgrad / wgrad) with the oracle's
fp64 GEMM on the oracle's own dequantized operands, to the tolerance
|err| <= 1e-5 * sum_k |a||b| per element."""
import numpy as np
import pytest
import torch

import oracle as orc
import fp4_microscaling_quantization_quant2d_amd as fq
from fp4_microscaling_quantization_quant2d_amd import workloads as wl
from gpu_util import assert_planes_equal, check_gemm_tol, note, to_dev

pytestmark = pytest.mark.gpu

STREAMS = {"X": 1, "W": 2, "dY": 3}


def _quant_all(X, W, dY, seed=0):
    """GPU and oracle quantization of one layer's tensors."""
    g, o = {}, {}
    for nm, t in (("X", X), ("W", W), ("dY", dY)):
        g[nm] = fq.fp4q_quant2d(to_dev(t), seed=seed, stream_id=STREAMS[nm])
        o[nm] = orc.quant2d(t, orc.ROUND_SR, seed=seed, stream=STREAMS[nm])
    return g, o


def _deq(o, nm, shape):
    c, _, s = o[nm]
    return orc.dequant_fp4(c, s, shape[0], shape[1])


def _layer_full_check(X, W, dY, what):
    g, o = _quant_all(X, W, dY)
    for nm, t in (("X", X), ("W", W), ("dY", dY)):
        assert_planes_equal(g[nm], o[nm], "%s %s" % (what, nm))
    Xd, Wd, dYd = _deq(o, "X", X.shape), _deq(o, "W", W.shape), _deq(o, "dY", dY.shape)
    worst = 0.0
    for op, a, b, ra, rb in (("fwd", "X", "W", Xd, Wd), ("dgrad", "dY", "W", dYd, Wd),
                             ("wgrad", "dY", "X", dYd, Xd)):
        note("gemm %s %s" % (what, op))
        C = fq.fp4q_gemm(op, g[a], g[b])
        torch.cuda.synchronize()
        ref, bound = orc.gemm(op, ra, rb)
        worst = max(worst, check_gemm_tol(C.cpu().numpy(), ref, bound, "%s %s" % (what, op)))
    return worst


def test_tiny_all_ops():
    t = wl.tiny()
    _layer_full_check(t["A"], t["W"], t["dY"], "tiny")


@pytest.mark.parametrize("T,K,N", [(100, 200, 72), (32, 32, 32), (33, 65, 97), (512, 640, 384),
                                   (260, 300, 520), (64, 1056, 96), (1, 1, 1), (1, 70, 3), (3, 1, 257)])
def test_ragged_and_multi_tile(T, K, N):
    L = wl.linear_layer("tiny:ragged", T, K, N, T * 7 + K)
    _layer_full_check(L.X, L.W, L.dY, "%dx%dx%d" % (T, K, N))


def test_exact_on_grid_values():
    """Operands on the E2M1 grid with unit scales: every product and partial
    sum is exact in fp32, so the GPU must match the fp64 result exactly."""
    rng = np.random.default_rng(4)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)
    X = (grid[rng.integers(0, 8, (64, 128))] * rng.choice([-1, 1], (64, 128))).astype(np.float32)
    W = (grid[rng.integers(0, 8, (96, 128))] * rng.choice([-1, 1], (96, 128))).astype(np.float32)
    X[:, 0] = 6.0
    W[:, 0] = 6.0
    X[0, :] = 6.0
    W[0, :] = 6.0
    note("gemm exact grid")
    gx = fq.fp4q_quant2d(to_dev(X), round_mode="rne")
    gw = fq.fp4q_quant2d(to_dev(W), round_mode="rne")
    C = fq.fp4q_gemm("fwd", gx, gw).cpu().numpy()
    assert np.array_equal(C.astype(np.float64), X.astype(np.float64) @ W.astype(np.float64).T)


def _sampled_layer_check(L, what, n_samples=4096):
    """Full-size layer: every GPU plane vs the oracle, GEMMs at sampled outputs."""
    rng = np.random.default_rng(99)
    g, o = _quant_all(L.X, L.W, L.dY)
    for nm in ("X", "W", "dY"):
        assert_planes_equal(g[nm], o[nm], "%s %s" % (what, nm))
    Xd = _deq(o, "X", L.X.shape)
    Wd = _deq(o, "W", L.W.shape)
    dYd = _deq(o, "dY", L.dY.shape)
    T, K, N = L.T, L.K, L.N
    for op, a, b, ra, rb, (m, n) in (("fwd", "X", "W", Xd, Wd, (T, N)),
                                     ("dgrad", "dY", "W", dYd, Wd, (T, K)),
                                     ("wgrad", "dY", "X", dYd, Xd, (N, K))):
        note("gemm %s %s (%d x %d)" % (what, op, m, n))
        C = fq.fp4q_gemm(op, g[a], g[b])
        ci = np.concatenate([rng.integers(0, m, n_samples), [0, m - 1, m - 1, 0]])
        cj = np.concatenate([rng.integers(0, n, n_samples), [0, n - 1, 0, n - 1]])
        got = C[torch.from_numpy(ci).cuda(), torch.from_numpy(cj).cuda()].cpu().numpy()
        del C
        ref, bound = orc.gemm_sampled(op, ra, rb, ci, cj)
        check_gemm_tol(got, ref, bound, "%s %s" % (what, op))


@pytest.mark.parametrize("i", [0, 1])
def test_1b_layers_sampled(i):
    _sampled_layer_check(wl.layer_1b(i), "1B layer %d" % i)


@pytest.mark.parametrize("i", [0, 1, 2, 3], ids=[nm for nm, _, _ in wl.LAYERS_7B])
def test_7b_layers_sampled(i):
    """Every 7B layer (QKV, O, up, down): all three planes of X, W and dY
    bit-exact at full size, and fwd / dgrad / wgrad at 4096 sampled outputs
    plus the four corners, in the launch configuration the benchmark uses."""
    _sampled_layer_check(wl.layer_7b(i), "7B " + wl.LAYERS_7B[i][0], n_samples=4096)


# Grids of 512 or more 256x256 tiles (two or more per CU), one op per shape
# with the large grid: fwd, dgrad (transposed B scales), wgrad (both
# transposed).  K = 1056 ends inside a 256-value pair; the last shape has
# ragged edges in both output dimensions.
@pytest.mark.parametrize("T,K,N", [(4096, 1056, 8192), (4096, 8192, 1056), (1056, 4096, 8192),
                                   (4056, 1056, 8092)])
def test_large_grids_sampled(T, K, N):
    L = wl.linear_layer("tiny:grid", T, K, N, T + 3 * K + 7 * N)
    _sampled_layer_check(L, "grid %dx%dx%d" % (T, K, N), n_samples=20000)


def test_gemm_into_strided_output():
    """C with a leading dimension larger than N; the gap stays untouched."""
    L = wl.linear_layer("tiny:ldc", 96, 128, 64, 1)
    g, o = _quant_all(L.X, L.W, L.dY)
    C = torch.full((96, 80), 7.0, device="cuda")
    note("gemm strided C")
    fq.fp4q_gemm("fwd", g["X"], g["W"], c=C[:, :64])
    ref, bound = orc.gemm("fwd", _deq(o, "X", L.X.shape), _deq(o, "W", L.W.shape))
    Ch = C.cpu().numpy()
    check_gemm_tol(Ch[:, :64], ref, bound, "strided")
    assert np.all(Ch[:, 64:] == 7.0)


def _padded_scales(q, pad_byte):
    """The same quantized tensor with its scale grid copied into rows padded
    to a multiple of 8 bytes (plus 8), the padding filled with pad_byte."""
    R32, C32 = q.scales.shape
    wide = torch.full((R32, (C32 + 7) // 8 * 8 + 8), pad_byte, dtype=torch.uint8, device="cuda")
    wide[:, :C32].copy_(q.scales)
    return fq.QTensor(q.fmt, q.rows, q.cols, q.codes, wide[:, :C32], q.codes_t)


@pytest.mark.parametrize("T,K,N", [(300, 1184, 200), (520, 96, 744)])
def test_padded_scale_grids(T, K, N):
    """Scale grids with padded rows (ld_s beyond C/32, garbage in the
    padding) give the same C, bit for bit, as the tight grids, for ragged
    K-block counts and partial slab tiles in every orientation; both are
    within the bound of the oracle."""
    L = wl.linear_layer("tiny:scalepad", T, K, N, T + 3 * K + 5 * N)
    g, o = _quant_all(L.X, L.W, L.dY)
    gp = {nm: _padded_scales(q, 0xA7) for nm, q in g.items()}
    Xd, Wd, dYd = _deq(o, "X", L.X.shape), _deq(o, "W", L.W.shape), _deq(o, "dY", L.dY.shape)
    for op, a, b, ra, rb in (("fwd", "X", "W", Xd, Wd), ("dgrad", "dY", "W", dYd, Wd),
                             ("wgrad", "dY", "X", dYd, Xd)):
        note("gemm padded scale grids %dx%dx%d %s" % (T, K, N, op))
        tight = fq.fp4q_gemm(op, g[a], g[b])
        padded = fq.fp4q_gemm(op, gp[a], gp[b])
        torch.cuda.synchronize()
        assert torch.equal(tight, padded), "%s: padded scale grids change C" % op
        ref, bound = orc.gemm(op, ra, rb)
        check_gemm_tol(padded.cpu().numpy(), ref, bound, "padded %s" % op)


@pytest.mark.parametrize("T,K,N", [(64, 20480, 96), (20480, 64, 96)])
def test_long_contraction(T, K, N):
    """Contractions of 20480: fwd over K (first shape) and wgrad over the
    tokens (second shape) run past the first two batches of preloaded scale
    bytes."""
    L = wl.linear_layer("tiny:longk", T, K, N, T + K)
    _layer_full_check(L.X, L.W, L.dY, "long %dx%dx%d" % (T, K, N))


def _batched(q, n_items, rows, rows_t):
    """View a stacked 2D-FP4 quantization as n_items independent matrices of
    `rows` rows each; the transposed plane advances rows/2 bytes per item."""
    ld, lds = q.codes.shape[1], q.scales.shape[1]
    return fq.QTensor(fq.FMT_FP4_2D32, rows, q.cols, q.codes.view(n_items, rows, ld),
                      q.scales.view(n_items, rows // 32, lds), q.codes_t, batch=n_items,
                      bstride=rows * ld, bstride_t=rows // 2, bstride_s=(rows // 32) * lds)


def test_batched_fp4_all_ops():
    """Three independent layers stacked along the token (X, dY) and output
    (W) dimensions, multiplied as one batched call per op."""
    B, T, K, N = 3, 96, 160, 64
    L = wl.linear_layer("tiny:batch", B * T, K, B * N, 5)
    X, W = L.X, L.W
    dY = wl.f32_to_bf16_bits(np.random.default_rng(6).standard_normal((B * T, N)).astype(np.float32) * 1e-3)
    g, o = _quant_all(X, W, dY)
    Xd, Wd, dYd = _deq(o, "X", X.shape), _deq(o, "W", W.shape), _deq(o, "dY", dY.shape)
    bx, bw, bdy = _batched(g["X"], B, T, T), _batched(g["W"], B, N, N), _batched(g["dY"], B, T, T)
    for op, a, b, ra, rb, ma, mb in (("fwd", bx, bw, Xd, Wd, T, N), ("dgrad", bdy, bw, dYd, Wd, T, N),
                                     ("wgrad", bdy, bx, dYd, Xd, T, T)):
        note("gemm batched fp4 %s" % op)
        C = fq.fp4q_gemm(op, a, b).cpu().numpy()
        assert C.shape[0] == B
        for i in range(B):
            ref, bound = orc.gemm(op, ra[i * ma:(i + 1) * ma], rb[i * mb:(i + 1) * mb])
            check_gemm_tol(C[i], ref, bound, "batched %s item %d" % (op, i))
