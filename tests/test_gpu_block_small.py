"""GPU parity of the 16x16 and 8x8 scale blocks (Table 4 of "Stable FP4
Training via Transposition-Invariant Block Quantization" compares block sides
8, 16, 32, 64): the quantizer bit-exact against the oracle's square-block
quantizer (codes, transposed codes and the grid over the 32-padded planes),
and fwd / dgrad / wgrad on such operands -- each 32-K MFMA split into one MFMA
per sub-block -- within 1e-5 * sum|a||b| of the oracle's fp64 product of its
own dequantized operands, including contractions that 8x8 blocks run in
accumulating chunks and the full 7B QKV and down layers at sampled outputs."""
import numpy as np
import pytest
import torch

import oracle as orc
import fp4_microscaling_quantization_quant2d_amd as fq
from fp4_microscaling_quantization_quant2d_amd import workloads as wl
from gpu_util import assert_planes_equal, check_gemm_tol, note, to_dev

pytestmark = pytest.mark.gpu

OPS = (("fwd", "X", "W"), ("dgrad", "dY", "W"), ("wgrad", "dY", "X"))


def _quant(x, b, mode="sr", seed=0, stream=0):
    out = fq.alloc_fp4(x.shape[0], x.shape[1], block=b)
    return fq.fp4q_quant2d(to_dev(x), out=out, round_mode=mode, seed=seed, stream_id=stream)


@pytest.mark.parametrize("b", [16, 8])
@pytest.mark.parametrize("shape", [(1, 1), (33, 65), (100, 300), (129, 257), (256, 256), (8, 40)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantizer_bit_exact(b, shape, dtype):
    rng = np.random.default_rng(shape[0] * 7 + shape[1] + b)
    x = (rng.standard_normal(shape) * np.exp(2 * rng.standard_normal((shape[0], 1)))
         * np.exp(rng.standard_normal((1, shape[1])))).astype(np.float32)
    if dtype == "bf16":
        x = wl.f32_to_bf16_bits(x)
    for mode, om in (("sr", orc.ROUND_SR), ("rne", orc.ROUND_RNE)):
        note("quant b%d %s %s %s" % (b, shape, dtype, mode))
        q = _quant(x, b, mode, seed=99, stream=3)
        assert_planes_equal(q, orc.quant2d_block(x, b, om, seed=99, stream=3), "b%d %s %s" % (b, shape, mode))


def _layer(T, K, N, b, seed=0):
    L = wl.linear_layer("tiny:sub%d" % b, T, K, N, T + 3 * K + 5 * N + b)
    g, deq = {}, {}
    for sid, nm in enumerate(("X", "W", "dY"), start=1):
        t = getattr(L, nm)
        g[nm] = _quant(t, b, seed=seed, stream=sid)
        c, ct, s = orc.quant2d_block(t, b, orc.ROUND_SR, seed=seed, stream=sid)
        assert_planes_equal(g[nm], (c, ct, s), "b%d %s" % (b, nm))
        deq[nm] = orc.dequant_fp4_blocks(c, s, t.shape[0], t.shape[1], b, b)
    return L, g, deq


@pytest.mark.parametrize("b", [16, 8])
@pytest.mark.parametrize("T,K,N", [(100, 200, 72), (32, 32, 32), (260, 300, 520), (512, 640, 384),
                                   (64, 1056, 96)])
def test_gemm_all_ops(b, T, K, N):
    L, g, deq = _layer(T, K, N, b)
    for op, a, bb in OPS:
        note("gemm b%d %s %dx%dx%d" % (b, op, T, K, N))
        C = fq.fp4q_gemm(op, g[a], g[bb])
        torch.cuda.synchronize()
        ref, bound = orc.gemm(op, deq[a], deq[bb])
        check_gemm_tol(C.cpu().numpy(), ref, bound, "b%d %s" % (b, op))


@pytest.mark.parametrize("b", [16, 8])
def test_long_contraction_and_accumulate(b):
    """Contractions of 8448 (fwd over K, wgrad over the tokens): 8x8 blocks
    run them as three chunks accumulating in C; and C += A B^T on top of
    existing values."""
    for T, K, N in ((64, 8448, 96), (8448, 64, 96)):
        L, g, deq = _layer(T, K, N, b, seed=3)
        for op, a, bb in OPS:
            note("gemm b%d long %s %dx%dx%d" % (b, op, T, K, N))
            C = fq.fp4q_gemm(op, g[a], g[bb])
            torch.cuda.synchronize()
            ref, bound = orc.gemm(op, deq[a], deq[bb])
            check_gemm_tol(C.cpu().numpy(), ref, bound, "b%d long %s" % (b, op))
    L, g, deq = _layer(96, 320, 160, b, seed=4)
    C0 = torch.randn(96, 160, device="cuda")
    C = C0.clone()
    note("gemm b%d accumulate" % b)
    fq.fp4q_gemm("fwd", g["X"], g["W"], c=C, accumulate=True)
    ref, bound = orc.gemm("fwd", deq["X"], deq["W"])
    old = C0.cpu().numpy().astype(np.float64)
    got = C.cpu().numpy().astype(np.float64)
    err = np.abs(got - (old + ref))
    assert np.all(err <= 1e-5 * bound + 2.0 ** -23 * np.abs(old + ref) + 1e-300)


@pytest.mark.parametrize("b", [16, 8])
@pytest.mark.parametrize("i", [0, 3])
def test_7b_layers_sampled(b, i):
    """Full 7B QKV (K = 4096) and down (K = 11008) layers at b = 16 and 8:
    all planes bit-exact, GEMMs at 2048 sampled outputs plus the corners."""
    L = wl.layer_7b(i)
    rng = np.random.default_rng(31 + i + b)
    g, deq = {}, {}
    for sid, nm in enumerate(("X", "W", "dY"), start=1):
        t = getattr(L, nm)
        note("7B b%d layer %d quant %s" % (b, i, nm))
        g[nm] = _quant(t, b, seed=0, stream=sid)
        c, ct, s = orc.quant2d_block(t, b, orc.ROUND_SR, seed=0, stream=sid)
        assert_planes_equal(g[nm], (c, ct, s), "7B b%d %s" % (b, nm))
        deq[nm] = orc.dequant_fp4_blocks(c, s, t.shape[0], t.shape[1], b, b)
        del c, ct, s
    T, K, N = L.T, L.K, L.N
    for (op, a, bb), (m, n) in zip(OPS, ((T, N), (T, K), (N, K))):
        note("7B b%d layer %d %s" % (b, i, op))
        C = fq.fp4q_gemm(op, g[a], g[bb])
        ci = np.concatenate([rng.integers(0, m, 2048), [0, m - 1, m - 1, 0]])
        cj = np.concatenate([rng.integers(0, n, 2048), [0, n - 1, 0, n - 1]])
        got = C[torch.from_numpy(ci).cuda(), torch.from_numpy(cj).cuda()].cpu().numpy()
        del C
        ref, bound = orc.gemm_sampled(op, deq[a], deq[bb], ci, cj)
        check_gemm_tol(got, ref, bound, "7B b%d %s" % (b, op))


def test_mixed_block_sides_refused():
    L, g16, _ = _layer(64, 64, 64, 16)
    g32 = fq.fp4q_quant2d(to_dev(L.W), seed=0, stream_id=2)
    with pytest.raises(fq.Fp4qError):
        fq.fp4q_gemm("fwd", g16["X"], g32)
