"""GPU parity for 64x64 scale blocks (FP4Q_FMT_FP4_2D64): quantization
bit-exact against the oracle's square-block quantizer (codes, transposed
codes, scale grid), GEMMs on 64-block and mixed 32/64-block operands within
|err| <= 1e-5 * sum|a||b| of the oracle's fp64 product of its own
dequantized operands, and dequantization."""
import numpy as np
import pytest
import torch

import oracle as orc
import fp4_microscaling_quantization_quant2d_amd as fq
from fp4_microscaling_quantization_quant2d_amd import workloads as wl
from fp4_microscaling_quantization_quant2d_amd.workloads import f32_to_bf16_bits
from gpu_util import assert_planes_equal, check_gemm_tol, note, to_dev

pytestmark = pytest.mark.gpu

STREAMS = {"X": 1, "W": 2, "dY": 3}


def _input(shape, seed, dtype):
    rng = np.random.default_rng(seed)
    r, c = shape
    x = (rng.standard_normal(shape) * np.exp(rng.standard_normal((r, 1)))).astype(np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


@pytest.mark.parametrize("shape", [(1, 1), (33, 65), (100, 130), (128, 128), (200, 96), (300, 257),
                                   (64, 64), (65, 64), (129, 385)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", ["sr", "rne"])
def test_quant64_bit_exact(shape, dtype, mode):
    x = _input(shape, sum(shape), dtype)
    note("quant2d b64 %s %s %s" % (shape, dtype, mode))
    q = fq.fp4q_quant2d(to_dev(x), out=fq.alloc_fp4(*shape, block=64), round_mode=mode, seed=4, stream_id=6)
    ref = orc.quant2d_block(x, 64, orc.ROUND_SR if mode == "sr" else orc.ROUND_RNE, seed=4, stream=6)
    assert q.fmt == fq.FMT_FP4_2D64 and tuple(q.scales.shape) == ref[2].shape
    assert_planes_equal(q, ref, "b64 %s" % (shape,))


def test_quant64_batch():
    shapes = [(100, 130), (256, 64), (33, 200)]
    xs = [_input(s, 9 + k, "bf16") for k, s in enumerate(shapes)]
    outs = fq.fp4q_quant2d_batch([(to_dev(x), fq.alloc_fp4(*s, block=64), 20 + k)
                                  for k, (x, s) in enumerate(zip(xs, shapes))], seed=2)
    for k, (x, o) in enumerate(zip(xs, outs)):
        assert_planes_equal(o, orc.quant2d_block(x, 64, orc.ROUND_SR, seed=2, stream=20 + k), "batch %d" % k)


def _quant(t, nm, block, seed=0):
    g = fq.fp4q_quant2d(to_dev(t), out=fq.alloc_fp4(*t.shape, block=block), seed=seed, stream_id=STREAMS[nm])
    c, _, s = orc.quant2d_block(t, block, orc.ROUND_SR, seed=seed, stream=STREAMS[nm])
    return g, orc.dequant_fp4_blocks(c, s, t.shape[0], t.shape[1], block, block)


def _layer_check(L, blocks, what):
    q, d = {}, {}
    for nm in ("X", "W", "dY"):
        q[nm], d[nm] = _quant(getattr(L, nm), nm, blocks[nm])
    for op, a, b in (("fwd", "X", "W"), ("dgrad", "dY", "W"), ("wgrad", "dY", "X")):
        note("gemm %s %s blocks %s" % (what, op, blocks))
        C = fq.fp4q_gemm(op, q[a], q[b])
        torch.cuda.synchronize()
        ref, bound = orc.gemm(op, d[a], d[b])
        check_gemm_tol(C.cpu().numpy(), ref, bound, "%s %s" % (what, op))


@pytest.mark.parametrize("T,K,N", [(320, 448, 288), (512, 640, 384), (100, 200, 72), (64, 1056, 96)])
def test_gemm_64_blocks_all_ops(T, K, N):
    L = wl.linear_layer("tiny:b64", T, K, N, T * 5 + K)
    _layer_check(L, {"X": 64, "W": 64, "dY": 64}, "%dx%dx%d" % (T, K, N))


@pytest.mark.parametrize("blocks", [{"X": 64, "W": 32, "dY": 64}, {"X": 32, "W": 64, "dY": 32},
                                    {"X": 64, "W": 32, "dY": 32}])
def test_gemm_mixed_blocks(blocks):
    L = wl.linear_layer("tiny:b64mix", 288, 520, 320, 11)
    _layer_check(L, blocks, "mixed")


def test_dequant64_both_planes():
    x = _input((130, 200), 3, "bf16")
    q = fq.fp4q_quant2d(to_dev(x), out=fq.alloc_fp4(130, 200, block=64), seed=1, stream_id=1)
    c, ct, s = orc.quant2d_block(x, 64, orc.ROUND_SR, seed=1, stream=1)
    y = fq.fp4q_dequant(q).cpu().numpy()
    yt = fq.fp4q_dequant(q, transposed=True).cpu().numpy()
    assert np.array_equal(y.astype(np.float64), orc.dequant_fp4_blocks(c, s, 130, 200, 64, 64))
    assert np.array_equal(yt.astype(np.float64),
                          orc.dequant_fp4_blocks(ct, np.ascontiguousarray(s.T), 200, 130, 64, 64))


def test_7b_qkv_64_blocks_sampled():
    """Full-size QKV layer with 64x64 blocks: planes bit-exact, GEMMs at sampled outputs."""
    L = wl.layer_7b(0)
    rng = np.random.default_rng(5)
    q, d = {}, {}
    for nm in ("X", "W", "dY"):
        t = getattr(L, nm)
        q[nm] = fq.fp4q_quant2d(to_dev(t), out=fq.alloc_fp4(*t.shape, block=64), seed=0, stream_id=STREAMS[nm])
        ref = orc.quant2d_block(t, 64, orc.ROUND_SR, seed=0, stream=STREAMS[nm])
        assert_planes_equal(q[nm], ref, "7B b64 %s" % nm)
        d[nm] = orc.dequant_fp4_blocks(ref[0], ref[2], t.shape[0], t.shape[1], 64, 64)
    T, K, N = L.T, L.K, L.N
    for op, a, b, (m, n) in (("fwd", "X", "W", (T, N)), ("dgrad", "dY", "W", (T, K)), ("wgrad", "dY", "X", (N, K))):
        note("gemm 7B b64 %s" % op)
        C = fq.fp4q_gemm(op, q[a], q[b])
        ci = rng.integers(0, m, 3000)
        cj = rng.integers(0, n, 3000)
        got = C[torch.from_numpy(ci).cuda(), torch.from_numpy(cj).cuda()].cpu().numpy()
        del C
        ref, bound = orc.gemm_sampled(op, d[a], d[b], ci, cj)
        check_gemm_tol(got, ref, bound, "7B b64 %s" % op)
