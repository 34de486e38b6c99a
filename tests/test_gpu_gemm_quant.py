"""GPU parity of fp4q_gemm_quant: a GEMM whose epilogue quantizes its own
fp32 result into 2D 32x32 FP4 planes (row plane, transposed plane, scale
grid) instead of writing it.  The fused planes must equal, bit for bit, the
oracle's 2D quantization of the fp32 C that fp4q_gemm returns for the same
operands (and that C is itself within 1e-5 * sum|a||b| of the oracle's fp64
product), for every op, ragged and multi-tile shapes, SR and RNE, 64x64-block
operands, a row-plane-only output, device-resident seeds, and a full-size
7B output."""
import numpy as np
import pytest
import torch

import oracle as orc
import fp4_microscaling_quantization_quant2d_amd as fq
from fp4_microscaling_quantization_quant2d_amd import workloads as wl
from gpu_util import assert_planes_equal, check_gemm_tol, note, to_dev

pytestmark = pytest.mark.gpu

OPERANDS = {"fwd": ("X", "W"), "dgrad": ("dY", "W"), "wgrad": ("dY", "X")}


def _layer(T, K, N, block=32):
    L = wl.linear_layer("tiny:qepi", T, K, N, T * 5 + K * 3 + N)
    g, deq = {}, {}
    for sid, nm in enumerate(("X", "W", "dY"), start=1):
        t = getattr(L, nm)
        out = fq.alloc_fp4(t.shape[0], t.shape[1], block=block)
        g[nm] = fq.fp4q_quant2d(to_dev(t), out=out, seed=1, stream_id=sid)
        if block == 32:
            c, _, s = orc.quant2d(t, orc.ROUND_SR, seed=1, stream=sid)
            deq[nm] = orc.dequant_fp4(c, s, t.shape[0], t.shape[1])
    return L, g, deq


@pytest.mark.parametrize("T,K,N", [(256, 256, 256), (100, 200, 72), (260, 300, 520), (512, 640, 384),
                                   (33, 1056, 97)])
@pytest.mark.parametrize("op", ["fwd", "dgrad", "wgrad"])
def test_fused_planes_equal_oracle_quant_of_c(T, K, N, op):
    L, g, deq = _layer(T, K, N)
    a, b = OPERANDS[op]
    note("gemm_quant %s %dx%dx%d" % (op, T, K, N))
    C = fq.fp4q_gemm(op, g[a], g[b])
    Q = fq.fp4q_gemm_quant(op, g[a], g[b], seed=77, stream_id=9)
    torch.cuda.synchronize()
    Ch = C.cpu().numpy()
    ref, bound = orc.gemm(op, deq[a], deq[b])
    check_gemm_tol(Ch, ref, bound, "C %s" % op)
    assert_planes_equal(Q, orc.quant2d(np.ascontiguousarray(Ch), orc.ROUND_SR, seed=77, stream=9),
                        "fused %s %dx%dx%d" % (op, T, K, N))


@pytest.mark.parametrize("op", ["fwd", "dgrad", "wgrad"])
def test_rne_rows_only_and_64_blocks(op):
    """RNE rounding, a row-plane-only output, and operands with 64x64 blocks."""
    L, g, _ = _layer(300, 520, 200, block=64)
    a, b = OPERANDS[op]
    note("gemm_quant rne/rows-only/b64 %s" % op)
    C = fq.fp4q_gemm(op, g[a], g[b]).cpu().numpy()
    Qr = fq.fp4q_gemm_quant(op, g[a], g[b], round_mode="rne")
    assert_planes_equal(Qr, orc.quant2d(C, orc.ROUND_RNE), "rne %s" % op)
    Qs = fq.fp4q_gemm_quant(op, g[a], g[b], seed=5, stream_id=2, transposed=False)
    torch.cuda.synchronize()
    rc, _, rs = orc.quant2d(C, orc.ROUND_SR, seed=5, stream=2)
    assert Qs.codes_t is None
    assert np.array_equal(Qs.codes.cpu().numpy(), rc) and np.array_equal(Qs.scales.cpu().numpy(), rs)


def test_device_seed_in_a_graph():
    """The epilogue reads a device-resident seed when the kernel runs: a
    captured graph replayed under two seeds gives each seed's planes."""
    L, g, _ = _layer(192, 256, 320)
    C = fq.fp4q_gemm("fwd", g["X"], g["W"]).cpu().numpy()
    out = fq.alloc_fp4(192, 320)
    seed_dev = torch.zeros(1, dtype=torch.int64, device="cuda")

    def seq():
        fq.fp4q_gemm_quant("fwd", g["X"], g["W"], out=out, seed=1000, stream_id=4, seed_dev=seed_dev)

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        seq()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        seq()
    for dseed in (3, 4):
        note("gemm_quant graph seed %d" % dseed)
        seed_dev.fill_(dseed)
        graph.replay()
        torch.cuda.synchronize()
        assert_planes_equal(out, orc.quant2d(C, orc.ROUND_SR, seed=1000 + dseed, stream=4), "seed %d" % dseed)


def test_7b_down_dgrad_full_size():
    """The 7B down projection's dgrad, dX = dY W [8192 x 11008] (the up
    projection's output-gradient shape): every fused plane against the
    oracle's quantization of the plain launch's fp32 C, at full size."""
    L = wl.layer_7b(3)
    note("gemm_quant 7B down dgrad: quantize operands")
    qdy = fq.fp4q_quant2d(to_dev(L.dY), seed=0, stream_id=3)
    qw = fq.fp4q_quant2d(to_dev(L.W), seed=0, stream_id=2)
    note("gemm_quant 7B down dgrad: plain and fused")
    C = fq.fp4q_gemm("dgrad", qdy, qw)
    Q = fq.fp4q_gemm_quant("dgrad", qdy, qw, seed=0, stream_id=19)
    torch.cuda.synchronize()
    Ch = C.cpu().numpy()
    del C
    assert_planes_equal(Q, orc.quant2d(Ch, orc.ROUND_SR, seed=0, stream=19), "7B down dgrad")
