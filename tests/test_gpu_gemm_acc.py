"""GPU parity of weight-gradient accumulation (fp4q_gemm_ex with
FP4Q_GEMM_ACCUMULATE: C += op(a, b), the dW = dY^T X of "Stable FP4 Training
via Transposition-Invariant Block Quantization", Sec. 3 "Application to
linear layers", summed over micro-batches).

Tolerance: the product's own bound |err| <= 1e-5 * sum|a||b| plus one fp32
rounding of the sum, at most 2^-24 of |C_old + product|; the test allows
1e-5 * sum|a||b| + 2^-23 * |C_old| (the product's share of the last rounding
is far inside its own 1e-5 bound)."""
import numpy as np
import pytest
import torch

import oracle as orc
import fp4_microscaling_quantization_quant2d_amd as fq
from fp4_microscaling_quantization_quant2d_amd import workloads as wl
from gpu_util import note, to_dev

pytestmark = pytest.mark.gpu

STREAMS = {"X": 1, "W": 2, "dY": 3}
VIEWS = {"fwd": (("X", 0), ("W", 0)), "dgrad": (("dY", 0), ("W", 1)), "wgrad": (("dY", 1), ("X", 1))}


def _quant(t, nm, layout):
    r, c = t.shape
    g = fq.fp4q_quant2d(to_dev(t), out=fq.alloc_fp4(r, c, block=layout), seed=1, stream_id=STREAMS[nm])
    if layout == "1d":
        codes, codes_t, s, st = orc.quant_act1d(t, seed=1, stream=STREAMS[nm])
        return g, (orc.dequant_fp4_blocks(codes, s, r, c, 1, 32), orc.dequant_fp4_blocks(codes_t, st, c, r, 1, 32).T)
    c2, _, s2 = orc.quant2d_block(t, layout, seed=1, stream=STREAMS[nm])
    d = orc.dequant_fp4_blocks(c2, s2, r, c, layout, layout)
    return g, (d, d)


def _check_acc(got, c_old, ref, bound, what):
    err = np.abs(got.astype(np.float64) - (c_old.astype(np.float64) + ref))
    tol = 1e-5 * bound + 2.0 ** -23 * np.abs(c_old.astype(np.float64))
    bad = err > tol
    assert not bad.any(), "%s: %d elements out of tolerance, first at %s" % (what, int(bad.sum()),
                                                                             np.argwhere(bad)[0].tolist())


@pytest.mark.parametrize("T,K,N", [(320, 448, 288), (512, 512, 256), (100, 200, 72)])
@pytest.mark.parametrize("layouts", [{"X": 32, "W": 32, "dY": 32}, {"X": "1d", "W": 32, "dY": 32},
                                     {"X": 64, "W": 64, "dY": 64}])
def test_accumulate_all_ops(T, K, N, layouts):
    L = wl.linear_layer("tiny:acc", T, K, N, T + 7 * K)
    q, d = {}, {}
    for nm in ("X", "W", "dY"):
        q[nm], d[nm] = _quant(getattr(L, nm), nm, layouts[nm])
    rng = np.random.default_rng(T + K)
    for op in ("fwd", "dgrad", "wgrad"):
        (a, va), (b, vb) = VIEWS[op]
        if layouts[a] == "1d":
            continue  # accumulation takes an A operand with a square-block grid
        M, Nn = fq.gemm_out_shape(op, q[a], q[b])
        c_old = (rng.standard_normal((M, Nn)) * 3.0).astype(np.float32)
        c = torch.from_numpy(c_old.copy()).cuda()
        note("gemm acc %s %dx%dx%d %s" % (op, T, K, N, layouts))
        fq.fp4q_gemm(op, q[a], q[b], c=c, accumulate=True)
        torch.cuda.synchronize()
        ref, bound = orc.gemm(op, d[a][va], d[b][vb])
        _check_acc(c.cpu().numpy(), c_old, ref, bound, "%s %s" % (op, layouts))


def test_accumulate_twice_equals_sum_of_two_micro_batches():
    """Two micro-batches of one layer accumulated into one dW, then compared
    with the oracle's sum of the two products (strided C as well)."""
    T, K, N = 256, 384, 320
    Ls = [wl.linear_layer("tiny:acc2", T, K, N, 100 + i) for i in range(2)]
    dw = torch.zeros((N, K + 8), dtype=torch.float32, device="cuda")[:, :K]
    total = np.zeros((N, K))
    bound = np.zeros((N, K))
    for i, L in enumerate(Ls):
        qd, dd = _quant(L.dY, "dY", 32)
        qx, dx = _quant(L.X, "X", 32)
        note("gemm acc micro-batch %d" % i)
        fq.fp4q_gemm("wgrad", qd, qx, c=dw, accumulate=True)
        r, b = orc.gemm("wgrad", dd[1], dx[1])
        total += r
        bound += b
    torch.cuda.synchronize()
    got = dw.cpu().numpy().astype(np.float64)
    # two fp32 roundings of partial sums
    tol = 1e-5 * bound + 2.0 ** -22 * np.abs(total)
    assert (np.abs(got - total) <= tol).all()


def test_7b_qkv_wgrad_accumulate_sampled():
    """Full-size QKV weight gradient accumulated onto a resident dW, at sampled outputs."""
    L = wl.layer_7b(0)
    qd = fq.fp4q_quant2d(to_dev(L.dY), seed=0, stream_id=3)
    qx = fq.fp4q_quant2d(to_dev(L.X), seed=0, stream_id=1)
    cd, _, sd = orc.quant2d(L.dY, seed=0, stream=3)
    cx, _, sx = orc.quant2d(L.X, seed=0, stream=1)
    dd = orc.dequant_fp4(cd, sd, L.T, L.N)
    dx = orc.dequant_fp4(cx, sx, L.T, L.K)
    g = torch.Generator(device="cuda").manual_seed(3)
    c = torch.randn((L.N, L.K), device="cuda", generator=g)
    rng = np.random.default_rng(2)
    ci = rng.integers(0, L.N, 3000)
    cj = rng.integers(0, L.K, 3000)
    idx = (torch.from_numpy(ci).cuda(), torch.from_numpy(cj).cuda())
    c_old = c[idx].cpu().numpy()
    note("gemm acc 7B qkv wgrad")
    fq.fp4q_gemm("wgrad", qd, qx, c=c, accumulate=True)
    got = c[idx].cpu().numpy()
    ref, bound = orc.gemm_sampled("wgrad", dd, dx, ci, cj)
    _check_acc(got, c_old, ref, bound, "7B qkv wgrad acc")
