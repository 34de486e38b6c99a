"""GPU parity of the bf16-output GEMMs (fp4q_gemm_ex with
FP4Q_GEMM_OUT_BF16).  Each output is the fp32 result rounded to nearest-even
bf16, so against the oracle's fp64 product it is within the fp32 bound
1e-5 * sum|a||b| plus half a bf16 ulp, at most 2^-8 of |C| (bf16 keeps 8
significant bits); the test allows 1e-5 * sum|a||b| * (1 + 2^-8) +
2^-8 * |ref|.  Covers all three ops with ragged tiles, both block sides,
the batched MXFP8 S = Q K^T and the full 7B QKV layer at sampled outputs."""
import numpy as np
import pytest
import torch

import oracle as orc
import fp4_microscaling_quantization_quant2d_amd as fq
from fp4_microscaling_quantization_quant2d_amd import workloads as wl
from gpu_util import note, to_dev

pytestmark = pytest.mark.gpu

STREAMS = {"X": 1, "W": 2, "dY": 3}


def check_bf16(got, ref, bound, what):
    g = got.float().cpu().numpy().astype(np.float64) if isinstance(got, torch.Tensor) else got
    tol = 1e-5 * bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(ref)
    bad = np.abs(g - ref) > tol
    assert not bad.any(), "%s: %d out of tolerance, first at %s" % (what, int(bad.sum()),
                                                                    np.argwhere(bad)[0].tolist())


@pytest.mark.parametrize("T,K,N", [(320, 448, 288), (512, 512, 256), (100, 200, 72)])
@pytest.mark.parametrize("block", [32, 64])
def test_bf16_output_all_ops(T, K, N, block):
    L = wl.linear_layer("tiny:bf16out", T, K, N, 3 * T + K)
    q, d = {}, {}
    for nm in ("X", "W", "dY"):
        t = getattr(L, nm)
        q[nm] = fq.fp4q_quant2d(to_dev(t), out=fq.alloc_fp4(*t.shape, block=block), seed=2,
                                stream_id=STREAMS[nm])
        c, _, s = orc.quant2d_block(t, block, orc.ROUND_SR, seed=2, stream=STREAMS[nm])
        d[nm] = orc.dequant_fp4_blocks(c, s, t.shape[0], t.shape[1], block, block)
    for op, a, b in (("fwd", "X", "W"), ("dgrad", "dY", "W"), ("wgrad", "dY", "X")):
        note("gemm bf16 out %s %dx%dx%d b%d" % (op, T, K, N, block))
        C = fq.fp4q_gemm(op, q[a], q[b], out_dtype=torch.bfloat16)
        assert C.dtype == torch.bfloat16
        torch.cuda.synchronize()
        ref, bound = orc.gemm(op, d[a], d[b])
        check_bf16(C, ref, bound, "%s b%d" % (op, block))
        # the bf16 result is the rounding of the fp32 one: equal, or one bf16 ulp apart
        # where the two accumulations straddle a rounding boundary
        C32 = fq.fp4q_gemm(op, q[a], q[b])
        diff = (C.float() - C32.to(torch.bfloat16).float()).abs()
        ulp = C32.abs().clamp_min(1e-30) * 2.0 ** -7
        assert bool((diff <= ulp).all())


def test_bf16_output_strided_c():
    L = wl.linear_layer("tiny:bf16strided", 256, 256, 160, 5)
    qx = fq.fp4q_quant2d(to_dev(L.X), seed=0, stream_id=1)
    qw = fq.fp4q_quant2d(to_dev(L.W), seed=0, stream_id=2)
    big = torch.full((256, 200), 7.0, dtype=torch.bfloat16, device="cuda")
    note("gemm bf16 out strided")
    fq.fp4q_gemm("fwd", qx, qw, c=big[:, 8:168])
    torch.cuda.synchronize()
    assert bool((big[:, :8] == 7.0).all()) and bool((big[:, 168:] == 7.0).all())
    c, _, s = orc.quant2d(L.X, seed=0, stream=1)
    xd = orc.dequant_fp4(c, s, 256, 256)
    c, _, s = orc.quant2d(L.W, seed=0, stream=2)
    wd = orc.dequant_fp4(c, s, 160, 256)
    ref, bound = orc.gemm(orc.OP_FWD, xd, wd)
    check_bf16(big[:, 8:168], ref, bound, "strided")


def test_bf16_output_mxfp8_batched():
    rng = np.random.default_rng(4)
    B, S, D = 3, 288, 128
    qs = rng.standard_normal((B * S, D)).astype(np.float32)
    ks = rng.standard_normal((B * S, D)).astype(np.float32)
    def batched(t):
        """The [B*S x D] quantization viewed as B stacked [S x D] matrices."""
        return fq.QTensor(t.fmt, S, D, t.codes, t.scales, batch=B, bstride=S * t.codes.stride(0),
                          bstride_s=S * t.scales.stride(0))

    qq = batched(fq.fp4q_quant1d_mxfp8(to_dev(qs)))
    qk = batched(fq.fp4q_quant1d_mxfp8(to_dev(ks)))
    note("gemm bf16 out mxfp8 batched")
    C = fq.fp4q_gemm("fwd", qq, qk, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    cq, sq = orc.quant1d_mxfp8(qs)
    ck, sk = orc.quant1d_mxfp8(ks)
    dq = orc.dequant_mxfp8(cq, sq, B * S, D)
    dk = orc.dequant_mxfp8(ck, sk, B * S, D)
    for i in range(B):
        ref, bound = orc.gemm(orc.OP_FWD, dq[i * S:(i + 1) * S], dk[i * S:(i + 1) * S])
        check_bf16(C[i], ref, bound, "S batch %d" % i)


def test_7b_qkv_bf16_output_sampled():
    L = wl.layer_7b(0)
    q, d = {}, {}
    for nm in ("X", "W", "dY"):
        t = getattr(L, nm)
        q[nm] = fq.fp4q_quant2d(to_dev(t), seed=0, stream_id=STREAMS[nm])
        c, _, s = orc.quant2d(t, seed=0, stream=STREAMS[nm])
        d[nm] = orc.dequant_fp4(c, s, *t.shape)
    rng = np.random.default_rng(6)
    for op, a, b in (("fwd", "X", "W"), ("dgrad", "dY", "W"), ("wgrad", "dY", "X")):
        note("gemm bf16 out 7B %s" % op)
        C = fq.fp4q_gemm(op, q[a], q[b], out_dtype=torch.bfloat16)
        m, n = C.shape
        ci, cj = rng.integers(0, m, 3000), rng.integers(0, n, 3000)
        got = C[torch.from_numpy(ci).cuda(), torch.from_numpy(cj).cuda()]
        del C
        ref, bound = orc.gemm_sampled(op, d[a], d[b], ci, cj)
        check_bf16(got, ref, bound, "7B %s" % op)


@pytest.mark.parametrize("device_offsets", [False, True])
def test_bf16_output_grouped(device_offsets):
    """Grouped expert products with bf16 C (host and device offsets), per
    expert against the oracle; empty experts give a zero dW."""
    rng = np.random.default_rng(21)
    counts = [40, 0, 96, 7, 64, 33]
    E, H, F = len(counts), 96, 64
    off = np.concatenate([[0], np.cumsum([(c + 31) // 32 * 32 for c in counts])]).astype(np.int64)
    rows = int(off[-1])
    X = np.zeros((rows, H), np.float32)
    dY = np.zeros((rows, F), np.float32)
    for e, c in enumerate(counts):
        X[off[e]:off[e] + c] = rng.standard_normal((c, H))
        dY[off[e]:off[e] + c] = rng.standard_normal((c, F)) * 1e-3
    W = (rng.standard_normal((E * F, H)) * 0.02).astype(np.float32)
    ts = {"X": X, "W": W, "dY": dY}
    q = {nm: fq.fp4q_quant2d(to_dev(t), seed=0, stream_id=STREAMS[nm]) for nm, t in ts.items()}
    d = {}
    for nm, t in ts.items():
        c, _, s = orc.quant2d(t, seed=0, stream=STREAMS[nm])
        d[nm] = orc.dequant_fp4(c, s, *t.shape)
    groups = torch.from_numpy(off).cuda() if device_offsets else off.tolist()
    note("grouped bf16 out, device offsets %s" % device_offsets)
    Y = fq.fp4q_gemm("fwd", q["X"], q["W"], groups=groups, out_dtype=torch.bfloat16)
    dX = fq.fp4q_gemm("dgrad", q["dY"], q["W"], groups=groups, out_dtype=torch.bfloat16)
    dW = fq.fp4q_gemm("wgrad", q["dY"], q["X"], groups=groups, out_dtype=torch.bfloat16,
                      max_group_rows=128)
    torch.cuda.synchronize()
    Y, dX, dW = (t.float().cpu().numpy().astype(np.float64) for t in (Y, dX, dW))
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            assert not dW[e * F:(e + 1) * F].any()
            continue
        We = d["W"][e * F:(e + 1) * F]
        ref, bound = orc.gemm(orc.OP_FWD, d["X"][r0:r1], We)
        check_bf16(Y[r0:r1], ref, bound, "fwd e%d" % e)
        ref, bound = orc.gemm(orc.OP_DGRAD, d["dY"][r0:r1], We)
        check_bf16(dX[r0:r1], ref, bound, "dgrad e%d" % e)
        ref, bound = orc.gemm(orc.OP_WGRAD, d["dY"][r0:r1], d["X"][r0:r1])
        check_bf16(dW[e * F:(e + 1) * F], ref, bound, "wgrad e%d" % e)
