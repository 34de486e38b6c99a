"""GPU parity of the grouped (expert) MXFP4 GEMMs with the oracle: per-expert
2D quantization of the gathered token buffer (one quant2d call, 32-aligned
expert segments) and grouped fwd / dgrad / wgrad."""
import numpy as np
import pytest
import torch

import oracle as orc
import fp4_microscaling_quantization_quant2d_amd as fq
from fp4_microscaling_quantization_quant2d_amd import workloads as wl
from gpu_util import assert_planes_equal, check_gemm_tol, note, to_dev

pytestmark = pytest.mark.gpu


def _band(x, r0, r1, stream):
    """Oracle dequantization of rows [r0, r1) (32-aligned) of x's 2D quantization."""
    if r1 <= r0:
        return np.zeros((0, x.shape[1]))
    c, _, s = orc.quant2d(x, orc.ROUND_SR, seed=0, stream=stream, tile_rows=(r0 // 32, (r1 + 31) // 32))
    return orc.dequant_fp4(np.ascontiguousarray(c[r0:r1]), np.ascontiguousarray(s[r0 // 32:(r1 + 31) // 32]),
                           r1 - r0, x.shape[1])


def _small_moe():
    rng = np.random.default_rng(12)
    counts = [40, 0, 96, 7, 64, 33]          # an empty expert and ragged ones
    E, H, F = len(counts), 96, 64
    padded = [(c + 31) // 32 * 32 for c in counts]
    off = np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)
    rows = int(off[-1])
    X = np.zeros((rows, H), np.float32)
    dY = np.zeros((rows, F), np.float32)
    for e, c in enumerate(counts):
        X[off[e]:off[e] + c] = rng.standard_normal((c, H))
        dY[off[e]:off[e] + c] = rng.standard_normal((c, F)) * 1e-3
    W = (rng.standard_normal((E * F, H)) * 0.02).astype(np.float32)
    bf = wl.f32_to_bf16_bits
    return E, H, F, off, bf(X), bf(W), bf(dY)


def test_grouped_small_all_ops():
    E, H, F, off, X, W, dY = _small_moe()
    g = {nm: fq.fp4q_quant2d(to_dev(t), seed=0, stream_id=i + 1) for i, (nm, t) in
         enumerate((("X", X), ("W", W), ("dY", dY)))}
    o = {nm: orc.quant2d(t, orc.ROUND_SR, seed=0, stream=i + 1) for i, (nm, t) in
         enumerate((("X", X), ("W", W), ("dY", dY)))}
    for nm in g:
        assert_planes_equal(g[nm], o[nm], "moe-small " + nm)
    Xd = orc.dequant_fp4(o["X"][0], o["X"][2], *X.shape)
    Wd = orc.dequant_fp4(o["W"][0], o["W"][2], *W.shape)
    dYd = orc.dequant_fp4(o["dY"][0], o["dY"][2], *dY.shape)
    offs = off.tolist()
    note("moe small grouped fwd/dgrad/wgrad")
    Y = fq.fp4q_gemm("fwd", g["X"], g["W"], groups=offs).cpu().numpy()
    dX = fq.fp4q_gemm("dgrad", g["dY"], g["W"], groups=offs).cpu().numpy()
    dW = fq.fp4q_gemm("wgrad", g["dY"], g["X"], groups=offs).cpu().numpy()
    assert Y.shape == (off[-1], F) and dX.shape == (off[-1], H) and dW.shape == (E * F, H)
    for e in range(E):
        r0, r1 = offs[e], offs[e + 1]
        We = Wd[e * F:(e + 1) * F]
        if r1 > r0:
            ref, b = orc.gemm("fwd", Xd[r0:r1], We)
            check_gemm_tol(Y[r0:r1], ref, b, "fwd expert %d" % e)
            ref, b = orc.gemm("dgrad", dYd[r0:r1], We)
            check_gemm_tol(dX[r0:r1], ref, b, "dgrad expert %d" % e)
            ref, b = orc.gemm("wgrad", dYd[r0:r1], Xd[r0:r1])
            check_gemm_tol(dW[e * F:(e + 1) * F], ref, b, "wgrad expert %d" % e)
        else:
            assert np.all(dW[e * F:(e + 1) * F] == 0)


def test_moe_config_sampled_experts():
    """30B-class MoE layer (8192 tokens, hidden 2048, 128 experts of 768,
    top-8): every quantized plane of X, W_up, dY, A, W_down and dY_down
    bit-exact against the oracle, and the up and down projections' grouped
    fwd/dgrad/wgrad checked on a sample of experts (first, last, largest,
    smallest, random)."""
    m = wl.config_moe()
    offs = m.row_off.tolist()
    E, H, F = m.E, m.H, m.F
    rng = np.random.default_rng(5)
    sizes = np.diff(m.row_off)
    experts = sorted({0, E - 1, int(np.argmax(sizes)), int(np.argmin(sizes))} |
                     set(rng.integers(0, E, 3).tolist()))
    for name, X, W, dY, n_out, n_in in (("up", m.X, m.W_up, m.dY, F, H),
                                        ("down", m.A, m.W_down, m.dY_down, H, F)):
        note("moe %s quant" % name)
        g = {"X": fq.fp4q_quant2d(to_dev(X), seed=0, stream_id=1),
             "W": fq.fp4q_quant2d(to_dev(W), seed=0, stream_id=2),
             "dY": fq.fp4q_quant2d(to_dev(dY), seed=0, stream_id=3)}
        # every plane of the config's quantized tensors, bit for bit
        for nm, t, sid in (("X", X, 1), ("W", W, 2), ("dY", dY, 3)):
            note("moe %s %s planes vs the oracle (%d x %d)" % (name, nm, t.shape[0], t.shape[1]))
            assert_planes_equal(g[nm], orc.quant2d(t, orc.ROUND_SR, seed=0, stream=sid),
                                "moe %s %s" % (name, nm))
        note("moe %s grouped gemms" % name)
        Y = fq.fp4q_gemm("fwd", g["X"], g["W"], groups=offs)
        dX = fq.fp4q_gemm("dgrad", g["dY"], g["W"], groups=offs)
        dW = fq.fp4q_gemm("wgrad", g["dY"], g["X"], groups=offs)
        torch.cuda.synchronize()
        for e in experts:
            r0, r1 = offs[e], offs[e + 1]
            Xe = _band(X, r0, r1, 1)
            dYe = _band(dY, r0, r1, 3)
            We = _band(W, e * n_out, (e + 1) * n_out, 2)
            ci = rng.integers(0, max(1, r1 - r0), 300)
            for op, got, a, b, (mm, nn), base in (
                    ("fwd", Y, Xe, We, (r1 - r0, n_out), r0),
                    ("dgrad", dX, dYe, We, (r1 - r0, n_in), r0),
                    ("wgrad", dW, dYe, Xe, (n_out, n_in), e * n_out)):
                if mm == 0:
                    continue
                i = rng.integers(0, mm, 400)
                j = rng.integers(0, nn, 400)
                ref, bd = orc.gemm_sampled(op, a, b, i, j)
                gv = got[torch.from_numpy(i + base).cuda(), torch.from_numpy(j).cuda()].cpu().numpy()
                check_gemm_tol(gv, ref, bd, "moe %s %s expert %d" % (name, op, e))


def test_grouped_every_tail_block_count():
    """Experts whose last row tile holds 1 to 8 valid 32-row blocks (some of
    them ragged inside the last block), over one, two and three row tiles:
    grouped fwd and dgrad (whose waves skip the MFMAs of blocks past an
    expert's last row) and wgrad within the parity bound of the oracle, and
    the device-offset launch identical to the host-offset one."""
    rng = np.random.default_rng(31)
    counts = [27, 64, 96, 123, 160, 192, 224, 256, 300, 480, 545, 767]
    E, H, F = len(counts), 160, 128
    padded = [(c + 31) // 32 * 32 for c in counts]
    off = np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)
    rows = int(off[-1])
    X = np.zeros((rows, H), np.float32)
    dY = np.zeros((rows, F), np.float32)
    for e, c in enumerate(counts):
        X[off[e]:off[e] + c] = rng.standard_normal((c, H))
        dY[off[e]:off[e] + c] = rng.standard_normal((c, F)) * 1e-3
    W = (rng.standard_normal((E * F, H)) * 0.02).astype(np.float32)
    bf = wl.f32_to_bf16_bits
    X, W, dY = bf(X), bf(W), bf(dY)
    g = {nm: fq.fp4q_quant2d(to_dev(t), seed=0, stream_id=i + 1) for i, (nm, t) in
         enumerate((("X", X), ("W", W), ("dY", dY)))}
    o = {nm: orc.quant2d(t, orc.ROUND_SR, seed=0, stream=i + 1) for i, (nm, t) in
         enumerate((("X", X), ("W", W), ("dY", dY)))}
    Xd = orc.dequant_fp4(o["X"][0], o["X"][2], *X.shape)
    Wd = orc.dequant_fp4(o["W"][0], o["W"][2], *W.shape)
    dYd = orc.dequant_fp4(o["dY"][0], o["dY"][2], *dY.shape)
    offs = off.tolist()
    note("moe tail block counts: host offsets")
    out = {op: fq.fp4q_gemm(op, g[a], g[b], groups=offs)
           for op, a, b in (("fwd", "X", "W"), ("dgrad", "dY", "W"), ("wgrad", "dY", "X"))}
    note("moe tail block counts: device offsets")
    dev = {op: fq.fp4q_gemm(op, g[a], g[b], groups=torch.from_numpy(off).cuda(), max_group_rows=max(padded))
           for op, a, b in (("fwd", "X", "W"), ("dgrad", "dY", "W"), ("wgrad", "dY", "X"))}
    torch.cuda.synchronize()
    for op in out:
        assert torch.equal(out[op], dev[op]), op
    Y, dX, dW = (out[k].cpu().numpy() for k in ("fwd", "dgrad", "wgrad"))
    for e in range(E):
        r0, r1 = offs[e], offs[e + 1]
        We = Wd[e * F:(e + 1) * F]
        ref, b = orc.gemm("fwd", Xd[r0:r1], We)
        check_gemm_tol(Y[r0:r1], ref, b, "fwd expert %d (%d rows)" % (e, counts[e]))
        ref, b = orc.gemm("dgrad", dYd[r0:r1], We)
        check_gemm_tol(dX[r0:r1], ref, b, "dgrad expert %d (%d rows)" % (e, counts[e]))
        ref, b = orc.gemm("wgrad", dYd[r0:r1], Xd[r0:r1])
        check_gemm_tol(dW[e * F:(e + 1) * F], ref, b, "wgrad expert %d (%d rows)" % (e, counts[e]))


@pytest.mark.parametrize("case", range(6))
def test_grouped_random_routings(case):
    """Seeded random expert layouts (empty, ragged and multi-tile experts,
    hidden and expert widths of several 32-multiples): grouped fwd, dgrad and
    wgrad within the parity bound of the oracle for every expert, host and
    device offsets identical."""
    rng = np.random.default_rng(1000 + case)
    E = int(rng.integers(2, 9))
    H = 32 * int(rng.integers(1, 12))
    F = 32 * int(rng.integers(1, 12))
    counts = [int(c) for c in rng.integers(0, 700, size=E)]
    counts[int(rng.integers(0, E))] = 0
    padded = [(c + 31) // 32 * 32 for c in counts]
    off = np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)
    rows = max(int(off[-1]), 32)
    X = np.zeros((rows, H), np.float32)
    dY = np.zeros((rows, F), np.float32)
    for e, c in enumerate(counts):
        X[off[e]:off[e] + c] = rng.standard_normal((c, H))
        dY[off[e]:off[e] + c] = rng.standard_normal((c, F)) * 1e-3
    W = (rng.standard_normal((E * F, H)) * 0.02).astype(np.float32)
    bf = wl.f32_to_bf16_bits
    X, W, dY = bf(X), bf(W), bf(dY)
    g = {nm: fq.fp4q_quant2d(to_dev(t), seed=case, stream_id=i + 1) for i, (nm, t) in
         enumerate((("X", X), ("W", W), ("dY", dY)))}
    o = {nm: orc.quant2d(t, orc.ROUND_SR, seed=case, stream=i + 1) for i, (nm, t) in
         enumerate((("X", X), ("W", W), ("dY", dY)))}
    Xd = orc.dequant_fp4(o["X"][0], o["X"][2], *X.shape)
    Wd = orc.dequant_fp4(o["W"][0], o["W"][2], *W.shape)
    dYd = orc.dequant_fp4(o["dY"][0], o["dY"][2], *dY.shape)
    offs = off.tolist()
    note("moe random routing %d: E=%d H=%d F=%d counts=%s" % (case, E, H, F, counts))
    ops = (("fwd", "X", "W"), ("dgrad", "dY", "W"), ("wgrad", "dY", "X"))
    out = {op: fq.fp4q_gemm(op, g[a], g[b], groups=offs) for op, a, b in ops}
    dev = {op: fq.fp4q_gemm(op, g[a], g[b], groups=torch.from_numpy(off).cuda(),
                            max_group_rows=max(max(padded), 32)) for op, a, b in ops}
    torch.cuda.synchronize()
    for op in out:
        assert torch.equal(out[op], dev[op]), op
    Y, dX, dW = (out[k].cpu().numpy() for k in ("fwd", "dgrad", "wgrad"))
    for e in range(E):
        r0, r1 = offs[e], offs[e + 1]
        if r1 == r0:
            assert not dW[e * F:(e + 1) * F].any()
            continue
        We = Wd[e * F:(e + 1) * F]
        ref, b = orc.gemm("fwd", Xd[r0:r1], We)
        check_gemm_tol(Y[r0:r1], ref, b, "case %d fwd expert %d" % (case, e))
        ref, b = orc.gemm("dgrad", dYd[r0:r1], We)
        check_gemm_tol(dX[r0:r1], ref, b, "case %d dgrad expert %d" % (case, e))
        ref, b = orc.gemm("wgrad", dYd[r0:r1], Xd[r0:r1])
        check_gemm_tol(dW[e * F:(e + 1) * F], ref, b, "case %d wgrad expert %d" % (case, e))
