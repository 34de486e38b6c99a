"""Grouped (expert) GEMMs with the group offsets in device memory
(FP4Q_GROUPS_DEVICE): results within the parity bound of the oracle on a
small MoE with empty and ragged experts, identical to the host-offset
launch, memory-safe clamping of offsets that break the rules (compared with
the host launch on the clamped offsets), and a HIP graph captured once and
replayed after the routing in the offsets tensor changed."""
import numpy as np
import pytest
import torch

import oracle as orc
import fp4_microscaling_quantization_quant2d_amd as fq
from fp4_microscaling_quantization_quant2d_amd import workloads as wl
from gpu_util import check_gemm_tol, note, to_dev

pytestmark = pytest.mark.gpu

E, H, F = 6, 96, 64


def _moe(counts, seed):
    rng = np.random.default_rng(seed)
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
    return off, bf(X), bf(W), bf(dY)


def _run(q, offs, max_rows):
    return {op: fq.fp4q_gemm(op, q[a], q[b], groups=offs, max_group_rows=max_rows)
            for op, a, b in (("fwd", "X", "W"), ("dgrad", "dY", "W"), ("wgrad", "dY", "X"))}


def test_device_offsets_match_oracle_and_host_launch():
    off, X, W, dY = _moe([40, 0, 96, 7, 64, 33], 12)
    q = {nm: fq.fp4q_quant2d(to_dev(t), seed=0, stream_id=i + 1)
         for i, (nm, t) in enumerate((("X", X), ("W", W), ("dY", dY)))}
    note("moe device offsets")
    dev = _run(q, torch.from_numpy(off).cuda(), 128)
    host = _run(q, off.tolist(), None)
    torch.cuda.synchronize()
    for op in dev:
        assert torch.equal(dev[op], host[op]), op
    o = {nm: orc.quant2d(t, orc.ROUND_SR, seed=0, stream=i + 1)
         for i, (nm, t) in enumerate((("X", X), ("W", W), ("dY", dY)))}
    Xd = orc.dequant_fp4(o["X"][0], o["X"][2], *X.shape)
    Wd = orc.dequant_fp4(o["W"][0], o["W"][2], *W.shape)
    dYd = orc.dequant_fp4(o["dY"][0], o["dY"][2], *dY.shape)
    Y, dX, dW = (dev[k].cpu().numpy() for k in ("fwd", "dgrad", "wgrad"))
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:  # an empty expert: no rows of Y or dX, a zero dW
            assert not dW[e * F:(e + 1) * F].any()
            continue
        We = Wd[e * F:(e + 1) * F]
        ref, bound = orc.gemm(orc.OP_FWD, Xd[r0:r1], We)
        check_gemm_tol(Y[r0:r1], ref, bound, "fwd e%d" % e)
        ref, bound = orc.gemm(orc.OP_DGRAD, dYd[r0:r1], We)
        check_gemm_tol(dX[r0:r1], ref, bound, "dgrad e%d" % e)
        ref, bound = orc.gemm(orc.OP_WGRAD, dYd[r0:r1], Xd[r0:r1])
        check_gemm_tol(dW[e * F:(e + 1) * F], ref, bound, "wgrad e%d" % e)


def _clamped(raw, tok, max_rows):
    """The documented sanitation of device offsets, group by group."""
    out = []
    for g in range(len(raw) - 1):
        a = min(max(raw[g], 0), tok) // 32 * 32
        b = min(max(raw[g + 1], a), tok) // 32 * 32
        out.append((a, b, min(b, a + max_rows)))
    return out


def test_out_of_rule_offsets_are_clamped():
    """Offsets past the tokens, decreasing, negative and unaligned: each
    group computes exactly its clamped range.  Reference: a host launch whose
    group g is that range (the other groups empty or leading rows), compared
    on the output rows only group g claims; rows no group claims keep their
    old values."""
    off, X, W, dY = _moe([64, 32, 96, 32, 64, 32], 5)
    tok = int(off[-1])
    raw = [-50, 70, 40, 200, 10000, 96, 300]
    ranges = _clamped(raw, tok, 64)
    q = {nm: fq.fp4q_quant2d(to_dev(t), seed=0, stream_id=i + 1)
         for i, (nm, t) in enumerate((("X", X), ("W", W), ("dY", dY)))}
    note("moe clamped device offsets")
    sentinel = 12345.0
    Y = torch.full((tok, F), sentinel, device="cuda")
    dX = torch.full((tok, H), sentinel, device="cuda")
    dW = torch.full((E * F, H), sentinel, device="cuda")
    offs = torch.tensor(raw, dtype=torch.int64, device="cuda")
    fq.fp4q_gemm("fwd", q["X"], q["W"], c=Y, groups=offs)
    fq.fp4q_gemm("dgrad", q["dY"], q["W"], c=dX, groups=offs)
    fq.fp4q_gemm("wgrad", q["dY"], q["X"], c=dW, groups=offs, max_group_rows=64)
    torch.cuda.synchronize()
    Yd, dXd, dWd = Y.cpu().numpy(), dX.cpu().numpy(), dW.cpu().numpy()
    claims = np.zeros(tok, int)
    for a, b, _ in ranges:
        claims[a:b] += 1
    for g, (a, b, bw) in enumerate(ranges):
        host_off = [0] + [a] * g + [b] * (E - g)
        Yh = fq.fp4q_gemm("fwd", q["X"], q["W"], groups=host_off).cpu().numpy()
        dXh = fq.fp4q_gemm("dgrad", q["dY"], q["W"], groups=host_off).cpu().numpy()
        dWh = fq.fp4q_gemm("wgrad", q["dY"], q["X"], groups=[0] + [a] * g + [bw] * (E - g)).cpu().numpy()
        rows = np.arange(a, b)[claims[a:b] == 1]
        assert np.array_equal(Yd[rows], Yh[rows]), "fwd group %d" % g
        assert np.array_equal(dXd[rows], dXh[rows]), "dgrad group %d" % g
        assert np.array_equal(dWd[g * F:(g + 1) * F], dWh[g * F:(g + 1) * F]), "wgrad group %d" % g
    unclaimed = claims == 0
    assert (Yd[unclaimed] == sentinel).all() and (dXd[unclaimed] == sentinel).all()


def test_graph_replay_follows_new_routing():
    """Capture the three grouped products once with device offsets; change
    the offsets tensor between replays and compare every replay with eager
    host-offset launches on the routing of that replay."""
    off, X, W, dY = _moe([64, 32, 96, 32, 64, 32], 8)
    tok = int(off[-1])
    q = {nm: fq.fp4q_quant2d(to_dev(t), seed=0, stream_id=i + 1)
         for i, (nm, t) in enumerate((("X", X), ("W", W), ("dY", dY)))}
    offs = torch.tensor(off, dtype=torch.int64, device="cuda")
    C = {"fwd": torch.zeros((tok, F), device="cuda"), "dgrad": torch.zeros((tok, H), device="cuda"),
         "wgrad": torch.zeros((E * F, H), device="cuda")}

    def seq():
        fq.fp4q_gemm("fwd", q["X"], q["W"], c=C["fwd"], groups=offs)
        fq.fp4q_gemm("dgrad", q["dY"], q["W"], c=C["dgrad"], groups=offs)
        fq.fp4q_gemm("wgrad", q["dY"], q["X"], c=C["wgrad"], groups=offs, max_group_rows=tok)

    note("moe graph capture with device offsets")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        seq()  # warm-up outside the capture (LDS limits are raised once per kernel)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        seq()
    rng = np.random.default_rng(3)
    for rep in range(4):
        cuts = np.sort(rng.choice(np.arange(1, tok // 32), E - 1, replace=False)) * 32
        new = np.concatenate([[0], cuts, [tok]]).astype(np.int64)
        offs.copy_(torch.from_numpy(new))
        for c in C.values():
            c.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = _run(q, new.tolist(), None)
        torch.cuda.synchronize()
        for op in C:
            assert torch.equal(C[op], eager[op]), "replay %d %s" % (rep, op)
