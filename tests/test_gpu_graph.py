"""The hot path captured in a HIP graph: replays, with eager work and
synchronizations between them, reproduce the eager results bit for bit
(quantizer planes and GEMM outputs), for the launches captured on one stream,
for the quantizers on a second stream with each GEMM waiting on events for
the operands it reads, and for the bench step's schedule (X and W in one
batch launch, wgrad on a second stream beside dgrad)."""
import numpy as np
import pytest
import torch

import fp4_microscaling_quantization_quant2d_amd as fq
from fp4_microscaling_quantization_quant2d_amd import workloads as wl
from gpu_util import note, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("streams", [1, 2, 3])
def test_graph_replays_match_eager(streams):
    L = wl.linear_layer("tiny:graph", 320, 448, 288, 3)
    x, w, dy = to_dev(L.X), to_dev(L.W), to_dev(L.dY)
    q = {nm: fq.alloc_fp4(*t.shape) for nm, t in (("X", x), ("W", w), ("dY", dy))}
    C = {"fwd": torch.empty((320, 288), device="cuda"), "dgrad": torch.empty((320, 448), device="cuda"),
         "wgrad": torch.empty((288, 448), device="cuda")}

    def seq():
        fq.fp4q_quant2d(x, q["X"], seed=11, stream_id=1)
        fq.fp4q_quant2d(w, q["W"], seed=11, stream_id=2)
        fq.fp4q_quant2d(dy, q["dY"], seed=11, stream_id=3)
        fq.fp4q_gemm("fwd", q["X"], q["W"], C["fwd"])
        fq.fp4q_gemm("dgrad", q["dY"], q["W"], C["dgrad"])
        fq.fp4q_gemm("wgrad", q["dY"], q["X"], C["wgrad"])

    side = torch.cuda.Stream()

    def two_streams():
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        done = {}
        with torch.cuda.stream(side):
            for nm, t, sid in (("X", x, 1), ("W", w, 2), ("dY", dy, 3)):
                fq.fp4q_quant2d(t, q[nm], seed=11, stream_id=sid)
                done[nm] = torch.cuda.Event()
                done[nm].record(side)
        main.wait_event(done["X"])
        main.wait_event(done["W"])
        fq.fp4q_gemm("fwd", q["X"], q["W"], C["fwd"])
        main.wait_event(done["dY"])
        fq.fp4q_gemm("dgrad", q["dY"], q["W"], C["dgrad"])
        fq.fp4q_gemm("wgrad", q["dY"], q["X"], C["wgrad"])
        main.wait_stream(side)

    def wgrad_beside():
        # the bench step's schedule: X and W in one batch launch, wgrad on a
        # second stream beside dgrad
        main = torch.cuda.current_stream()
        fq.fp4q_quant2d_batch([(x, q["X"], 1), (w, q["W"], 2)], seed=11)
        fq.fp4q_gemm("fwd", q["X"], q["W"], C["fwd"])
        fq.fp4q_quant2d(dy, q["dY"], seed=11, stream_id=3)
        side.wait_stream(main)
        fq.fp4q_gemm("dgrad", q["dY"], q["W"], C["dgrad"])
        with torch.cuda.stream(side):
            fq.fp4q_gemm("wgrad", q["dY"], q["X"], C["wgrad"])
        main.wait_stream(side)

    captured = {1: seq, 2: two_streams, 3: wgrad_beside}[streams]

    def snapshot():
        torch.cuda.synchronize()
        return {**{nm: (t.codes.clone(), t.codes_t.clone(), t.scales.clone()) for nm, t in q.items()},
                **{op: c.clone() for op, c in C.items()}}

    note("graph: eager reference")
    seq()
    ref = snapshot()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        captured()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    note("graph: capture (schedule %d)" % streams)
    with torch.cuda.graph(g):
        captured()
    other = to_dev(wl.f32_to_bf16_bits(np.random.default_rng(1).standard_normal((256, 256)).astype(np.float32)))
    for rep in range(4):
        # clobber the outputs eagerly, run unrelated eager work, then replay
        for t in q.values():
            t.codes.fill_(0x55)
            t.codes_t.fill_(0x55)
            t.scales.fill_(3)
        for c in C.values():
            c.fill_(-1.0)
        fq.fp4q_quant2d(other, seed=rep)
        torch.cuda.synchronize()
        note("graph: replay %d" % rep)
        g.replay()
        got = snapshot()
        for k, v in ref.items():
            if isinstance(v, tuple):
                for a, b in zip(v, got[k]):
                    assert torch.equal(a, b), "replay %d: %s planes differ" % (rep, k)
            else:
                assert torch.equal(v, got[k]), "replay %d: %s differs" % (rep, k)


def test_device_seed_draws_fresh_bits_per_replay():
    """A quantizer captured with a device-resident seed (fp4q_quant2d_batch_ex)
    reads the seed when the replay runs: with the seed changed between
    replays, each replay's planes equal the oracle's for the host seed plus
    that replay's device seed, and consecutive replays differ."""
    import oracle as orc
    from gpu_util import assert_planes_equal
    L = wl.linear_layer("tiny:devseed", 200, 320, 96, 4)
    x, w = to_dev(L.X), to_dev(L.W)
    qx, qw = fq.alloc_fp4(*x.shape), fq.alloc_fp4(*w.shape)
    seed_dev = torch.zeros(1, dtype=torch.int64, device="cuda")

    def seq():
        fq.fp4q_quant2d_batch([(x, qx, 5), (w, qw, 6)], seed=100, seed_dev=seed_dev)

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        seq()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq()
    prev = None
    for dseed in (7, 8, (1 << 40) + 3, -1):
        note("graph device seed %d" % dseed)
        seed_dev.fill_(dseed)
        g.replay()
        torch.cuda.synchronize()
        key = (100 + dseed) & ((1 << 64) - 1)
        assert_planes_equal(qx, orc.quant2d(L.X, orc.ROUND_SR, seed=key, stream=5), "X seed %d" % dseed)
        assert_planes_equal(qw, orc.quant2d(L.W, orc.ROUND_SR, seed=key, stream=6), "W seed %d" % dseed)
        cur = qx.codes.clone()
        if prev is not None:
            assert not torch.equal(cur, prev)
        prev = cur


def test_bench_graph_advances_device_seed():
    """The bench's captured step (wgrad on a second stream) with its
    quantizers on a device-resident seed that the graph advances at the end
    of every replay: replay r leaves exactly the planes and products of an
    eager step run with host seed 7 + r, and consecutive replays differ."""
    import importlib.util
    import pathlib
    spec = importlib.util.spec_from_file_location("bench_mod", pathlib.Path(__file__).parent.parent / "bench.py")
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    layers = [wl.linear_layer("tiny:seedgraph", 320, 448, 288, 1), wl.linear_layer("tiny:seedgraph", 320, 288, 96, 2)]
    step = bench.Step(layers, torch, fq)
    keys, outs = ("qX", "qW", "qdY"), ("Y", "dX", "dW")

    def snapshot():
        torch.cuda.synchronize()
        snap = {}
        for i, d in enumerate(step.layers):
            for k in keys:
                snap[(i, k)] = (d[k].codes.clone(), d[k].codes_t.clone(), d[k].scales.clone())
            for k in outs:
                snap[(i, k)] = d[k].clone()
        return snap

    refs = []
    for r in range(3):
        step.run(seed=7 + r)
        refs.append(snapshot())
    step.seed_dev = torch.zeros(1, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()

    def captured():
        step.run_two_streams(7, side)
        step.seed_dev.add_(1)

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        captured()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    note("bench graph with device seed: capture")
    with torch.cuda.graph(g):
        captured()
    step.seed_dev.zero_()
    prev = None
    for r in range(3):
        torch.cuda.synchronize()
        note("bench graph with device seed: replay %d" % r)
        g.replay()
        got = snapshot()
        for k, v in refs[r].items():
            if isinstance(v, tuple):
                for a, b in zip(v, got[k]):
                    assert torch.equal(a, b), "replay %d: layer %d %s planes differ" % (r, k[0], k[1])
            else:
                assert torch.equal(v, got[k]), "replay %d: layer %d %s differs" % (r, k[0], k[1])
        if prev is not None:
            assert not torch.equal(prev, got[(0, "qX")][0]), "replay %d drew the same bits as the last" % r
        prev = got[(0, "qX")][0]
    assert int(step.seed_dev.item()) == 3
