"""GPU parity of fp4q_quant2d_batch: each item of a batch launch is
quantized exactly as the oracle quantizes it alone (row and transposed
planes and scale bytes, bit for bit), for mixed shapes, both dtypes and
rounding modes, items without a transposed plane, and the largest batch."""
import numpy as np
import pytest
import torch

import oracle as orc
import fp4_microscaling_quantization_quant2d_amd as fq
from fp4_microscaling_quantization_quant2d_amd.workloads import f32_to_bf16_bits
from gpu_util import assert_planes_equal, note, to_dev

pytestmark = pytest.mark.gpu


def _inputs(shapes, seed, dtype):
    """Host inputs: float32, or bf16 as uint16 bit patterns (what to_dev and the oracle take)."""
    rng = np.random.default_rng(seed)
    xs = []
    for r, c in shapes:
        x = (rng.standard_normal((r, c)) * np.exp(rng.standard_normal((r, 1)))).astype(np.float32)
        xs.append(f32_to_bf16_bits(x) if dtype == "bf16" else x)
    return xs


def _check_batch(shapes, dtype, mode, seed, transposed=None):
    xs = _inputs(shapes, len(shapes) * 31 + seed, dtype)
    devs = [to_dev(x) for x in xs]
    outs = [fq.alloc_fp4(r, c, transposed=True if transposed is None else transposed[k])
            for k, (r, c) in enumerate(shapes)]
    note("quant2d_batch %s %s %s %d items" % (dtype, mode, shapes[:3], len(shapes)))
    fq.fp4q_quant2d_batch([(d, o, 100 + k) for k, (d, o) in enumerate(zip(devs, outs))],
                          round_mode=mode, seed=seed)
    torch.cuda.synchronize()
    rm = orc.ROUND_SR if mode == "sr" else orc.ROUND_RNE
    for k, o in enumerate(outs):
        ref = orc.quant2d(xs[k], rm, seed=seed, stream=100 + k)
        assert_planes_equal(o, ref, "batch item %d %s" % (k, shapes[k]))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", ["sr", "rne"])
def test_mixed_shapes(dtype, mode):
    _check_batch([(100, 200), (33, 65), (256, 256), (1, 1), (300, 129)], dtype, mode, seed=3)


def test_largest_batch_and_large_items():
    shapes = [(1024, 768), (7, 45), (2048, 96), (129, 257), (512, 512), (64, 2048), (31, 31), (640, 384)]
    assert len(shapes) == fq.QUANT2D_BATCH_MAX
    _check_batch(shapes, "bf16", "sr", seed=11)


def test_rows_only_items():
    _check_batch([(200, 100), (96, 160), (45, 7)], "bf16", "sr", seed=5, transposed=[False, True, False])


def test_batch_equals_single_calls():
    """The same items through fp4q_quant2d one by one give the same bytes."""
    shapes = [(4096, 1024), (1000, 3000), (64, 64)]
    xs = _inputs(shapes, 77, "bf16")
    devs = [to_dev(x) for x in xs]
    outs = fq.fp4q_quant2d_batch([(d, None, 7 + k) for k, d in enumerate(devs)], seed=21)
    for k, d in enumerate(devs):
        single = fq.fp4q_quant2d(d, seed=21, stream_id=7 + k)
        torch.cuda.synchronize()
        for a, b in ((outs[k].codes, single.codes), (outs[k].codes_t, single.codes_t),
                     (outs[k].scales, single.scales)):
            assert torch.equal(a, b), "item %d" % k


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unaligned_item_runs_the_whole_batch_unaligned(dtype):
    """One item with a leading dimension that breaks 16-byte rows sends every
    item of the launch through the element-wise load path; results stay exact."""
    shapes = [(200, 96), (130, 70), (64, 256)]
    xs = _inputs(shapes, 19, dtype)
    devs = []
    for k, x in enumerate(xs):
        d = to_dev(x)
        if k == 1:   # ldx = cols + 1 elements
            big = torch.zeros((d.shape[0], d.shape[1] + 1), dtype=d.dtype, device=d.device)
            big[:, : d.shape[1]] = d
            d = big[:, : d.shape[1]]
        devs.append(d)
    assert devs[1].stride(0) == shapes[1][1] + 1
    note("quant2d_batch unaligned %s" % dtype)
    outs = fq.fp4q_quant2d_batch([(d, None, 40 + k) for k, d in enumerate(devs)], seed=9)
    torch.cuda.synchronize()
    for k, o in enumerate(outs):
        ref = orc.quant2d(xs[k], orc.ROUND_SR, seed=9, stream=40 + k)
        assert_planes_equal(o, ref, "unaligned batch item %d" % k)
