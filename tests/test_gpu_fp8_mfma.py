"""Why the MXFP8 products ("Stable FP4 Training via Transposition-Invariant
Block Quantization", Sec. 3.2 "MXFP8 Attention": S = Q K^T on MXFP8 Q and
K) do not run on the block-scaled FP8 MFMA: that instruction rounds inside
its dot product, past the 1e-5 * sum|a||b| bound every product of this
library meets, while the library's route (each E4M3 code times its E8M0
scale converted exactly to bf16, then the bf16 MFMA with fp32 sums) stays
inside it on the same operands.

fp4q_probe_mfma_fp8 runs the FP8 instruction on one 32x32x64 block.  The
test checks the probe's lane layout first (its result is close to the exact
product everywhere), then that some element misses the bound, and that
fp4q_gemm's MXFP8 product of the same bytes meets it.  If a future chip's
FP8 MFMA met the bound, the second check fails and says so."""
import numpy as np
import pytest
import torch

import fp4_microscaling_quantization_quant2d_amd as fq
from gpu_util import check_gemm_tol

pytestmark = pytest.mark.gpu


def _e4m3_bytes(rng, shape):
    """Random finite E4M3FN bytes over the whole range (0x7F / 0xFF are NaN)."""
    b = rng.integers(0, 256, shape, dtype=np.uint8)
    nan = (b & 0x7F) == 0x7F
    b[nan] ^= 0x01
    return b


def _decode(codes, scales):
    """Exact fp64 values: E4M3 (torch's decode) times 2^(byte - 127) per
    32-value block of each row."""
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    s = np.exp2(scales.astype(np.float64) - 127.0)
    return v * np.repeat(s, 32, axis=1)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fp8_mfma_rounds_beyond_the_bound_library_route_does_not(seed):
    rng = np.random.default_rng(seed)
    a, b = _e4m3_bytes(rng, (32, 64)), _e4m3_bytes(rng, (32, 64))
    sa = rng.integers(122, 133, (32, 2)).astype(np.uint8)
    sb = rng.integers(122, 133, (32, 2)).astype(np.uint8)
    A, B = _decode(a, sa), _decode(b, sb)
    exact = A @ B.T
    bound = np.abs(A) @ np.abs(B).T

    dev = [torch.from_numpy(x.copy()).cuda() for x in (a, b, sa, sb)]
    c = fq.fp4q_probe_mfma_fp8(*dev).cpu().numpy().astype(np.float64)
    rel = np.abs(c - exact) / bound
    # the lane layout is right: the instruction's result is close everywhere
    assert np.median(rel) < 1e-3 and rel.max() < 1e-2, "probe layout: median %.3g max %.3g" % (
        np.median(rel), rel.max())
    # and its internal rounding misses the library's bound somewhere
    assert rel.max() > 1e-5, "the FP8 MFMA met 1e-5 * sum|a||b| (max %.3g)" % rel.max()

    # the library's MXFP8 product of the same bytes meets the bound
    qa, qb = fq.alloc_mxfp8(32, 64), fq.alloc_mxfp8(32, 64)
    qa.codes.copy_(dev[0]); qa.scales.copy_(dev[2])
    qb.codes.copy_(dev[1]); qb.scales.copy_(dev[3])
    S = fq.fp4q_gemm("fwd", qa, qb)
    torch.cuda.synchronize()
    check_gemm_tol(S.cpu().numpy(), exact, bound, "MXFP8 S = Q K^T on the probe's operands")
