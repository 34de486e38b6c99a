"""The allocation-free attention backward (fp4q_attn_bwd_noalloc), called
through the C ABI: on two calls in a row, the second with a smaller input,
its dQ, dK and dV equal those of fp4q_attn_bwd with a caller workspace bit
for bit (the same kernels; only where D is kept differs), and a size beyond
the static scratch is refused before anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

import fp4_microscaling_quantization_quant2d_amd as fq
from fp4_microscaling_quantization_quant2d_amd import workloads as wl
from gpu_util import note, to_dev

pytestmark = pytest.mark.gpu


def _case(bh, L, seed, causal):
    rng = np.random.default_rng(seed)
    mk = lambda s: to_dev(wl.f32_to_bf16_bits((rng.standard_normal((bh * L, 128)) * s).astype(np.float32)))
    q, k, v, g = mk(1.0), mk(1.0), mk(1.0), mk(0.1)
    qq, qk = fq.fp4q_quant1d_mxfp8(q), fq.fp4q_quant1d_mxfp8(k)
    O, lse = fq.fp4q_attn_fwd(qq, qk, v, bh, L, causal=causal)
    return qq, qk, v, g, O, lse


def test_noalloc_backward_matches_workspace_entry():
    L = fq.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for bh, n, causal in ((3, 300, True), (2, 100, False)):      # the second call smaller
        note("attn bwd noalloc bh=%d L=%d causal=%d" % (bh, n, causal))
        qq, qk, v, g, O, lse = _case(bh, n, bh * 1000 + n, causal)
        ref = fq.fp4q_attn_bwd(qq, qk, v, O, lse, g, bh, n, causal=causal)
        got = [torch.full((bh * n, 128), float("nan"), device="cuda") for _ in range(3)]
        dq, dk = qq.desc(), qk.desc()
        P = lambda t: ctypes.c_void_p(t.data_ptr())
        rc = L.fp4q_attn_bwd_noalloc(ctypes.byref(dq), ctypes.byref(dk), P(v), v.stride(0), P(O), O.stride(0),
                                     fq.DT_BF16, P(lse), P(g), g.stride(0), P(got[0]), P(got[1]), P(got[2]),
                                     got[0].stride(0), bh, n, ctypes.c_float(128 ** -0.5), 1 if causal else 0,
                                     stream)
        assert rc == 0, L.fp4q_last_error().decode()
        torch.cuda.synchronize()
        for a, b, what in zip(got, ref, ("dQ", "dK", "dV")):
            assert torch.equal(a, b), "%s differs from the workspace entry point" % what
    rc = L.fp4q_attn_bwd_noalloc(ctypes.byref(dq), ctypes.byref(dk), P(v), 128, P(O), 128, fq.DT_BF16, P(lse), P(g),
                                 128, P(got[0]), P(got[1]), P(got[2]), 128, 1, (1 << 20) + 1,
                                 ctypes.c_float(0.1), 1, stream)
    assert rc == -1 and "static scratch" in L.fp4q_last_error().decode()
