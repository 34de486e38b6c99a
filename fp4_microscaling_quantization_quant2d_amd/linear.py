"""A linear layer trained through the library's kernels ("Stable FP4 Training
via Transposition-Invariant Block Quantization", Sec. 3 "Application to
linear layers": Y = X W^T, dX = dY W, dW = dY^T X, all three on quantized
operands, with gradients passed straight through the quantizers).

Forward quantizes X and W (one batch launch when both take 32x32 blocks and
share a dtype) and runs FWD; backward quantizes dY once and runs DGRAD and
WGRAD on the saved quantized X and W -- each tensor is quantized exactly
once, and W's transposed plane serves DGRAD.  Every step runs in the HIP kernels; this
module only orders the calls.  Y and dW are fp32; dX has X's dtype (bf16 X:
the kernel's bf16 output, the fp32 result rounded to nearest even).
"""
import itertools
import weakref

import torch

from . import alloc_fp4, fp4q_gemm, fp4q_quant2d, fp4q_quant2d_batch

__all__ = ["fp4_linear", "FP4Linear"]


class _FP4LinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w, seed, stream_base, act_layout):
        T, K = x.shape
        if act_layout == 32 and x.dtype == w.dtype:  # a batch launch takes one dtype
            qx, qw = fp4q_quant2d_batch([(x, None, stream_base + 1), (w, None, stream_base + 2)], seed=seed)
        else:
            qx = fp4q_quant2d(x, out=alloc_fp4(T, K, x.device, block=act_layout), seed=seed,
                              stream_id=stream_base + 1)
            qw = fp4q_quant2d(w, seed=seed, stream_id=stream_base + 2)
        ctx.q = (qx, qw)
        ctx.seed, ctx.stream_base, ctx.x_dtype = seed, stream_base, x.dtype
        return fp4q_gemm("fwd", qx, qw)

    @staticmethod
    def backward(ctx, dy):
        qx, qw = ctx.q
        qdy = fp4q_quant2d(dy.contiguous(), seed=ctx.seed, stream_id=ctx.stream_base + 3)
        dx = dw = None
        if ctx.needs_input_grad[0]:
            # a bf16 X gets its gradient from the bf16 epilogue (the fp32
            # result rounded to nearest even)
            dx = fp4q_gemm("dgrad", qdy, qw, out_dtype=ctx.x_dtype)
        if ctx.needs_input_grad[1]:
            dw = fp4q_gemm("wgrad", qdy, qx)
        # ctx.q stays: a graph kept with retain_graph=True may run backward
        # again; autograd frees it with the graph
        return dx, dw, None, None, None


def fp4_linear(x, w, seed=0, stream_base=0, act_layout=32):
    """Y = X W^T with X [T x K] (bf16/fp32, CUDA, row-major) and W [N x K]
    (fp32 or bf16): the FP4 forward and the FP4 backward of the recipe.
    act_layout 32 (32x32 blocks, the transposition-invariant layout) or "1d"
    (the appendix's 1x32 activation blocks); W and dY always take 32x32.
    seed / stream_base key the Philox streams (X, W, dY use stream_base+1..3)."""
    return _FP4LinearFn.apply(x, w, seed, stream_base, act_layout)


_layer_ids = itertools.count()
_live_ids = weakref.WeakValueDictionary()


class FP4Linear(torch.nn.Module):
    """Bias-free linear layer with an fp32 master weight; every call draws
    fresh stochastic-rounding bits (the call counter is the Philox key).

    Each layer owns the Philox streams 16*layer_id + 1..3, so two layers of
    the same shape never draw the same bits: layer_id defaults to the next
    unused id, and an explicit id already held by a live layer is refused."""

    def __init__(self, in_features, out_features, layer_id=None, act_layout=32, device="cuda"):
        super().__init__()
        if layer_id is None:
            layer_id = next(_layer_ids)
            while layer_id in _live_ids:
                layer_id = next(_layer_ids)
        elif layer_id in _live_ids:
            raise ValueError("FP4Linear layer_id %d is already used by a live layer; its stochastic "
                             "rounding would repeat that layer's random bits" % layer_id)
        if not 0 <= layer_id < (1 << 27):
            raise ValueError("FP4Linear layer_id must be in [0, 2^27)")
        _live_ids[layer_id] = self
        self.layer_id = layer_id
        self.weight = torch.nn.Parameter(
            torch.randn(out_features, in_features, device=device) * (in_features ** -0.5))
        self.stream_base = 16 * layer_id
        self.act_layout = act_layout
        self.calls = 0

    def forward(self, x):
        self.calls += 1
        return fp4_linear(x, self.weight, seed=self.calls, stream_base=self.stream_base,
                          act_layout=self.act_layout)
