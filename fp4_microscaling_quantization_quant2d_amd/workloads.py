"""Seeded synthetic inputs for the five workloads.

This module only draws random numbers and lays them out; it holds none of the
quantization or GEMM arithmetic, so both the GPU path and the CPU oracle can
take their inputs from it.

Recipe (numpy PCG64, one SeedSequence per workload, one child stream per
tensor): values are drawn as float32 normals, scaled to the stated standard
deviation, optional outlier channels are multiplied in, and bf16 tensors are
produced by torch's round-to-nearest-even float32 -> bfloat16 cast.  bf16
tensors are returned as uint16 bit patterns (numpy has no bfloat16).

Shapes follow the linear layers the pages train (OLMo-1B, OLMo-7B, a 30B MoE)
and their MXFP8 attention pathway:
  tiny  : A, W, dY fp32 256x256, N(0,1), 655 random entries x20
  1b    : T=4096, hidden 2048, FFN 8192 (up and down projections)
  7b    : T=8192, hidden 4096: QKV 4096->12288, O 4096->4096,
          up 4096->11008, down 11008->4096
  moe   : 8192 tokens, hidden 2048, 128 experts of FFN 768, top-8 routing
  attn  : Q, K [4, 32, 4096, 128] bf16 N(0,1); O-projection 4096x4096 at
          16384 tokens
Activations are N(0,1) with max(1, round(0.001*C)) seeded columns scaled
x50; weights N(0, 0.02); output gradients N(0, 1e-3).
"""
from dataclasses import dataclass, field
from typing import Dict, List

import numpy as np

WORKLOAD_SEEDS = {"tiny": 1001, "1b": 1002, "7b": 1003, "moe": 1004, "attn": 1005}
X_STD, W_STD, DY_STD = 1.0, 0.02, 1e-3
OUTLIER_FRAC, OUTLIER_GAIN = 0.001, 50.0


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 (torch CPU cast), as uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape, std):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _activation(rng, rows, cols, std=X_STD):
    a = _normal(rng, (rows, cols), std)
    n_out = max(1, int(round(OUTLIER_FRAC * cols)))
    ch = rng.choice(cols, size=n_out, replace=False)
    a[:, ch] *= np.float32(OUTLIER_GAIN)
    return a


@dataclass
class Linear:
    """One linear layer y = x W^T: X [T x K], W [N x K], dY [T x N] (bf16 bits)."""
    name: str
    X: np.ndarray
    W: np.ndarray
    dY: np.ndarray

    @property
    def T(self):
        return self.X.shape[0]

    @property
    def K(self):
        return self.X.shape[1]

    @property
    def N(self):
        return self.W.shape[0]

    def flops(self):
        return 2.0 * self.T * self.N * self.K


def _children(name, n):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(WORKLOAD_SEEDS[name]).spawn(n)]


def linear_layer(name: str, T: int, K: int, N: int, stream_base: int) -> Linear:
    """bf16 X/W/dY for one layer; stream_base picks independent child streams."""
    ss = np.random.SeedSequence([WORKLOAD_SEEDS.get(name.split(":")[0], 7), stream_base])
    gx, gw, gd = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(3)]
    X = f32_to_bf16_bits(_activation(gx, T, K))
    W = f32_to_bf16_bits(_normal(gw, (N, K), W_STD))
    dY = f32_to_bf16_bits(_normal(gd, (T, N), DY_STD))
    return Linear(name, X, W, dY)


def tiny():
    """fp32 A, W, dY [256 x 256], N(0,1), exactly 655 (1%) entries x20 each."""
    out = {}
    for nm, rng in zip(("A", "W", "dY"), _children("tiny", 3)):
        a = _normal(rng, (256, 256), 1.0)
        idx = rng.choice(256 * 256, size=655, replace=False)
        a.reshape(-1)[idx] *= np.float32(20.0)
        out[nm] = a
    return out


LAYERS_1B = [("up", 2048, 8192), ("down", 8192, 2048)]          # (name, K, N)
LAYERS_7B = [("qkv", 4096, 12288), ("o", 4096, 4096), ("up", 4096, 11008),
             ("down", 11008, 4096)]


def config_1b(T=4096) -> List[Linear]:
    return [layer_1b(i, T) for i in range(len(LAYERS_1B))]


def config_7b(T=8192) -> List[Linear]:
    return [layer_7b(i, T) for i in range(len(LAYERS_7B))]


def layer_7b(i, T=8192) -> Linear:
    nm, K, N = LAYERS_7B[i]
    return linear_layer("7b:" + nm, T, K, N, i)


def layer_1b(i, T=4096) -> Linear:
    nm, K, N = LAYERS_1B[i]
    return linear_layer("1b:" + nm, T, K, N, i)


@dataclass
class MoE:
    """Grouped expert layer.  Token rows are gathered per expert, each expert's
    segment starting at a multiple of 32 (padding rows are zero).
      row_off [E+1] : segment starts in the gathered buffers
      counts  [E]   : valid rows per expert
      X   [rows x H]  gathered activations      W_up   [E*F x H]
      dY  [rows x F]  up-projection grads       W_down [E*H x F]
      A   [rows x F]  down-projection input     dY_down [rows x H]
    """
    E: int
    H: int
    F: int
    row_off: np.ndarray
    counts: np.ndarray
    X: np.ndarray
    W_up: np.ndarray
    dY: np.ndarray
    A: np.ndarray
    W_down: np.ndarray
    dY_down: np.ndarray
    assign: np.ndarray = field(default=None)


def config_moe(tokens=8192, H=2048, E=128, F=768, topk=8) -> MoE:
    g = _children("moe", 8)
    logits = g[0].standard_normal((tokens, E))
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    # top-k by probability; ties broken towards the lower expert index
    order = np.lexsort((np.broadcast_to(np.arange(E), p.shape), -p), axis=1)[:, :topk]
    counts = np.bincount(order.reshape(-1), minlength=E).astype(np.int64)
    padded = (counts + 31) // 32 * 32
    row_off = np.zeros(E + 1, dtype=np.int64)
    row_off[1:] = np.cumsum(padded)
    rows = int(row_off[-1])
    tok = np.empty(rows, dtype=np.int64)
    tok.fill(-1)
    fill = row_off[:-1].copy()
    for t in range(tokens):
        for e in order[t]:
            tok[fill[e]] = t
            fill[e] += 1
    valid = tok >= 0
    x_tok = _activation(g[1], tokens, H)
    X = np.zeros((rows, H), dtype=np.float32)
    X[valid] = x_tok[tok[valid]]
    dY = np.zeros((rows, F), dtype=np.float32)
    dY[valid] = _normal(g[2], (int(valid.sum()), F), DY_STD)
    A = np.zeros((rows, F), dtype=np.float32)
    A[valid] = _activation(g[3], int(valid.sum()), F)
    dYd = np.zeros((rows, H), dtype=np.float32)
    dYd[valid] = _normal(g[4], (int(valid.sum()), H), DY_STD)
    W_up = _normal(g[5], (E * F, H), W_STD)
    W_down = _normal(g[6], (E * H, F), W_STD)
    bf = f32_to_bf16_bits
    return MoE(E, H, F, row_off, counts, bf(X), bf(W_up), bf(dY), bf(A), bf(W_down), bf(dYd),
               assign=order)


@dataclass
class Attn:
    """Q, K [B, Hh, L, D] bf16 bits and the O-projection layer."""
    Q: np.ndarray
    K: np.ndarray
    o_proj: Linear


def config_attn(B=4, Hh=32, L=4096, D=128, T_o=16384, d_model=4096) -> Attn:
    g = _children("attn", 2)
    Q = f32_to_bf16_bits(_normal(g[0], (B, Hh, L, D), 1.0))
    K = f32_to_bf16_bits(_normal(g[1], (B, Hh, L, D), 1.0))
    o = linear_layer("attn:o", T_o, d_model, d_model, 0)
    return Attn(Q, K, o)


def total_7b_elements(T=8192) -> Dict[str, int]:
    """Element counts of the 7B step's quantized tensors (for byte accounting)."""
    n = {"X": 0, "W": 0, "dY": 0}
    for _, K, N in LAYERS_7B:
        n["X"] += T * K
        n["W"] += N * K
        n["dY"] += T * N
    return n
