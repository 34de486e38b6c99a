"""Pins of the oracle's attention with MXFP8 queries and keys (Sec. 3.2
"MXFP8 Attention" of "Stable FP4 Training via Transposition-Invariant Block
Quantization"; the pages name the format, not the attention arithmetic,
which is standard scaled dot-product attention).

The oracle is plain loops in fp64; it is pinned against
- numpy's fp64 matmul / exp softmax (a library routine) for O and lse;
- torch's fp64 autograd on the CPU (a library routine) for dQ, dK, dV;
- identities: V = 1 gives O = 1; Q = 0 gives the running mean of V (causal)
  or the mean (full); the rows of dS sum to zero, so sum_j dK_j = 0;
- central finite differences of a scalar loss on a tiny head (brute force);
- the MXFP8 inputs: dequantized codes are exact in fp64, so attention on
  them equals attention on those values."""
import numpy as np
import pytest
import torch


def _ref_fwd(Q, K, V, scale, causal):
    S = scale * (Q @ K.T)
    L = Q.shape[0]
    if causal:
        S = np.where(np.tril(np.ones((L, L), bool)), S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    P = E / l
    return P @ V, (m + np.log(l))[:, 0], P


def _torch_grads(Q, K, V, dO, scale, causal):
    q, k, v = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (Q, K, V))
    S = scale * q @ k.T
    if causal:
        S = S.masked_fill(~torch.tril(torch.ones(S.shape, dtype=torch.bool)), float("-inf"))
    O = torch.softmax(S, dim=1) @ v
    O.backward(torch.tensor(dO, dtype=torch.float64))
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def _inputs(L, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((L, d)) * s for s in (1.0, 1.0, 1.0, 0.1)]


@pytest.mark.parametrize("L,d", [(7, 4), (64, 32), (200, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_matches_numpy(orc, L, d, causal):
    Q, K, V, _ = _inputs(L, d, L + d)
    scale = d ** -0.5
    O, lse, pv = orc.attn_fwd(Q, K, V, scale, causal)
    Or, lr, P = _ref_fwd(Q, K, V, scale, causal)
    assert np.allclose(O, Or, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, lr, rtol=1e-13, atol=1e-13)
    assert np.allclose(pv, P @ np.abs(V), rtol=1e-12, atol=1e-13)
    rows = np.array([L - 1, 0, L // 2])
    Os, ls, _ = orc.attn_fwd(Q, K, V, scale, causal, rows=rows)
    assert np.array_equal(Os, O[rows]) and np.array_equal(ls, lse[rows])


@pytest.mark.parametrize("L,d", [(9, 4), (96, 64), (160, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd(orc, L, d, causal):
    Q, K, V, dO = _inputs(L, d, 3 * L + d)
    scale = 0.7 * d ** -0.5
    dQ, mq = orc.attn_bwd_dq(Q, K, V, dO, scale, causal)
    dK, dV, mk = orc.attn_bwd_dkdv(Q, K, V, dO, scale, causal)
    tq, tk, tv = _torch_grads(Q, K, V, dO, scale, causal)
    assert np.allclose(dQ, tq, rtol=1e-10, atol=1e-12)
    assert np.allclose(dK, tk, rtol=1e-10, atol=1e-12)
    assert np.allclose(dV, tv, rtol=1e-10, atol=1e-12)
    # magnitudes bound what they measure
    assert np.all(mq["ds_abs_k"] >= np.abs(dQ) * (1 - 1e-12))
    assert np.all(mk["ds_abs_q"] >= np.abs(dK) * (1 - 1e-12))
    assert np.all(mk["p_do"] >= np.abs(dV) * (1 - 1e-12))
    # p_q, p_k: the P-weighted magnitudes, against numpy
    _, _, P = _ref_fwd(Q, K, V, scale, causal)
    assert np.allclose(mk["p_q"], scale * P.T @ np.abs(Q), rtol=1e-12, atol=1e-14)
    assert np.allclose(mq["p_k"], scale * P @ np.abs(K), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_identities(orc, causal):
    L, d = 48, 16
    Q, K, V, dO = _inputs(L, d, 5)
    O, _, _ = orc.attn_fwd(Q, K, np.ones((L, d)), 0.3, causal)
    assert np.allclose(O, 1.0, rtol=0, atol=1e-14)
    O, lse, _ = orc.attn_fwd(np.zeros((L, d)), K, V, 0.3, causal)
    if causal:
        ref = np.cumsum(V, axis=0) / np.arange(1, L + 1)[:, None]
        assert np.allclose(lse, np.log(np.arange(1, L + 1)), atol=1e-14)
    else:
        ref = np.broadcast_to(V.mean(axis=0), V.shape)
    assert np.allclose(O, ref, atol=1e-13)
    dK, _, _ = orc.attn_bwd_dkdv(Q, K, V, dO, 0.3, causal)
    assert np.allclose(dK.sum(axis=0), 0.0, atol=1e-12)


def test_finite_differences(orc):
    """Loss = sum(O * G): the oracle's dQ, dK, dV equal central differences
    of the oracle's own forward pass (step 1e-6, fp64)."""
    L, d, scale = 5, 3, 0.8
    Q, K, V, G = _inputs(L, d, 11)
    G = G * 10
    dQ, _ = orc.attn_bwd_dq(Q, K, V, G, scale, True)
    dK, dV, _ = orc.attn_bwd_dkdv(Q, K, V, G, scale, True)

    def loss(Qx, Kx, Vx):
        return float((orc.attn_fwd(Qx, Kx, Vx, scale, True)[0] * G).sum())

    h = 1e-6
    for X, g, which in ((Q, dQ, 0), (K, dK, 1), (V, dV, 2)):
        num = np.zeros_like(X)
        for i in range(L):
            for t in range(d):
                args = [Q.copy(), K.copy(), V.copy()]
                args[which][i, t] += h
                up = loss(*args)
                args[which][i, t] -= 2 * h
                num[i, t] = (up - loss(*args)) / (2 * h)
        assert np.allclose(g, num, rtol=1e-6, atol=1e-8), which


def test_on_mxfp8_inputs(orc):
    """Q and K through the (pinned) MXFP8 quantizer: their dequantized values
    are exact in fp64, and attention on the codes is attention on them."""
    from fp4_microscaling_quantization_quant2d_amd import workloads as wl
    rng = np.random.default_rng(8)
    L, d = 64, 128
    Qb = wl.f32_to_bf16_bits(rng.standard_normal((L, d)).astype(np.float32))
    Kb = wl.f32_to_bf16_bits(rng.standard_normal((L, d)).astype(np.float32))
    qc, qs = orc.quant1d_mxfp8(Qb)
    kc, ks = orc.quant1d_mxfp8(Kb)
    Qd, Kd = orc.dequant_mxfp8(qc, qs, L, d), orc.dequant_mxfp8(kc, ks, L, d)
    V = rng.standard_normal((L, d))
    O, lse, _ = orc.attn_fwd(Qd, Kd, V, d ** -0.5, True)
    Or, lr, _ = _ref_fwd(Qd, Kd, V, d ** -0.5, True)
    assert np.allclose(O, Or, rtol=1e-12, atol=1e-13) and np.allclose(lse, lr, atol=1e-13)
    # MXFP8 (3 mantissa bits) moves the outputs off the bf16 ones, by little
    Ob, _, _ = _ref_fwd(wl.bf16_bits_to_f32(Qb).astype(np.float64), wl.bf16_bits_to_f32(Kb).astype(np.float64),
                        V, d ** -0.5, True)
    assert 0 < np.abs(O - Ob).max() < 0.25
