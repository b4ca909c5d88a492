"""Pins of the float64 backward oracle (CPU only).

The oracle's gradient (oracle.moba_backward) is checked against facts fixed outside it:
central finite differences of sum(dO * out) with the block selection held fixed, torch
autograd through an independent masked dense-softmax formulation (the MoBA mask built
from the selection), torch autograd through SDPA for the dense and k = 1 cases, and the
closed-form sums of dV and dK.
"""
import numpy as np
import pytest

import oracle
from workloads import small_workload, make_inputs, bf16_to_f64

torch = pytest.importorskip("torch")


def _inputs(hq, hkv, d, T, B, k, seed, recipe="offset"):
    w = small_workload("bwd", 1, hq, hkv, d, T, B, k, recipe, seed)
    inp = make_inputs(w)
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    dO = np.random.default_rng(seed + 100).standard_normal(Q.shape)
    return w, Q, K, V, dO


def _loss(Q, K, V, dO, B, scale, idx):
    """sum(dO * out) with the selection idx held fixed."""
    b, T, hq, d = Q.shape
    rows = [(0, t, h) for t in range(T) for h in range(hq)]
    sels = [[int(j) for j in idx[0, h, t] if j >= 0] for (_, t, h) in rows]
    out, _ = oracle.attend_rows(Q, K, V, B, scale, rows, sels)
    return sum(float(out[i] @ dO[0, t, h]) for i, (_, t, h) in enumerate(rows))


def test_backward_matches_finite_differences():
    w, Q, K, V, dO = _inputs(2, 1, 8, 64, 16, 2, 31)
    idx = oracle.select_blocks(Q, oracle.centroids(K, w.block), w.block, w.topk)
    dQ, dK, dV = oracle.moba_backward(Q, K, V, dO, w.block, w.topk, w.sm_scale, idx=idx)
    r = np.random.default_rng(5)
    h = 1e-6
    for X, dX in ((Q, dQ), (K, dK), (V, dV)):
        for _ in range(12):
            pos = tuple(int(r.integers(n)) for n in X.shape)
            old = X[pos]
            X[pos] = old + h
            lp = _loss(Q, K, V, dO, w.block, w.sm_scale, idx)
            X[pos] = old - h
            lm = _loss(Q, K, V, dO, w.block, w.sm_scale, idx)
            X[pos] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - dX[pos]) <= 1e-6 * max(1.0, abs(fd)), (pos, fd, dX[pos])


def _torch_masked_grads(Q, K, V, dO, scale, allowed):
    """Autograd through softmax(scale Q K^T masked to `allowed` [Hq, T, T]) V, fp64."""
    G = Q.shape[2] // K.shape[2]
    q = torch.tensor(Q[0].transpose(1, 0, 2), requires_grad=True)       # [Hq, T, d]
    k = torch.tensor(K[0].transpose(1, 0, 2), requires_grad=True)       # [Hkv, T, d]
    v = torch.tensor(V[0].transpose(1, 0, 2), requires_grad=True)
    ke, ve = k.repeat_interleave(G, 0), v.repeat_interleave(G, 0)
    s = scale * q @ ke.transpose(1, 2)
    s = s.masked_fill(~torch.tensor(allowed), float("-inf"))
    out = torch.softmax(s, -1) @ ve
    (out * torch.tensor(dO[0].transpose(1, 0, 2))).sum().backward()
    f = lambda x: x.grad.numpy().transpose(1, 0, 2)[None]
    return f(q), f(k), f(v)


@pytest.mark.parametrize("hq,hkv,d,T,B,k,seed", [(4, 2, 16, 128, 16, 3, 41),
                                                  (2, 2, 8, 96, 32, 2, 42),
                                                  (3, 1, 16, 80, 16, 5, 43)])
def test_backward_matches_autograd_of_masked_softmax(hq, hkv, d, T, B, k, seed):
    """The MoBA mask from the selection (allowed[h, t, u] = block(u) selected by (t, h)
    and u <= t), a dense masked softmax, and torch autograd."""
    w, Q, K, V, dO = _inputs(hq, hkv, d, T, B, k, seed)
    idx = oracle.select_blocks(Q, oracle.centroids(K, B), B, k)
    allowed = np.zeros((hq, T, T), bool)
    blk = np.arange(T) // B
    for h in range(hq):
        for t in range(T):
            S = set(int(j) for j in idx[0, h, t] if j >= 0)
            allowed[h, t] = np.isin(blk, list(S)) & (np.arange(T) <= t)
    ref = _torch_masked_grads(Q, K, V, dO, w.sm_scale, allowed)
    got = oracle.moba_backward(Q, K, V, dO, B, k, w.sm_scale, idx=idx)
    for g_, r_ in zip(got, ref):
        np.testing.assert_allclose(g_, r_, rtol=1e-9, atol=1e-11)


@pytest.mark.parametrize("k", [1, 99])
def test_backward_special_cases_match_sdpa(k):
    """k >= nb is dense causal attention; k = 1 is block-local causal attention.  Both
    against torch autograd through scaled_dot_product_attention (fp64)."""
    hq, hkv, d, T, B = 4, 2, 16, 64, 16
    w, Q, K, V, dO = _inputs(hq, hkv, d, T, B, k, 44, "iid")
    G = hq // hkv
    q = torch.tensor(Q[0].transpose(1, 0, 2)[None], requires_grad=True)
    kk = torch.tensor(K[0].transpose(1, 0, 2)[None], requires_grad=True)
    vv = torch.tensor(V[0].transpose(1, 0, 2)[None], requires_grad=True)
    t = torch.arange(T)
    mask = t[None, :] <= t[:, None]
    if k == 1:
        mask = mask & ((t[None, :] // B) == (t[:, None] // B))
    out = torch.nn.functional.scaled_dot_product_attention(
        q, kk.repeat_interleave(G, 1), vv.repeat_interleave(G, 1), attn_mask=mask,
        scale=w.sm_scale)
    (out * torch.tensor(dO[0].transpose(1, 0, 2)[None])).sum().backward()
    f = lambda x: x.grad[0].numpy().transpose(1, 0, 2)[None]
    got = oracle.moba_backward(Q, K, V, dO, B, k, w.sm_scale)
    for g_, r_ in zip(got, (f(q), f(kk), f(vv))):
        np.testing.assert_allclose(g_, r_, rtol=1e-9, atol=1e-11)


def test_backward_closed_form_sums():
    """Every row's softmax weights sum to 1 and its dz sum to 0, so summed over all
    keys of a kv-head, dV is the sum of dO over that head group's rows and dK is 0."""
    w, Q, K, V, dO = _inputs(4, 2, 16, 128, 32, 3, 45)
    dQ, dK, dV = oracle.moba_backward(Q, K, V, dO, w.block, w.topk, w.sm_scale)
    G = 2
    for g in range(2):
        np.testing.assert_allclose(dV[0, :, g].sum(0), dO[0, :, g * G:(g + 1) * G].sum((0, 1)),
                                   rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(dK[0, :, g].sum(0), 0.0, atol=1e-10)
