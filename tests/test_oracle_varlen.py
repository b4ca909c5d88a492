"""Pins of the float64 oracle for packed variable-length sequences (CPU only).

``oracle.moba_forward_varlen`` runs the definition once per sequence.  It is pinned
against ``oracle.moba_bruteforce_packed``, an independent mask formulation over the
packed token axis (one gate matrix over the blocks of every sequence, other
sequences' blocks banned), and against dense causal attention per sequence when every
block is selected.
"""
import numpy as np
import pytest
import torch

import oracle


def packed_qkv(seed, lengths, hq, hkv, d):
    r = np.random.default_rng(seed)
    total = int(sum(lengths))
    Q = r.standard_normal((total, hq, d))
    K = r.standard_normal((total, hkv, d))
    V = r.standard_normal((total, hkv, d))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return Q, K, V, cu


@pytest.mark.parametrize("lengths,B,k", [
    ((37, 100, 64, 5), 16, 3),        # ragged tails, a sequence shorter than a block
    ((48, 1, 96, 33), 16, 4),         # a one-token sequence, whole and partial blocks
    ((130, 70), 32, 2),
    ((64, 64, 64), 16, 8),            # k >= the number of blocks: every block
])
def test_varlen_matches_packed_bruteforce(lengths, B, k):
    Q, K, V, cu = packed_qkv(sum(lengths) + B, lengths, 4, 2, 16)
    sc = 0.3
    o1, l1, i1 = oracle.moba_forward_varlen(Q, K, V, cu, B, k, sc)
    o2, l2, i2 = oracle.moba_bruteforce_packed(Q, K, V, cu, B, k, sc)
    assert np.array_equal(i1, i2)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_varlen_equal_lengths_is_the_batched_forward():
    """Sequences of one length packed = a batch of that length."""
    b, T, hq, hkv, d, B, k = 3, 96, 4, 1, 16, 16, 3
    Q, K, V, cu = packed_qkv(5, [T] * b, hq, hkv, d)
    o1, l1, i1 = oracle.moba_forward_varlen(Q, K, V, cu, B, k, 0.25)
    o2, l2, i2, _ = oracle.moba_forward(Q.reshape(b, T, hq, d), K.reshape(b, T, hkv, d),
                                        V.reshape(b, T, hkv, d), B, k, 0.25)
    assert np.array_equal(i1, i2.transpose(1, 0, 2, 3).reshape(hq, b * T, k))
    np.testing.assert_allclose(o1, o2.reshape(b * T, hq, d), rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2.transpose(1, 0, 2).reshape(hq, b * T), rtol=0,
                               atol=1e-12)


def test_varlen_all_blocks_is_causal_attention_per_sequence():
    """k >= blocks per sequence: causal attention within each sequence (torch SDPA with
    a block-diagonal causal mask, fp64)."""
    lengths = (40, 17, 71)
    Q, K, V, cu = packed_qkv(11, lengths, 2, 2, 8)
    total = cu[-1]
    o1, l1, _ = oracle.moba_forward_varlen(Q, K, V, cu, 16, 8, 0.5)
    seq = np.searchsorted(cu, np.arange(total), side="right") - 1
    mask = (seq[:, None] == seq[None, :]) & (np.arange(total)[None, :] <= np.arange(total)[:, None])
    q = torch.from_numpy(Q).permute(1, 0, 2)
    kk = torch.from_numpy(K).permute(1, 0, 2)
    vv = torch.from_numpy(V).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, kk, vv, attn_mask=torch.from_numpy(mask), scale=0.5).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(o1, ref, rtol=0, atol=1e-12)
    z = 0.5 * np.einsum("thd,uhd->htu", Q, K)
    z = np.where(mask[None], z, -np.inf)
    m = z.max(axis=2)
    np.testing.assert_allclose(l1, m + np.log(np.exp(z - m[..., None]).sum(axis=2)),
                               rtol=0, atol=1e-12)


@pytest.mark.parametrize("lengths,B,k", [((37, 100, 64, 5), 16, 3), ((48, 1, 96), 16, 4)])
def test_varlen_backward_matches_packed_autograd(lengths, B, k):
    """Gradients of packed sequences against torch autograd through one dense masked
    softmax over the packed token axis: allowed[h, i, u] = u is in a block of i's own
    sequence that i selected (ids from the packed brute force) and u <= i (fp64)."""
    hq, hkv, d = 4, 2, 8
    Q, K, V, cu = packed_qkv(sum(lengths) + 7, lengths, hq, hkv, d)
    dO = np.random.default_rng(3).standard_normal(Q.shape)
    sc = 0.35
    _, _, idx = oracle.moba_bruteforce_packed(Q, K, V, cu, B, k, sc)
    total = int(cu[-1])
    seq = np.searchsorted(cu, np.arange(total), side="right") - 1
    pos = np.arange(total) - cu[seq]
    allowed = np.zeros((hq, total, total), bool)
    for h in range(hq):
        for i in range(total):
            S = set(int(j) for j in idx[h, i] if j >= 0)
            allowed[h, i] = ((seq == seq[i]) & np.isin(pos // B, list(S))
                             & (pos <= pos[i]))
    G = hq // hkv
    q = torch.tensor(Q.transpose(1, 0, 2), requires_grad=True)
    kk = torch.tensor(K.transpose(1, 0, 2), requires_grad=True)
    vv = torch.tensor(V.transpose(1, 0, 2), requires_grad=True)
    s = sc * q @ kk.repeat_interleave(G, 0).transpose(1, 2)
    s = s.masked_fill(~torch.tensor(allowed), float("-inf"))
    out = torch.softmax(s, -1) @ vv.repeat_interleave(G, 0)
    (out * torch.tensor(dO.transpose(1, 0, 2))).sum().backward()
    ref = [x.grad.numpy().transpose(1, 0, 2) for x in (q, kk, vv)]
    got = oracle.moba_backward_varlen(Q, K, V, dO, cu, B, k, sc)
    for g_, r_ in zip(got, ref):
        np.testing.assert_allclose(g_, r_, rtol=1e-9, atol=1e-11)
