"""Pins of the float64 oracle for the full-attention decode that follows a MoBA
prefill (``oracle.decode_attention``; CPU only).

* Against torch SDPA (fp64) with an explicit mask in which new token i sees keys
  0 .. Tk - n + i, including GQA.
* n = Tk is dense causal attention: it equals the MoBA forward with every block
  selected.
* Closed forms: one key (out = v, lse = scale q.k), constant values (out = v),
  zero queries (uniform weights: out = mean of the visible values, lse = ln(count)).
"""
import numpy as np
import pytest
import torch

import oracle


def rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("b,n,Tk,hq,hkv,d", [(1, 1, 50, 4, 2, 16), (2, 3, 37, 6, 2, 8),
                                             (1, 8, 8, 2, 1, 16), (1, 4, 130, 8, 8, 8)])
def test_decode_matches_sdpa_with_offset_mask(b, n, Tk, hq, hkv, d):
    Q, K, V = rand(1, b, n, hq, d), rand(2, b, Tk, hkv, d), rand(3, b, Tk, hkv, d)
    sc = 0.3
    out, lse = oracle.decode_attention(Q, K, V, sc)
    G = hq // hkv
    mask = np.arange(Tk)[None, :] <= (Tk - n + np.arange(n))[:, None]      # [n, Tk]
    q = torch.from_numpy(Q).permute(0, 2, 1, 3)                            # b, hq, n, d
    k = torch.from_numpy(K).permute(0, 2, 1, 3).repeat_interleave(G, 1)
    v = torch.from_numpy(V).permute(0, 2, 1, 3).repeat_interleave(G, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=torch.from_numpy(mask), scale=sc).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    z = sc * (q @ k.transpose(-1, -2)).numpy()
    z = np.where(mask[None, None], z, -np.inf)
    m = z.max(-1)
    np.testing.assert_allclose(lse, m + np.log(np.exp(z - m[..., None]).sum(-1)), rtol=0,
                               atol=1e-12)


def test_decode_all_new_tokens_is_dense_causal():
    """n = Tk: every token is new, so decode is causal attention over the sequence, the
    MoBA forward with every block selected."""
    T, hq, hkv, d = 64, 4, 2, 8
    Q, K, V = rand(4, 1, T, hq, d), rand(5, 1, T, hkv, d), rand(6, 1, T, hkv, d)
    out, lse = oracle.decode_attention(Q, K, V, 0.4)
    o2, l2, _, _ = oracle.moba_forward(Q, K, V, 16, 4, 0.4)
    np.testing.assert_allclose(out, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l2, rtol=0, atol=1e-12)


def test_decode_closed_forms():
    d = 8
    q, k, v = rand(7, 1, 1, 2, d), rand(8, 1, 1, 1, d), rand(9, 1, 1, 1, d)
    out, lse = oracle.decode_attention(q, k, v, 0.5)
    np.testing.assert_allclose(out[0, 0, 0], v[0, 0, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0, 0], 0.5 * q[0, 0, 0] @ k[0, 0, 0], rtol=1e-14)
    # constant values: any weights give out = v
    Tk, n = 40, 3
    vc = np.broadcast_to(rand(10, 1, 1, 1, d), (1, Tk, 1, d)).copy()
    out, _ = oracle.decode_attention(rand(11, 1, n, 2, d), rand(12, 1, Tk, 1, d), vc, 0.7)
    np.testing.assert_allclose(out, np.broadcast_to(vc[:, :1], out.shape), rtol=0, atol=1e-13)
    # zero queries: uniform over the visible keys
    V = rand(13, 1, Tk, 1, d)
    out, lse = oracle.decode_attention(np.zeros((1, n, 2, d)), rand(14, 1, Tk, 1, d), V, 0.7)
    for i in range(n):
        cnt = Tk - n + i + 1
        np.testing.assert_allclose(out[0, i, 1], V[0, :cnt, 0].mean(0), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[0, 1, i], np.log(cnt), rtol=1e-14)
