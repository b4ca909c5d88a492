"""The HIP backward on a partial last block and on packed variable-length sequences,
against the float64 oracle (``oracle.moba_backward`` / ``oracle.moba_backward_varlen``,
pinned by tests/test_oracle_backward.py and tests/test_oracle_varlen.py).

Tolerances are those of tests/test_gpu_backward.py (mean |err| <= 2u mean |g|, max
|err| <= 4u max |g|, u = 2^-8).  Each case checks first that the GPU selection equals
the oracle's, so that the oracle's gradients (from its own selection) are the reference.
"""
import numpy as np
import pytest

import oracle
from workloads import small_workload, make_inputs, make_output_grad, bf16_to_f64
from test_gpu_backward import check_grads, say, dev, f64
from test_gpu_varlen import packed_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moba():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_sparse_long_pool_amd as m
    return m


RAGGED = [
    # b, T, hq, hkv, d, B, topk
    (1, 1000, 4, 2, 128, 128, 4),      # 7 whole blocks and a 104-token tail
    (2, 1100, 8, 2, 64, 256, 3),       # 76-token tail, batch 2
    (1, 300, 2, 1, 128, 256, 2),       # one whole block and a 44-token tail
    (1, 770, 4, 4, 64, 48, 5),         # B = 48, a 2-token tail
    (1, 530, 8, 1, 128, 16, 9),        # B = 16, G = 8, a 2-token tail
    (1, 90, 2, 1, 128, 128, 3),        # one partial block only
]


@pytest.mark.parametrize("b,T,hq,hkv,d,B,k", RAGGED)
def test_backward_ragged_seqlen_all_elements(moba, b, T, hq, hkv, d, B, k):
    w = small_workload("ragged_bwd", b, hq, hkv, d, T, B, k, "offset", seed=T + 3 * B)
    say(f"[bwd ragged] b={b} T={T} hq={hq} hkv={hkv} d={d} B={B} k={k}")
    inp = make_inputs(w)
    g_bits = make_output_grad(w)
    q, kk, v = (dev(inp[x]) for x in "qkv")
    out, lse, idx = moba.forward(q, kk, v, B, k, w.sm_scale)
    dq, dk, dv = moba.backward(q, kk, v, out, lse, idx, dev(g_bits), B, k, w.sm_scale)
    torch.cuda.synchronize()
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    ref_idx = oracle.select_blocks(Q, oracle.centroids(K, B), B, k)
    ndiff = int((idx.cpu().numpy() != ref_idx).any(axis=-1).sum())
    assert ndiff == 0, f"{ndiff} rows select other blocks than the oracle; pick another seed"
    ref = oracle.moba_backward(Q, K, V, bf16_to_f64(g_bits), B, k, w.sm_scale)
    check_grads((f64(dq), f64(dk), f64(dv)), ref)


def packed_fwd_bwd(moba, lengths, hq, hkv, d, B, k, seed, **kw):
    qb, kb, vb, cu = packed_inputs(lengths, hq, hkv, d, seed, B=B)
    gb = packed_inputs(lengths, hq, hkv, d, seed + 2)[0]      # i.i.d. N(0,1) bf16 [total, hq, d]
    scale = 1.0 / np.sqrt(d)
    q, kk, v = dev(qb), dev(kb), dev(vb)
    out, lse, idx = moba.forward_varlen(q, kk, v, cu, B, k, scale)
    dq, dk, dv = moba.backward_varlen(q, kk, v, out, lse, idx, dev(gb), cu, B, k, scale, **kw)
    torch.cuda.synchronize()
    return (qb, kb, vb, gb, cu, scale), idx.cpu().numpy(), (f64(dq), f64(dk), f64(dv))


PACKED = [
    # lengths, hq, hkv, d, B, topk
    ((1000, 37, 2048, 513, 1), 8, 2, 128, 128, 4),
    ((300, 1500, 64, 900), 8, 8, 64, 64, 9),
    ((16, 17, 15, 700, 33), 16, 2, 128, 16, 6),
    ((2500,), 4, 2, 128, 512, 2),
    ((0, 640, 0, 129), 4, 1, 128, 128, 3),       # empty sequences in the pack
    ((300, 129, 700), 6, 2, 128, 128, 4),        # G = 3
]


@pytest.mark.parametrize("lengths,hq,hkv,d,B,k", PACKED)
def test_backward_varlen_all_elements(moba, lengths, hq, hkv, d, B, k):
    say(f"[bwd varlen] lengths={lengths} hq={hq} hkv={hkv} d={d} B={B} k={k}")
    (qb, kb, vb, gb, cu, scale), gi, got = packed_fwd_bwd(moba, lengths, hq, hkv, d, B, k,
                                                           seed=sum(lengths) + B)
    Q, K, V, dO = (bf16_to_f64(x) for x in (qb, kb, vb, gb))
    for s in range(len(lengths)):
        a, e = int(cu[s]), int(cu[s + 1])
        if e == a:
            continue
        ref_idx = oracle.select_blocks(Q[None, a:e], oracle.centroids(K[None, a:e], B), B, k)
        ndiff = int((gi[:, a:e] != ref_idx[0]).any(axis=-1).sum())
        assert ndiff == 0, f"sequence {s}: {ndiff} rows select other blocks than the oracle"
    ref = oracle.moba_backward_varlen(Q, K, V, dO, cu, B, k, scale)
    check_grads(got, ref)


def test_backward_varlen_equal_lengths_match_batch(moba):
    """Packed sequences of one length give the bits of the batched backward."""
    b, T, hq, hkv, d, B, k = 3, 2048, 8, 2, 128, 128, 4
    w = small_workload("eq_bwd", b, hq, hkv, d, T, B, k, "offset", seed=78)
    inp = make_inputs(w)
    q, kk, v = (dev(inp[x]) for x in "qkv")
    g = dev(make_output_grad(w))
    out, lse, idx = moba.forward(q, kk, v, B, k)
    a = moba.backward(q, kk, v, out, lse, idx, g, B, k)
    cu = np.arange(b + 1) * T
    o2, l2, i2 = moba.forward_varlen(q.reshape(b * T, hq, d), kk.reshape(b * T, hkv, d),
                                     v.reshape(b * T, hkv, d), cu, B, k)
    c = moba.backward_varlen(q.reshape(b * T, hq, d), kk.reshape(b * T, hkv, d),
                             v.reshape(b * T, hkv, d), o2, l2, i2, g.reshape(b * T, hq, d),
                             cu, B, k)
    torch.cuda.synchronize()
    for x, y in zip(a, c):
        assert torch.equal(x.reshape(y.shape), y)


def test_backward_varlen_one_kv_head_per_pass_is_identical(moba):
    lengths, hq, hkv, d, B, k = (1000, 2048, 37), 8, 4, 128, 128, 4
    _, _, full = packed_fwd_bwd(moba, lengths, hq, hkv, d, B, k, seed=9)
    total = sum(lengths)
    _, mn = moba.backward_varlen_workspace_bytes(len(lengths), total, max(lengths), hq, hkv,
                                                 d, B, k)
    ws = torch.empty(mn, dtype=torch.uint8, device="cuda")
    _, _, part = packed_fwd_bwd(moba, lengths, hq, hkv, d, B, k, seed=9, workspace=ws)
    for x, y in zip(full, part):
        assert np.array_equal(x, y)


def test_backward_varlen_rejects_bad_args(moba):
    lengths = (100, 50)
    qb, kb, vb, cu = packed_inputs(lengths, 2, 1, 64, 3)
    q, kk, v = dev(qb), dev(kb), dev(vb)
    out, lse, idx = moba.forward_varlen(q, kk, v, cu, 16, 2)
    for bad in ([0, 100], [1, 100, 150], [0, 120, 100, 150]):
        with pytest.raises(ValueError):
            moba.backward_varlen(q, kk, v, out, lse, idx, out, bad, 16, 2)
    with pytest.raises(ValueError):
        moba.backward_varlen(q, kk, v, out, lse[:, :10], idx, out, cu, 16, 2)
