"""Partial last blocks and packed variable-length sequences on the GPU, against the
float64 oracle (which runs the definition once per sequence; pinned by
tests/test_oracle_varlen.py).  Tolerances and the near-tie rule are those of
tests/parity_util.py.
"""
import sys

import numpy as np
import pytest

import oracle
from workloads import (small_workload, make_inputs, bf16_to_f64, to_torch_bf16,
                       f32_to_bf16_bits)
from parity_util import compare_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def moba():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_sparse_long_pool_amd as m
    return m


def dev(bits):
    return to_torch_bf16(bits, "cuda")


@pytest.mark.parametrize("b,T,hq,hkv,d,B,k", [
    (1, 1000, 4, 2, 128, 128, 4),      # 7 whole blocks and 104 tokens
    (2, 2100, 8, 2, 64, 256, 3),       # 52-token tail, batch 2
    (1, 300, 2, 1, 128, 256, 2),       # one whole block and a 44-token tail
    (1, 1040, 8, 1, 128, 16, 33),      # B = 16 with a whole last block (control)
    (1, 770, 4, 4, 64, 48, 5),         # B = 48, a 2-token tail
])
def test_ragged_seqlen_all_rows(moba, b, T, hq, hkv, d, B, k):
    """seqlen not a multiple of block: every row against the oracle."""
    w = small_workload("ragged", b, hq, hkv, d, T, B, k, "offset", seed=T + B)
    say(f"[ragged] b={b} T={T} hq={hq} hkv={hkv} d={d} B={B} k={k}")
    inp = make_inputs(w)
    out, lse, idx = moba.forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), B, k)
    torch.cuda.synchronize()
    go = out.float().cpu().numpy()
    gl = lse.cpu().numpy()
    gi = idx.cpu().numpy()
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    rows = [(bi, t, h) for bi in range(b) for t in range(T) for h in range(hq)]
    stats = compare_rows(Q, K, V, B, k, w.sm_scale, rows,
                         np.stack([go[bi, t, h] for bi, t, h in rows]),
                         np.array([gl[bi, h, t] for bi, t, h in rows]),
                         np.stack([gi[bi, h, t] for bi, t, h in rows]))
    say(f"       {stats}")


def packed_inputs(lengths, hq, hkv, d, seed, offset=0.5, B=None):
    """Packed bf16 Q/K/V: N(0,1), plus a per-(sequence, block, kv-head) key offset so
    that gate scores separate (as the offset recipe does for one sequence)."""
    r = np.random.default_rng(seed)
    total = int(sum(lengths))
    Q = r.standard_normal((total, hq, d), dtype=np.float32)
    K = r.standard_normal((total, hkv, d), dtype=np.float32)
    V = r.standard_normal((total, hkv, d), dtype=np.float32)
    if B is not None:
        a = 0
        for n in lengths:
            for j0 in range(0, n, B):
                K[a + j0:a + min(j0 + B, n)] += offset * r.standard_normal((1, hkv, d),
                                                                           dtype=np.float32)
            a += n
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return f32_to_bf16_bits(Q), f32_to_bf16_bits(K), f32_to_bf16_bits(V), cu


def check_packed(moba, lengths, hq, hkv, d, B, k, seed, label):
    say(f"[varlen] {label}: lengths={lengths} hq={hq} hkv={hkv} d={d} B={B} k={k}")
    qb, kb, vb, cu = packed_inputs(lengths, hq, hkv, d, seed, B=B)
    scale = 1.0 / np.sqrt(d)
    out, lse, idx = moba.forward_varlen(dev(qb), dev(kb), dev(vb), cu, B, k, scale)
    torch.cuda.synchronize()
    go = out.float().cpu().numpy()
    gl = lse.cpu().numpy()
    gi = idx.cpu().numpy()
    Q, K, V = bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb)
    worst = {}
    for s in range(len(lengths)):
        a, e = int(cu[s]), int(cu[s + 1])
        if e == a:
            continue
        rows = [(0, t, h) for t in range(e - a) for h in range(hq)]
        st = compare_rows(Q[None, a:e], K[None, a:e], V[None, a:e], B, k, scale, rows,
                          np.stack([go[a + t, h] for _, t, h in rows]),
                          np.array([gl[h, a + t] for _, t, h in rows]),
                          np.stack([gi[h, a + t] for _, t, h in rows]))
        for key in ("out_max", "out_mean", "lse_max"):
            worst[key] = max(worst.get(key, 0.0), st[key])
    say(f"       worst over sequences: {worst}")
    return go, gl, gi


@pytest.mark.parametrize("lengths,hq,hkv,d,B,k", [
    ((1000, 37, 2048, 513, 1), 8, 2, 128, 128, 4),
    ((4096, 4096), 4, 1, 64, 256, 3),
    ((300, 1500, 64, 900), 8, 8, 128, 64, 9),
    ((2500,), 4, 2, 128, 512, 2),
    ((16, 17, 15, 2000, 33), 16, 2, 128, 16, 6),
    # top-12 over up to 94 blocks of 32 keys: the index stages each chunk's entries
    ((3000, 700, 2500, 45), 4, 2, 64, 32, 12),
])
def test_varlen_all_rows(moba, lengths, hq, hkv, d, B, k):
    check_packed(moba, lengths, hq, hkv, d, B, k, seed=sum(lengths) + B, label="all rows")


def test_varlen_equal_lengths_match_batch(moba):
    """Packed sequences of one length give the bits of the batched entry point."""
    b, T, hq, hkv, d, B, k = 3, 2048, 8, 2, 128, 128, 4
    w = small_workload("eq", b, hq, hkv, d, T, B, k, "offset", seed=77)
    inp = make_inputs(w)
    q, kk, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    out, lse, idx = moba.forward(q, kk, v, B, k)
    cu = np.arange(b + 1) * T
    o2, l2, i2 = moba.forward_varlen(q.reshape(b * T, hq, d), kk.reshape(b * T, hkv, d),
                                     v.reshape(b * T, hkv, d), cu, B, k)
    torch.cuda.synchronize()
    assert torch.equal(out.reshape(b * T, hq, d), o2)
    assert torch.equal(lse.permute(1, 0, 2).reshape(hq, b * T), l2)
    assert torch.equal(idx.permute(1, 0, 2, 3).reshape(hq, b * T, k), i2)


def test_varlen_one_kv_head_per_pass_is_identical(moba):
    lengths = (1000, 2048, 37)
    qb, kb, vb, cu = packed_inputs(lengths, 8, 4, 128, 5, B=128)
    q, k, v = dev(qb), dev(kb), dev(vb)
    a = moba.forward_varlen(q, k, v, cu, 128, 4)
    _, mn = moba.varlen_workspace_bytes(len(lengths), int(cu[-1]), max(lengths), 8, 4, 128,
                                        128, 4)
    ws = torch.empty(mn, dtype=torch.uint8, device="cuda")
    b = moba.forward_varlen(q, k, v, cu, 128, 4, workspace=ws)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_varlen_rejects_bad_cu_seqlens(moba):
    qb, kb, vb, cu = packed_inputs((100, 50), 2, 1, 64, 3)
    q, k, v = dev(qb), dev(kb), dev(vb)
    for bad in ([0, 100], [1, 100, 150], [0, 120, 100, 150]):
        with pytest.raises(ValueError):
            moba.forward_varlen(q, k, v, bad, 16, 2)
