"""The edges of the library's shape contract on the GPU, against the float64 oracle
through the C ABI:

* topk >= the number of blocks: every causal block is selected, so the layer is dense
  causal attention (README bullet "Seamlessly Transition between Full and Sparse
  Attention"); the library then runs the dense kernel and writes the all-blocks idx.
  Any topk is accepted there, e.g. topk = 40 over 32 blocks.  Forward (batched and
  packed) and backward.
* 33 to 64 history slots (topk up to 65 with more blocks than that): the gate's
  64-long running list and index entries with 6 slot bits.  Forward and backward.
* more than 2048 blocks (up to 8192): the index works over block ranges.
* dense causal attention for any seqlen (not a multiple of 16).

Tolerances are those of tests/parity_util.py (forward) and tests/test_gpu_backward.py
(gradients).
"""
import sys

import numpy as np
import pytest

import oracle
from workloads import (small_workload, make_inputs, make_output_grad, bf16_to_f64,
                       to_torch_bf16)
from parity_util import compare_rows, check_selection_row, sample_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

U = 2.0 ** -8


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


def all_rows_forward(moba, w):
    inp = make_inputs(w)
    out, lse, idx = moba.forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), w.block,
                                 w.topk, w.sm_scale)
    torch.cuda.synchronize()
    go, gl, gi = out.float().cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy()
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    rows = [(b, t, h) for b in range(w.batch) for t in range(w.seqlen) for h in range(w.hq)]
    stats = compare_rows(Q, K, V, w.block, w.topk, w.sm_scale, rows,
                         np.stack([go[b, t, h] for b, t, h in rows]),
                         np.array([gl[b, h, t] for b, t, h in rows]),
                         np.stack([gi[b, h, t] for b, t, h in rows]))
    say(f"       {stats}")
    return inp, gi


def check_grads(got, ref):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        err = np.abs(g - r)
        mx = float(err.max()) / max(float(np.abs(r).max()), 1e-30)
        mn = float(err.mean()) / max(float(np.abs(r).mean()), 1e-30)
        say(f"       {name}: max rel {mx:.2e}, mean rel {mn:.2e}")
        assert mx <= 4 * U and mn <= 2 * U, name


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("b,T,hq,hkv,d,B,k", [
    (1, 4096, 4, 2, 128, 128, 40),     # topk 40 over 32 blocks
    (2, 1000, 4, 1, 64, 128, 8),       # topk 8 = nb (partial last block), batch 2
    (1, 777, 8, 2, 128, 16, 200),      # 49 blocks of 16, topk 200, seqlen % 16 != 0
])
def test_all_blocks_selected_is_dense(moba, b, T, hq, hkv, d, B, k):
    w = small_workload("allblk", b, hq, hkv, d, T, B, k, "offset", seed=T + k)
    say(f"[contract] topk >= nb: b={b} T={T} hq={hq} hkv={hkv} d={d} B={B} k={k}")
    full, mn = moba.workspace_bytes(b, T, hq, hkv, d, B, k)
    assert full == mn == 256
    inp, gi = all_rows_forward(moba, w)
    c = np.arange(T) // B
    want = np.where(np.arange(k)[None, :] <= c[:, None], np.arange(k)[None, :], -1)
    assert np.array_equal(gi, np.broadcast_to(want, gi.shape))
    # backward of the same layer: the dense causal backward
    g_bits = make_output_grad(w)
    q, kk, v = (dev(inp[x]) for x in "qkv")
    out, lse, idx = moba.forward(q, kk, v, B, k, w.sm_scale)
    dq, dk, dv = moba.backward(q, kk, v, out, lse, idx, dev(g_bits), B, k, w.sm_scale)
    torch.cuda.synchronize()
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    ref = oracle.moba_backward(Q, K, V, bf16_to_f64(g_bits), B, k, w.sm_scale)
    check_grads((f64(dq), f64(dk), f64(dv)), ref)


def test_all_blocks_selected_packed(moba):
    """Packed sequences whose longest has no more blocks than topk: dense per sequence."""
    lengths, hq, hkv, d, B, k = (300, 1024, 17, 700), 4, 2, 128, 128, 8
    r = np.random.default_rng(5)
    from workloads import f32_to_bf16_bits
    total = sum(lengths)
    qb, kb, vb = (f32_to_bf16_bits(r.standard_normal((total, h, d), dtype=np.float32))
                  for h in (hq, hkv, hkv))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    sc = 1.0 / np.sqrt(d)
    out, lse, idx = moba.forward_varlen(dev(qb), dev(kb), dev(vb), cu, B, k, sc)
    torch.cuda.synchronize()
    Q, K, V = (bf16_to_f64(x) for x in (qb, kb, vb))
    ro, rl, ri = oracle.moba_forward_varlen(Q, K, V, cu, B, k, sc)
    assert np.array_equal(idx.cpu().numpy(), ri)
    d_o = np.abs(out.float().cpu().numpy() - ro)
    assert d_o.max() <= 2e-2 and d_o.mean() <= 2e-3
    assert np.abs(lse.cpu().numpy() - rl).max() <= 1e-3
    g = r.standard_normal((total, hq, d), dtype=np.float32)
    gb = f32_to_bf16_bits(g)
    dq, dk, dv = moba.backward_varlen(dev(qb), dev(kb), dev(vb), out, lse, idx, dev(gb), cu,
                                      B, k, sc)
    torch.cuda.synchronize()
    ref = oracle.moba_backward_varlen(Q, K, V, bf16_to_f64(gb), cu, B, k, sc)
    check_grads((f64(dq), f64(dk), f64(dv)), ref)


@pytest.mark.parametrize("b,T,hq,hkv,d,B,k", [
    (1, 6144, 4, 2, 128, 128, 40),     # 39 history slots of up to 47 candidates
    (1, 4480, 2, 1, 64, 64, 65),       # 64 history slots (the most), 70 blocks
])
def test_many_history_slots(moba, b, T, hq, hkv, d, B, k):
    w = small_workload("slots", b, hq, hkv, d, T, B, k, "offset", seed=T + 3 * k)
    say(f"[contract] {k - 1} history slots: b={b} T={T} hq={hq} hkv={hkv} d={d} B={B}")
    inp, _ = all_rows_forward(moba, w)
    g_bits = make_output_grad(w)
    q, kk, v = (dev(inp[x]) for x in "qkv")
    out, lse, idx = moba.forward(q, kk, v, B, k, w.sm_scale)
    dq, dk, dv = moba.backward(q, kk, v, out, lse, idx, dev(g_bits), B, k, w.sm_scale)
    torch.cuda.synchronize()
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    gi = idx.cpu().numpy()
    ref_idx = oracle.select_blocks(Q, oracle.centroids(K, B), B, k)
    if np.array_equal(gi, ref_idx):          # the gradients hold the selection fixed
        ref = oracle.moba_backward(Q, K, V, bf16_to_f64(g_bits), B, k, w.sm_scale)
    else:                                     # near ties: the GPU's own (valid) selection
        ref = oracle.moba_backward(Q, K, V, bf16_to_f64(g_bits), B, k, w.sm_scale, idx=gi)
    check_grads((f64(dq), f64(dk), f64(dv)), ref)


def test_more_than_2048_blocks_every_row(moba):
    """3001 blocks of 16 tokens (the last one partial): every idx row against the
    oracle's selection, sampled rows' out and lse."""
    w = small_workload("nb3001", 1, 2, 1, 64, 16 * 3000 + 5, 16, 8, "offset", seed=41)
    assert w.num_blocks == 3001
    inp = make_inputs(w)
    out, lse, idx = moba.forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), w.block,
                                 w.topk, w.sm_scale)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    C = oracle.centroids(K, w.block)
    say("[contract] 3001 blocks: oracle selection of every row")
    ref = oracle.select_blocks(Q, C, w.block, w.topk)
    mism = np.argwhere((gi != ref).any(axis=-1))
    for bi, h, t in mism:
        s = oracle.gate_scores_rows(Q, C, w.block, [(bi, t, h)])[0]
        ok, ex, _ = check_selection_row(gi[bi, h, t], s, t // w.block, w.topk)
        assert ok and ex, (bi, h, t)
    rows = sample_rows(1, w.seqlen, w.hq, w.block, per_block=0, seed=7,
                       extra=[(0, w.seqlen - 1, 1), (0, 0, 0)])[::8]
    bi_, t_, h_ = (np.array(x) for x in zip(*rows))
    ib, it, ih = (torch.as_tensor(x, device="cuda") for x in (bi_, t_, h_))
    stats = compare_rows(Q, K, V, w.block, w.topk, w.sm_scale, rows,
                         out[ib, it, ih].float().cpu().numpy(), lse[ib, ih, it].cpu().numpy(),
                         gi[bi_, h_, t_], C=C)
    say(f"       {len(mism)} rows differ, all near ties; {stats}")


def test_4096_blocks_of_128(moba):
    """512K tokens in 4096 blocks of 128 (two query heads of one kv-head, d = 64, top-8):
    every idx row's properties, and sampled rows against the oracle."""
    w = small_workload("nb4096", 1, 2, 1, 64, 524288, 128, 8, "offset", seed=43)
    assert w.num_blocks == 4096
    inp = make_inputs(w)
    out, lse, idx = moba.forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), w.block,
                                 w.topk, w.sm_scale)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    c = (np.arange(w.seqlen) // w.block)[None, None, :]
    n_valid = np.minimum(w.topk, c + 1)
    valid = np.arange(w.topk)[None, None, None, :] < n_valid[..., None]
    assert np.all(np.where(valid, gi >= 0, gi == -1))
    assert np.all(np.where(valid, gi <= c[..., None], True))
    assert np.all(np.where(valid[..., 1:], np.diff(gi, axis=-1) > 0, True))
    last = np.take_along_axis(gi, (n_valid - 1)[..., None].repeat(w.hq, 1), -1)[..., 0]
    assert np.all(last == c)
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    rows = sample_rows(1, w.seqlen, w.hq, w.block, per_block=0, seed=9,
                       extra=[(0, w.seqlen - 1, 1), (0, 0, 0)])[::16]
    bi_, t_, h_ = (np.array(x) for x in zip(*rows))
    ib, it, ih = (torch.as_tensor(x, device="cuda") for x in (bi_, t_, h_))
    stats = compare_rows(Q, K, V, w.block, w.topk, w.sm_scale, rows,
                         out[ib, it, ih].float().cpu().numpy(), lse[ib, ih, it].cpu().numpy(),
                         gi[bi_, h_, t_])
    say(f"[contract] 4096 blocks: {stats}")


@pytest.mark.parametrize("b,hq,hkv,d,T", [(1, 4, 2, 128, 1000), (2, 2, 1, 64, 37),
                                           (1, 2, 2, 128, 1)])
def test_dense_forward_any_seqlen(moba, b, hq, hkv, d, T):
    w = small_workload("dense_any", b, hq, hkv, d, T, 16, 1, "iid", seed=T)
    inp = make_inputs(w)
    out, lse = moba.dense_forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]))
    torch.cuda.synchronize()
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    ro, rl, _, _ = oracle.moba_forward(Q, K, V, T, 1, w.sm_scale)   # one block: dense
    d_o = np.abs(out.float().cpu().numpy() - ro)
    assert d_o.max() <= 2e-2 and d_o.mean() <= 2e-3
    assert np.abs(lse.cpu().numpy() - rl).max() <= 1e-3
