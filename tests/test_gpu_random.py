"""Randomly drawn shapes (seeded, the same every run) through the forward, the
backward, the packed forward and the decode, every row or element against the
oracle.  They complement the hand-picked cases with combinations nobody chose: odd
lengths, block sizes from 16 to 256 (and 256 to 2048 for the chained history kernel),
G = 1 to 8, top-k from 1 to 13 (6 to 17 over many blocks of at most 128 keys), d = 64
and 128.
Bars are those of tests/parity_util.py (forward), tests/test_gpu_backward.py
(backward) and tests/test_gpu_decode.py (decode).
"""
import sys

import numpy as np
import pytest

import oracle
from workloads import small_workload, make_inputs, make_output_grad, bf16_to_f64
from parity_util import compare_rows, check_selection_row
from test_gpu_backward import check_grads, f64
from test_gpu_varlen import check_packed
from test_gpu_decode import bits, check

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


def dev(b):
    from workloads import to_torch_bf16
    return to_torch_bf16(b, "cuda")


def draw(seed, groups=(1, 2, 3, 4, 8), max_rows=20000):
    """(b, T, hq, hkv, d, B, k) with at most max_rows query rows."""
    r = np.random.default_rng(seed)
    d = int(r.choice([64, 128]))
    G = int(r.choice(groups))
    hkv = int(r.choice([1, 2]))
    hq = G * hkv
    B = 16 * int(r.integers(1, 17))
    k = int(r.integers(1, 14))
    b = int(r.choice([1, 2]))
    T = int(r.integers(1, max(2, min(max_rows // (b * hq), 40 * B))))
    return b, T, hq, hkv, d, B, k


@pytest.mark.parametrize("seed", range(100, 112))
def test_forward_random_shape(moba, seed):
    b, T, hq, hkv, d, B, k = draw(seed)
    say(f"[random fwd] seed={seed}: b={b} T={T} hq={hq} hkv={hkv} d={d} B={B} k={k}")
    w = small_workload("rnd", b, hq, hkv, d, T, B, k, "offset", seed=seed)
    inp = make_inputs(w)
    out, lse, idx = moba.forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), B, k)
    torch.cuda.synchronize()
    go, gl, gi = out.float().cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy()
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    rows = [(bi, t, h) for bi in range(b) for t in range(T) for h in range(hq)]
    st = compare_rows(Q, K, V, B, k, w.sm_scale, rows,
                      np.stack([go[bi, t, h] for bi, t, h in rows]),
                      np.array([gl[bi, h, t] for bi, t, h in rows]),
                      np.stack([gi[bi, h, t] for bi, t, h in rows]))
    say(f"       {st}")


def draw_resident(seed, max_rows=24000):
    """(b, T, hq, hkv, d, B, k) with blocks of at most 128 keys (the history kernel that
    holds the block in LDS, with its paired loads and stores), top-6 to top-17 and a
    ragged length of at least k + 2 blocks, up to 160 blocks: rows with 5 to 16 history
    parts, index tiles with odd tails, and (with at least 8 history slots over many
    blocks) the index's staged scatter."""
    r = np.random.default_rng(seed)
    d = int(r.choice([64, 128]))
    G = int(r.choice([1, 2, 4, 8]))
    hkv = int(r.choice([1, 2]))
    hq = G * hkv
    B = 16 * int(r.integers(1, 9))
    k = int(r.integers(6, 18))
    b = int(r.choice([1, 2]))
    lo = (k + 2) * B
    hi = max(min(max_rows // (b * hq), 160 * B), lo + 2)
    T = int(r.integers(lo, hi))
    return b, T, hq, hkv, d, B, k


@pytest.mark.parametrize("seed", range(400, 410))
def test_forward_random_small_blocks(moba, seed):
    b, T, hq, hkv, d, B, k = draw_resident(seed)
    nb = -(-T // B)
    staged = k - 1 >= 8 and 256 * (k - 1) < 32 * nb
    say(f"[random small-block fwd] seed={seed}: b={b} T={T} hq={hq} hkv={hkv} d={d} "
        f"B={B} k={k} nb={nb} staged_index={staged}")
    w = small_workload("rnd_res", b, hq, hkv, d, T, B, k, "offset", seed=seed)
    inp = make_inputs(w)
    out, lse, idx = moba.forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), B, k)
    torch.cuda.synchronize()
    go, gl, gi = out.float().cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy()
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    rows = [(bi, t, h) for bi in range(b) for t in range(T) for h in range(hq)]
    st = compare_rows(Q, K, V, B, k, w.sm_scale, rows,
                      np.stack([go[bi, t, h] for bi, t, h in rows]),
                      np.array([gl[bi, h, t] for bi, t, h in rows]),
                      np.stack([gi[bi, h, t] for bi, t, h in rows]))
    say(f"       {st}")


def draw_chained(seed, max_rows=24000):
    """(b, T, hq, hkv, d, B, k) with blocks of 256 to 2048 keys (multiples of 64: the
    persistent chained history kernel fed by its tile queue), more than k + 1 blocks
    (so the rows of the later blocks choose among their history blocks) and a ragged
    T; the launches range from fewer tiles than workgroups to several per workgroup."""
    r = np.random.default_rng(seed)
    d = int(r.choice([64, 128]))
    G = int(r.choice([1, 2, 4]))
    hkv = int(r.choice([1, 2]))
    hq = G * hkv
    k = int(r.integers(2, 7))
    bmax = max(4, min(32, max_rows // (hq * (k + 2) * 64)))
    B = 64 * int(r.integers(4, bmax + 1))
    lo = (k + 1) * B + 1
    T = int(r.integers(lo, max(lo + 1, min(max_rows // hq, (k + 5) * B))))
    return 1, T, hq, hkv, d, B, k


@pytest.mark.parametrize("seed", range(300, 306))
def test_forward_random_chained_history(moba, seed):
    b, T, hq, hkv, d, B, k = draw_chained(seed)
    say(f"[random chained fwd] seed={seed}: b={b} T={T} hq={hq} hkv={hkv} d={d} B={B} k={k}")
    w = small_workload("rndc", b, hq, hkv, d, T, B, k, "offset", seed=seed)
    inp = make_inputs(w)
    out, lse, idx = moba.forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), B, k)
    torch.cuda.synchronize()
    go, gl, gi = out.float().cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy()
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    rows = [(bi, t, h) for bi in range(b) for t in range(T) for h in range(hq)]
    st = compare_rows(Q, K, V, B, k, w.sm_scale, rows,
                      np.stack([go[bi, t, h] for bi, t, h in rows]),
                      np.array([gl[bi, h, t] for bi, t, h in rows]),
                      np.stack([gi[bi, h, t] for bi, t, h in rows]))
    say(f"       {st}")


@pytest.mark.parametrize("seed", range(200, 206))
def test_backward_random_shape(moba, seed):
    """The oracle's gradients with the GPU's selection held fixed (each idx row checked
    valid first), so near ties in the gate cannot make the comparison fail."""
    b, T, hq, hkv, d, B, k = draw(seed, groups=(1, 2, 3, 4, 5, 7, 8), max_rows=6000)
    say(f"[random bwd] seed={seed}: b={b} T={T} hq={hq} hkv={hkv} d={d} B={B} k={k}")
    w = small_workload("rndb", b, hq, hkv, d, T, B, k, "offset", seed=seed)
    inp = make_inputs(w)
    g_bits = make_output_grad(w)
    q, kk, v = (dev(inp[x]) for x in "qkv")
    out, lse, idx = moba.forward(q, kk, v, B, k)
    dq, dk, dv = moba.backward(q, kk, v, out, lse, idx, dev(g_bits), B, k)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    C = oracle.centroids(K, B)
    for bi in range(b):
        for h in range(hq):
            rows = [(bi, t, h) for t in range(T)]
            scores = oracle.gate_scores_rows(Q, C, B, rows)
            for t in range(T):
                ok, _, _ = check_selection_row(gi[bi, h, t], scores[t], t // B, k)
                assert ok, (bi, h, t, gi[bi, h, t].tolist())
    ref = oracle.moba_backward(Q, K, V, bf16_to_f64(g_bits), B, k, w.sm_scale, idx=gi)
    check_grads((f64(dq), f64(dk), f64(dv)), ref)


@pytest.mark.parametrize("seed", range(300, 306))
def test_varlen_random_mix(moba, seed):
    r = np.random.default_rng(seed)
    nseq = int(r.integers(1, 6))
    lengths = tuple(int(x) for x in r.integers(1, 900, nseq))
    G = int(r.choice([1, 2, 4, 8]))
    hkv = int(r.choice([1, 2]))
    d = int(r.choice([64, 128]))
    B = 16 * int(r.integers(1, 9))
    k = int(r.integers(1, 10))
    check_packed(moba, lengths, G * hkv, hkv, d, B, k, seed=seed, label=f"random seed {seed}")


@pytest.mark.parametrize("seed", range(400, 406))
def test_decode_random_shape(moba, seed):
    r = np.random.default_rng(seed)
    G = int(r.choice([1, 2, 4, 8]))
    hkv = int(r.choice([1, 2, 8]))
    d = int(r.choice([64, 128]))
    b = int(r.choice([1, 2]))
    n = int(r.integers(1, 64 // G + 1))      # up to two 32-row tiles
    Tk = int(r.integers(n, 6000))
    say(f"[random decode] seed={seed}: b={b} n={n} Tk={Tk} hq={G * hkv} hkv={hkv} d={d}")
    qb, kb, vb = bits(seed, b, n, G * hkv, d), bits(seed + 1, b, Tk, hkv, d), bits(seed + 2, b, Tk, hkv, d)
    sc = 1.0 / np.sqrt(d)
    out, lse = moba.decode(dev(qb), dev(kb), dev(vb), sc)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_attention(bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb), sc)
    check(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, "all rows")
