"""The packed-sequence mix that bench.py times, against the float64 oracle: the
128K-token Llama-3.1-8B-shaped inputs cut into six requests of 40000, 30000, 25000,
20000, 10000 and 6072 tokens (B = 1024, top-8, every last block partial), each its own
MoBA problem (readings of packed sequences: each sequence routes and attends only
within itself, its block ids counted from its first token).

Forward: every idx row against the oracle's selection of its sequence (near-tie rule of
tests/parity_util.py), and sampled rows' out and lse.  Backward: the upstream gradient
is zero except on a sample R of rows, so dk and dv of every key are sums over R alone
and the oracle gives them in full; dq of R row by row, and dq = 0 exactly elsewhere.
Gradient tolerances are those of tests/test_gpu_backward.py.
"""
import sys

import numpy as np
import pytest

import oracle
from workloads import get_workload, make_inputs, make_output_grad, bf16_to_f64, to_torch_bf16
from parity_util import check_selection_row, compare_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

LENGTHS = (40000, 30000, 25000, 20000, 10000, 6072)
BLOCK, TOPK = 1024, 8
U = 2.0 ** -8
MAX_REL, MEAN_REL = 4 * U, 2 * U


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def moba():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_sparse_long_pool_amd as m
    return m


def test_mix_is_the_benchmarked_one():
    import bench
    assert tuple(bench.VARLEN_LENGTHS) == LENGTHS
    assert (bench.VARLEN_BLOCK, bench.VARLEN_TOPK) == (BLOCK, TOPK)


def rel_stats(name, got, ref):
    err = np.abs(got - ref)
    s = (float(err.max()) / max(float(np.abs(ref).max()), 1e-30),
         float(err.mean()) / max(float(np.abs(ref).mean()), 1e-30))
    say(f"       {name}: max rel {s[0]:.2e}, mean rel {s[1]:.2e}")
    assert s[0] <= MAX_REL and s[1] <= MEAN_REL, name
    return s


def test_packed_mix_forward_backward(moba):
    w = get_workload("llama8b_128k")
    assert sum(LENGTHS) == w.seqlen and w.batch == 1
    say("[mix] generating inputs")
    inp = make_inputs(w)
    g_bits = make_output_grad(w)[0]                       # [total, hq, d]
    total, hq, hkv, d = w.seqlen, w.hq, w.hkv, w.head_dim
    G, sc = hq // hkv, w.sm_scale
    cu = np.concatenate([[0], np.cumsum(LENGTHS)]).astype(np.int64)
    q = to_torch_bf16(inp["q"][0], "cuda")
    k = to_torch_bf16(inp["k"][0], "cuda")
    v = to_torch_bf16(inp["v"][0], "cuda")
    say("[mix] GPU forward")
    out, lse, idx = moba.forward_varlen(q, k, v, cu, BLOCK, TOPK, sc)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()                                 # [hq, total, k]
    Q, K, V = (bf16_to_f64(inp[x][0]) for x in "qkv")     # packed [total, heads, d]
    rng = np.random.default_rng(1024)
    R = []                                                 # (global t, h, selection)
    for s, (a, e) in enumerate(zip(cu[:-1], cu[1:])):
        a, e = int(a), int(e)
        n = e - a
        Qs, Ks, Vs = Q[None, a:e], K[None, a:e], V[None, a:e]
        C = oracle.centroids(Ks, BLOCK)
        ref = oracle.select_blocks(Qs, C, BLOCK, TOPK)[0]  # [hq, n, k]
        mism = np.argwhere((gi[:, a:e] != ref).any(axis=-1))
        exempt = 0
        for h, t in mism:
            sc_row = oracle.gate_scores_rows(Qs, C, BLOCK, [(0, int(t), int(h))])[0]
            ok, ex, _ = check_selection_row(gi[h, a + t], sc_row, int(t) // BLOCK, TOPK)
            assert ok, (s, int(h), int(t), gi[h, a + t].tolist(), ref[h, t].tolist())
            exempt += ex
        nb = -(-n // BLOCK)
        rows = {(0, n - 1, hq - 1), (0, 0, 0)}
        for c in range(nb):
            lo, hi = c * BLOCK, min((c + 1) * BLOCK, n)
            for t in (lo, hi - 1, int(rng.integers(lo, hi))):
                rows.add((0, t, int(rng.integers(hq))))
        rows = sorted(rows)
        ti = np.array([a + t for _, t, _ in rows])
        hi_ = np.array([h for _, _, h in rows])
        it, ih = torch.as_tensor(ti, device="cuda"), torch.as_tensor(hi_, device="cuda")
        stats = compare_rows(Qs, Ks, Vs, BLOCK, TOPK, sc, rows,
                             out[it, ih].float().cpu().numpy(), lse[ih, it].cpu().numpy(),
                             gi[hi_, ti], C=C)
        say(f"[mix] sequence {s} ({n} tokens): {len(mism)} idx rows differ, all near "
            f"ties ({exempt} exempt); {stats}")
        # rows of R: a random token and head per query block, where the GPU's selection
        # is the oracle's (the backward holds the selection fixed)
        for c in range(nb):
            t = int(rng.integers(c * BLOCK, min((c + 1) * BLOCK, n)))
            h = int(rng.integers(hq))
            S = [int(j) for j in ref[h, t] if j >= 0]
            if np.array_equal(gi[h, a + t], ref[h, t]):
                R.append((a, e, t, h, S))

    say(f"[mix] GPU backward with dout on {len(R)} rows only")
    sparse = np.zeros_like(g_bits)
    for a, _, t, h, _ in R:
        sparse[a + t, h] = g_bits[a + t, h]
    dq, dk, dv = moba.backward_varlen(q, k, v, out, lse, idx, to_torch_bf16(sparse, "cuda"),
                                      cu, BLOCK, TOPK, sc)
    torch.cuda.synchronize()
    in_r = torch.zeros((total, hq), dtype=torch.bool, device="cuda")
    for a, _, t, h, _ in R:
        in_r[a + t, h] = True
    assert bool((dq[~in_r] == 0).all()), "dq of a row without upstream gradient"
    dk = dk.float().cpu().numpy().astype(np.float64)
    dv = dv.float().cpu().numpy().astype(np.float64)
    rk, rv = np.zeros_like(dk), np.zeros_like(dv)
    touched = np.zeros(dk.shape[:2], bool)
    got, ref_dq = [], []
    for a, e, t, h, S in R:
        g = h // G
        keys = oracle.attended_keys(S, t, BLOCK, e - a)
        dqr, dkr, dvr = oracle.attend_row_grad(Q[a + t, h], K[a:e, g], V[a:e, g], keys, sc,
                                               bf16_to_f64(sparse[a + t, h]))
        rk[a + keys, g] += dkr
        rv[a + keys, g] += dvr
        touched[a + keys, g] = True
        got.append(dq[a + t, h].float().cpu().numpy())
        ref_dq.append(dqr)
    rel_stats("dq of R", np.array(got, np.float64), np.array(ref_dq))
    assert np.all(dk[~touched] == 0) and np.all(dv[~touched] == 0)
    for g in range(hkv):
        m = touched[:, g]
        rel_stats(f"dk g{g}", dk[m, g], rk[m, g])
        rel_stats(f"dv g{g}", dv[m, g], rv[m, g])
