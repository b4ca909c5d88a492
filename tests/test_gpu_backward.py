"""Parity of the HIP backward (through the C ABI) with the float64 oracle, on the GPU.

The GPU forward's selection must equal the oracle's selection bit for bit on these
inputs (each case is drawn so that no row sits at a near-tie, and the test checks it),
so the oracle's gradients, computed from its own selection, are the reference.

Tolerance.  The HIP path rounds P and dS to bfloat16 before the products that use
them (relative error <= u = 2^-8 each), accumulates in float32, builds D from the bf16
forward output, and rounds dq, dk, dv to bfloat16 (<= u relative, u/2 on average).
The operand roundings add errors of random sign, about u/sqrt(3) times the root sum of
squares of the summed terms; for dq and dk those terms cancel strongly (the dS of a
row sum to zero), so the error is a larger fraction of the result than one rounding.
Bound used: mean |err| <= 2u * mean |g| and max |err| <= 4u * max |g|.
"""
import sys

import numpy as np
import pytest

import oracle
from workloads import (small_workload, get_workload, make_inputs, make_output_grad,
                       bf16_to_f64, to_torch_bf16)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

U = 2.0 ** -8                 # bf16 unit roundoff
MAX_REL = 4 * U               # max |err| / max |g|
MEAN_REL = 2 * U               # mean |err| / mean |g|


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


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def gpu_fwd_bwd(moba, w, inp, dout_bits, **kw):
    q, k, v = (dev(inp[x]) for x in "qkv")
    out, lse, idx = moba.forward(q, k, v, w.block, w.topk, w.sm_scale)
    dq, dk, dv = moba.backward(q, k, v, out, lse, idx, dev(dout_bits), w.block, w.topk,
                               w.sm_scale, **kw)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), f64(dq), f64(dk), f64(dv)


def grad_stats(name, got, ref):
    err = np.abs(got - ref)
    s = {"max_err": float(err.max()), "max_ref": float(np.abs(ref).max()),
         "mean_err": float(err.mean()), "mean_ref": float(np.abs(ref).mean())}
    s["max_rel"] = s["max_err"] / max(s["max_ref"], 1e-30)
    s["mean_rel"] = s["mean_err"] / max(s["mean_ref"], 1e-30)
    say(f"       {name}: max_err {s['max_err']:.3e} (max|g| {s['max_ref']:.3e}, "
        f"rel {s['max_rel']:.2e})  mean_err {s['mean_err']:.3e} (mean|g| "
        f"{s['mean_ref']:.3e}, rel {s['mean_rel']:.2e})")
    return s


def check_grads(got, ref):
    stats = {name: grad_stats(name, g, r) for name, g, r in zip(("dq", "dk", "dv"), got, ref)}
    for name, s in stats.items():
        assert s["max_rel"] <= MAX_REL, f"{name}: max error {s['max_err']:.3e}"
        assert s["mean_rel"] <= MEAN_REL, f"{name}: mean error {s['mean_err']:.3e}"


SMALL = [
    # name, b, hq, hkv, d, T, B, topk, recipe, seed
    ("tiny_d64", 1, 2, 1, 64, 1024, 128, 4, "offset", 31),
    ("gqa4_d128", 1, 8, 2, 128, 2048, 128, 4, "offset", 32),
    ("b2_g2_d64", 2, 4, 2, 64, 1024, 64, 5, "offset", 33),
    ("blk48_ragged", 1, 4, 1, 64, 1536, 48, 3, "offset", 34),
    ("blk16_k9", 1, 2, 2, 128, 512, 16, 9, "offset", 35),
    ("topk1_no_history", 1, 4, 2, 128, 1024, 256, 1, "iid", 36),
    ("g8", 1, 8, 1, 128, 1024, 128, 3, "offset", 37),
    ("dense_k_over_nb", 1, 2, 1, 128, 768, 256, 9, "iid", 38),
    ("blk320_tail", 1, 2, 1, 128, 1280, 320, 3, "offset", 39),
    # G not dividing the eight waves of the dQ kernel, and G above eight
    ("g3", 1, 6, 2, 128, 1024, 128, 4, "offset", 43),
    ("g7_b2", 2, 7, 1, 64, 768, 128, 3, "offset", 44),
    ("g12", 1, 12, 1, 128, 512, 64, 5, "offset", 45),
    ("g16_d64", 1, 16, 1, 64, 512, 128, 3, "offset", 46),
    # top-16 over 125 blocks of 32 keys: the index stages each chunk's entries in LDS
    ("k16_b32_staged", 1, 2, 1, 64, 4000, 32, 16, "offset", 47),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_backward_small_all_elements(moba, case):
    name, b, hq, hkv, d, T, B, k, recipe, seed = case
    w = small_workload(name, b, hq, hkv, d, T, B, k, recipe, seed)
    say(f"[bwd] {name}: b={b} T={T} hq={hq} hkv={hkv} d={d} B={B} k={k}")
    inp = make_inputs(w)
    g_bits = make_output_grad(w)
    gi, dq, dk, dv = gpu_fwd_bwd(moba, w, inp, g_bits)
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    ref_idx = oracle.select_blocks(Q, oracle.centroids(K, B), B, k)
    ndiff = int((gi != ref_idx).any(axis=-1).sum())
    assert ndiff == 0, f"{ndiff} rows select other blocks than the oracle; pick another seed"
    ref = oracle.moba_backward(Q, K, V, bf16_to_f64(g_bits), B, k, w.sm_scale)
    check_grads((dq, dk, dv), ref)


def test_backward_zero_grad_is_zero(moba):
    """dout = 0 gives exactly zero gradients."""
    w = small_workload("zg", 1, 4, 2, 128, 1024, 128, 4, "offset", 40)
    inp = make_inputs(w)
    _, dq, dk, dv = gpu_fwd_bwd(moba, w, inp, np.zeros_like(inp["q"]))
    assert not dq.any() and not dk.any() and not dv.any()


def test_backward_deterministic_and_chunked(moba):
    """Two runs give identical bits, and a workspace that forces one kv-head per pass
    gives the same bits as all heads at once."""
    w = small_workload("det", 1, 8, 4, 128, 2048, 128, 5, "offset", 41)
    inp = make_inputs(w)
    g_bits = make_output_grad(w)
    a = gpu_fwd_bwd(moba, w, inp, g_bits)
    bb = gpu_fwd_bwd(moba, w, inp, g_bits)
    _, mn = moba.backward_workspace_bytes(1, w.seqlen, w.hq, w.hkv, w.head_dim, w.block,
                                          w.topk)
    ws = torch.empty(mn, dtype=torch.uint8, device="cuda")
    c = gpu_fwd_bwd(moba, w, inp, g_bits, workspace=ws)
    for x, y, z in zip(a[1:], bb[1:], c[1:]):
        assert np.array_equal(x, y) and np.array_equal(x, z)


def test_backward_rejects_bad_args(moba):
    w = small_workload("bad", 1, 4, 2, 128, 1024, 128, 4, "offset", 42)
    inp = make_inputs(w)
    q, k, v = (dev(inp[x]) for x in "qkv")
    out, lse, idx = moba.forward(q, k, v, w.block, w.topk)
    full, mn = moba.backward_workspace_bytes(1, 1024, 4, 2, 128, 128, 4)
    assert 0 < mn <= full
    small = torch.empty(mn // 2, dtype=torch.uint8, device="cuda")
    with pytest.raises(moba.MobaError):
        moba.backward(q, k, v, out, lse, idx, out, w.block, w.topk, workspace=small)
    # any number of query heads per kv-head is supported
    assert moba.backward_workspace_bytes(1, 1024, 6, 2, 128, 128, 4)[0] > 0


def test_backward_32k_sampled_rows_and_sums(moba):
    """Llama-3.1-8B heads at 32K (B=512, top-3): dq of sampled rows against the oracle
    row by row, the keys of the last block (attended only by their own block's rows)
    against the oracle in full, and for every kv-head the sums that hold at any size:
    sum_u dv_u = sum over its query rows of dout, sum_u dk_u = 0."""
    w = get_workload("llama8b_32k")
    say("[bwd] llama8b_32k: generating inputs")
    inp = make_inputs(w)
    g_bits = make_output_grad(w)
    say("[bwd] llama8b_32k: running the GPU path")
    gi, dq, dk, dv = gpu_fwd_bwd(moba, w, inp, g_bits)
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    dO = bf16_to_f64(g_bits)
    B, T, G, sc = w.block, w.seqlen, w.hq // w.hkv, w.sm_scale
    C = oracle.centroids(K, B)
    rng = np.random.default_rng(7)
    say("[bwd] llama8b_32k: sampled dq rows")
    ts = np.concatenate([rng.integers(0, T, 96), [0, B - 1, B, T - 1]])
    got, ref = [], []
    for t in ts:
        for h in rng.choice(w.hq, 2, replace=False):
            _, _, sels, _ = oracle.moba_rows(Q, K, V, B, w.topk, sc, [(0, int(t), int(h))], C)
            if not np.array_equal(np.asarray(sels[0]), gi[0, h, t][gi[0, h, t] >= 0]):
                continue   # a near-tie row: its selection differs, skip it
            keys = oracle.attended_keys(sels[0], int(t), B, T)
            r, _, _ = oracle.attend_row_grad(Q[0, t, h], K[0, :, h // G], V[0, :, h // G],
                                             keys, sc, dO[0, t, h])
            got.append(dq[0, t, h])
            ref.append(r)
    assert len(got) >= 150
    s = grad_stats("dq rows", np.array(got), np.array(ref))
    assert s["max_rel"] <= MAX_REL and s["mean_rel"] <= MEAN_REL
    say("[bwd] llama8b_32k: last block dk, dv")
    j = w.num_blocks - 1
    keys0 = np.arange(j * B, T)
    checked = 0
    for g in range(w.hkv):
        rows = [(0, t, h) for h in range(g * G, (g + 1) * G) for t in range(j * B, T)]
        _, _, sels, _ = oracle.moba_rows(Q, K, V, B, w.topk, sc, rows, C)
        if any(not np.array_equal(np.asarray(S), gi[0, h, t][gi[0, h, t] >= 0])
               for (_, t, h), S in zip(rows, sels)):
            say(f"       kv-head {g}: a near-tie row selects differently, skipped")
            continue
        rk = np.zeros((B, w.head_dim))
        rv = np.zeros((B, w.head_dim))
        for (_, t, h), S in zip(rows, sels):
            keys = oracle.attended_keys(S, t, B, T)
            _, dkr, dvr = oracle.attend_row_grad(Q[0, t, h], K[0, :, g], V[0, :, g],
                                                 keys, sc, dO[0, t, h])
            m = keys >= j * B
            rk[keys[m] - j * B] += dkr[m]
            rv[keys[m] - j * B] += dvr[m]
        sk = grad_stats(f"dk last block g{g}", dk[0, keys0, g], rk)
        sv = grad_stats(f"dv last block g{g}", dv[0, keys0, g], rv)
        for s in (sk, sv):
            assert s["max_rel"] <= MAX_REL and s["mean_rel"] <= MEAN_REL
        checked += 1
    assert checked >= w.hkv - 2
    say("[bwd] llama8b_32k: sums over keys")
    for g in range(w.hkv):
        want_v = dO[0, :, g * G:(g + 1) * G].sum(axis=(0, 1))
        got_v = dv[0, :, g].sum(axis=0)
        got_k = dk[0, :, g].sum(axis=0)
        # each of T bf16 elements carries <= u relative rounding: bound by u * sum |.|
        assert np.all(np.abs(got_v - want_v) <= U * np.abs(dv[0, :, g]).sum(axis=0) + 1e-6)
        assert np.all(np.abs(got_k) <= U * np.abs(dk[0, :, g]).sum(axis=0) + 1e-6)


def _rows_with_oracle_selection(Q, C, gi, B, topk, cand):
    """The candidate rows [(t, h)] whose GPU selection equals the oracle's, with that
    selection; rows at a near tie (where the two may legitimately differ) are left out,
    and any other difference fails."""
    from parity_util import check_selection_row
    rows = [(0, int(t), int(h)) for t, h in cand]
    scores = oracle.gate_scores_rows(Q, C, B, rows)
    sels = oracle.select_rows(scores, [t // B for _, t, _ in rows], topk)
    keep = []
    for (_, t, h), S, s in zip(rows, sels, scores):
        g = gi[0, h, t]
        if np.array_equal(np.asarray(S), g[g >= 0]):
            keep.append((t, h, S))
        else:
            ok, exempt, _ = check_selection_row(g, s, t // B, topk)
            assert ok and exempt, (t, h, g.tolist(), S)
    return keep


def test_backward_128k_sampled_and_sparse_upstream(moba):
    """Llama-3.1-8B heads at 128K (B=4096, top-12), the configuration the benchmark
    times, where one block's list holds up to ~360K gathered rows.

    1. dout i.i.d. N(0,1): dq of sampled rows in every query block (the first and last
       token of blocks 11, 12 and 31 among them) against the oracle row by row, and
       for every kv-head the sums over keys, which hold at any size:
       sum_u dv_u = sum of dout over the group's rows, sum_u dk_u = 0.
    2. dout zero except on a sample R of rows spread over all query blocks: every
       gradient is then a sum over R alone (dk_u, dv_u collect scale p (dO.v - D) q and
       p dO only from rows with dO != 0, and dq_t = 0 wherever dO_t = 0), so the oracle
       gives dk and dv of EVERY key and every kv-head, while the GPU still builds and
       walks the full-length lists of the history blocks."""
    w = get_workload("llama8b_128k")
    B, T, G, sc, k_ = w.block, w.seqlen, w.hq // w.hkv, w.sm_scale, w.topk
    say("[bwd128k] generating inputs")
    inp = make_inputs(w)
    g_bits = make_output_grad(w)
    q, k, v = (dev(inp[x]) for x in "qkv")
    say("[bwd128k] GPU forward + backward (dense dout)")
    out, lse, idx = moba.forward(q, k, v, B, k_, sc)
    dq, dk, dv = moba.backward(q, k, v, out, lse, idx, dev(g_bits), B, k_, sc)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    dq_s = dq.float().cpu().numpy()
    dk_f, dv_f = f64(dk), f64(dv)
    del dq, dk, dv
    K, V = bf16_to_f64(inp["k"]), bf16_to_f64(inp["v"])
    Q = bf16_to_f64(inp["q"])
    C = oracle.centroids(K, B)
    rng = np.random.default_rng(128)

    # 1. sampled dq rows under the dense upstream gradient, and the key sums
    cand = [(int(c * B + rng.integers(B)), int(rng.integers(w.hq)))
            for c in range(w.num_blocks) for _ in range(4)]
    cand += [(t, int(rng.integers(w.hq))) for c in (11, 12, 31) for t in (c * B, c * B + B - 1)]
    rows = _rows_with_oracle_selection(Q, C, gi, B, k_, cand)
    assert len(rows) >= len(cand) - 8
    say(f"[bwd128k] dq of {len(rows)} sampled rows")
    got, ref = [], []
    for t, h, S in rows:
        keys = oracle.attended_keys(S, t, B, T)
        r, _, _ = oracle.attend_row_grad(Q[0, t, h], K[0, :, h // G], V[0, :, h // G], keys,
                                         sc, bf16_to_f64(g_bits[0, t, h]))
        got.append(dq_s[0, t, h])
        ref.append(r)
    s = grad_stats("dq rows", np.array(got, np.float64), np.array(ref))
    assert s["max_rel"] <= MAX_REL and s["mean_rel"] <= MEAN_REL
    say("[bwd128k] sums over keys, every kv-head")
    for g in range(w.hkv):
        want_v = bf16_to_f64(g_bits[0, :, g * G:(g + 1) * G]).sum(axis=(0, 1))
        assert np.all(np.abs(dv_f[0, :, g].sum(axis=0) - want_v)
                      <= U * np.abs(dv_f[0, :, g]).sum(axis=0) + 1e-6)
        assert np.all(np.abs(dk_f[0, :, g].sum(axis=0))
                      <= U * np.abs(dk_f[0, :, g]).sum(axis=0) + 1e-6)
    del dk_f, dv_f, dq_s

    # 2. the upstream gradient on a sample R of rows only
    cand = [(int(c * B + rng.integers(B)), int(rng.integers(w.hq)))
            for c in range(w.num_blocks) for _ in range(3)]
    cand += [(c * B, 0) for c in (11, 12)] + [(T - 1, w.hq - 1)]
    R = _rows_with_oracle_selection(Q, C, gi, B, k_, dict.fromkeys(cand))
    sparse = np.zeros_like(g_bits)
    for t, h, _ in R:
        sparse[0, t, h] = g_bits[0, t, h]
    say(f"[bwd128k] GPU backward with dout on {len(R)} rows only")
    dq2, dk2, dv2 = moba.backward(q, k, v, out, lse, idx, dev(sparse), B, k_, sc)
    torch.cuda.synchronize()
    in_r = torch.zeros((T, w.hq), dtype=torch.bool, device="cuda")
    for t, h, _ in R:
        in_r[t, h] = True
    assert bool((dq2[0][~in_r] == 0).all()), "dq of a row without upstream gradient"
    dq_r = {(t, h): dq2[0, t, h].float().cpu().numpy().astype(np.float64) for t, h, _ in R}
    del dq2, in_r
    dk2, dv2 = f64(dk2), f64(dv2)
    rk = np.zeros(K.shape[1:])
    rv = np.zeros(V.shape[1:])
    touched = np.zeros(K.shape[1:3], bool)
    got, ref = [], []
    for t, h, S in R:
        g = h // G
        keys = oracle.attended_keys(S, t, B, T)
        dqr, dkr, dvr = oracle.attend_row_grad(Q[0, t, h], K[0, :, g], V[0, :, g], keys, sc,
                                               bf16_to_f64(sparse[0, t, h]))
        rk[keys, g] += dkr
        rv[keys, g] += dvr
        touched[keys, g] = True
        got.append(dq_r[(t, h)])
        ref.append(dqr)
    s = grad_stats("dq of R", np.array(got), np.array(ref))
    assert s["max_rel"] <= MAX_REL and s["mean_rel"] <= MEAN_REL
    say(f"[bwd128k] dk, dv of every key ({int(touched.sum())} (key, kv-head) pairs "
        "touched by R)")
    assert np.all(dk2[0][~touched] == 0) and np.all(dv2[0][~touched] == 0)
    for g in range(w.hkv):
        m = touched[:, g]
        sk = grad_stats(f"dk g{g}", dk2[0, m, g], rk[m, g])
        sv = grad_stats(f"dv g{g}", dv2[0, m, g], rv[m, g])
        for s in (sk, sv):
            assert s["max_rel"] <= MAX_REL and s["mean_rel"] <= MEAN_REL
