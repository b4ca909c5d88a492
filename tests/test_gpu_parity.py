"""Parity of the HIP path (through the C ABI) with the float64 oracle, on the GPU.

Inputs are the seeded synthetic workloads; the oracle reads the same bf16 values
widened exactly to float64.  Tolerances are those of tests/parity_util.py.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from workloads import (small_workload, get_workload, make_inputs, bf16_to_f64,
                       to_torch_bf16)
from parity_util import (check_selection_row, compare_rows, sample_rows, OUT_MAX,
                         OUT_MEAN, LSE_MAX)

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


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to("cuda")


def dev(bits):
    return to_torch_bf16(bits, "cuda")


def run_forward(moba, q, k, v, w, **kw):
    out, lse, idx = moba.forward(dev(q), dev(k), dev(v), w.block, w.topk, w.sm_scale, **kw)
    torch.cuda.synchronize()
    return (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            idx.cpu().numpy())


def full_compare(moba, w, inp=None, label=""):
    """Every row: idx (exemption rule), out, lse."""
    if inp is None:
        inp = make_inputs(w)
    say(f"[full] {label or w.name}: b={w.batch} T={w.seqlen} hq={w.hq} hkv={w.hkv} "
        f"d={w.head_dim} B={w.block} k={w.topk}")
    go, gl, gi = run_forward(moba, inp["q"], inp["k"], inp["v"], w)
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    rows = [(bi, t, h) for bi in range(w.batch) for t in range(w.seqlen) for h in range(w.hq)]
    stats = compare_rows(Q, K, V, w.block, w.topk, w.sm_scale, rows,
                         np.stack([go[bi, t, h] for bi, t, h in rows]),
                         np.array([gl[bi, h, t] for bi, t, h in rows]),
                         np.stack([gi[bi, h, t] for bi, t, h in rows]))
    say(f"       {stats}")
    return go, gl, gi


# ------------------------------------------------------------------------- (a1)
@pytest.mark.parametrize("b,T,hkv,d,B", [
    (1, 2048, 1, 64, 128), (2, 4096, 8, 128, 512), (1, 1024, 2, 128, 16),
    (1, 8192, 8, 128, 4096), (1, 512, 32, 64, 256),
    # at least 256 (sequence, block, kv-head) triples: the one-pass kernel
    (1, 8192, 8, 128, 128), (2, 4096, 4, 64, 64), (1, 8000, 8, 128, 128),
    (1, 16384, 8, 128, 512),
])
def test_pool_centroids(moba, b, T, hkv, d, B):
    w = small_workload("pool", b, hkv, hkv, d, T, B, 1, "offset", seed=T + d)
    inp = make_inputs(w)
    say(f"[pool] b={b} T={T} hkv={hkv} d={d} B={B}")
    c = moba.pool_centroids(dev(inp["k"]), B)
    torch.cuda.synchronize()
    ref = oracle.centroids(bf16_to_f64(inp["k"]), B)
    got = c.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got, ref, rtol=2e-6, atol=2e-6)


@pytest.mark.parametrize("T,hkv,B", [(1024, 2, 256), (4096, 8, 16)])
def test_pool_constant_blocks_exact(moba, T, hkv, B):
    """A block of one constant key has exactly that centroid (power-of-two B); the
    second shape has 2048 (block, kv-head) pairs, so the one-pass kernel runs."""
    b, d = 1, 64
    k = np.zeros((b, T, hkv, d), np.uint16)
    vals = np.array([0x3FA0, 0xC040, 0x3E80, 0x4110], np.uint16)   # 1.25, -3, 0.25, 9
    for j in range(T // B):
        k[:, j * B:(j + 1) * B] = vals[j % 4]
    c = moba.pool_centroids(dev(k), B).cpu().numpy()
    for j in range(T // B):
        assert np.all(c[0, :, j] == bf16_to_f64(vals[j % 4:j % 4 + 1])[0])


# ------------------------------------------------------------------------- (a2)
@pytest.mark.parametrize("b,T,hq,hkv,d,B,k,recipe", [
    (1, 2048, 1, 1, 64, 128, 4, "iid"),          # tiny workload shape
    (1, 8192, 8, 2, 128, 128, 5, "offset"),       # nb=64: two 32-block tiles
    (1, 8192, 4, 1, 128, 64, 17, "offset"),       # nb=128, KH=16 fills the 16-list
    (1, 4096, 4, 4, 64, 32, 20, "iid"),           # KH=19 -> 32-list, nb=128
    (2, 4096, 16, 2, 128, 16, 33, "iid"),         # B=16 (tiles straddle blocks), k max
    (1, 16384, 32, 8, 128, 512, 3, "iid"),        # GQA 4
    (1, 4096, 8, 8, 128, 256, 1, "iid"),          # no history slots
    (1, 2048, 1, 1, 64, 16, 5, "offset"),         # G=1, B=16: a tile spans two blocks
    (1, 4096, 4, 2, 64, 128, 24, "iid"),          # nb=32 single tile, KH=23 -> 32-list
])
def test_gate_topk(moba, b, T, hq, hkv, d, B, k, recipe):
    w = small_workload("gate", b, hq, hkv, d, T, B, k, recipe, seed=T + k)
    inp = make_inputs(w)
    say(f"[gate] b={b} T={T} hq={hq} hkv={hkv} d={d} B={B} k={k}")
    cent = moba.pool_centroids(dev(inp["k"]), B)
    idx = moba.gate_topk(dev(inp["q"]), cent, B, k).cpu().numpy()
    Q, K = bf16_to_f64(inp["q"]), bf16_to_f64(inp["k"])
    C = oracle.centroids(K, B)
    ref = oracle.select_blocks(Q, C, B, k)
    mism = np.argwhere((idx != ref).any(axis=-1))
    say(f"       rows differing before the near-tie rule: {len(mism)} of {b * hq * T}")
    exempt = 0
    for bi, h, t in mism:
        s = oracle.gate_scores_rows(Q, C, B, [(bi, t, h)])[0]
        ok, ex, _ = check_selection_row(idx[bi, h, t], s, t // B, k)
        assert ok, (bi, h, t, idx[bi, h, t].tolist(), ref[bi, h, t].tolist())
        exempt += ex
    assert exempt == len(mism)


def test_gate_zero_query_ties(moba):
    """Q = 0: every score is exactly 0 -> lower block indices win, exactly."""
    b, T, hq, hkv, d, B, k = 1, 4096, 8, 2, 128, 64, 6
    w = small_workload("z", b, hq, hkv, d, T, B, k, "iid", seed=3)
    inp = make_inputs(w)
    q = np.zeros_like(inp["q"])
    cent = moba.pool_centroids(dev(inp["k"]), B)
    idx = moba.gate_topk(dev(q), cent, B, k).cpu().numpy()
    for t in range(0, T, 37):
        c = t // B
        exp = list(range(min(k - 1, c))) + [c]
        exp += [-1] * (k - len(exp))
        assert (idx[0, :, t] == np.array(exp)).all(), (t, idx[0, :, t])


def test_gate_duplicated_block_tie(moba):
    """Block 3's keys copied into block 9: equal centroids, exact tie -> block 3."""
    b, T, hq, hkv, d, B, k = 1, 2048, 2, 1, 128, 128, 2
    w = small_workload("dup", b, hq, hkv, d, T, B, k, "iid", seed=4)
    inp = make_inputs(w)
    kk = inp["k"].copy()
    kk[:, 9 * B:10 * B] = kk[:, 3 * B:4 * B]
    K = bf16_to_f64(kk)
    C = oracle.centroids(K, B)
    qf = np.zeros((b, T, hq, d))
    qf[:, 10 * B:] = C[0, 0, 3] * 8.0           # aim every later query at block 3
    from workloads import f32_to_bf16_bits
    q = f32_to_bf16_bits(qf.astype(np.float32))
    cent = moba.pool_centroids(dev(kk), B)
    cc = cent.cpu().numpy()
    assert np.array_equal(cc[0, 0, 3], cc[0, 0, 9])
    idx = moba.gate_topk(dev(q), cent, B, k).cpu().numpy()
    assert np.all(idx[0, :, 10 * B:, 0] == 3)


# ------------------------------------------------------------------------- (a3)
def cpu_index(idx, hkv, B, topk, kv_begin, kv_count, chunk=256):
    """The documented list order, (chunk of 256 rows, slot, row), built on the CPU."""
    b, hq, T, _ = idx.shape
    G = hq // hkv
    nb = -(-T // B)
    lists = [[] for _ in range(b * kv_count * nb)]
    for bi in range(b):
        for gi in range(kv_count):
            g = kv_begin + gi
            sub = idx[bi, g * G:(g + 1) * G]                     # [G, T, topk]
            rows = sub.transpose(1, 0, 2).reshape(T * G, topk)   # row r = t*G + hl
            c = (np.arange(T * G) // G) // B
            for c0 in range(0, T * G, chunk):
                for s in range(topk - 1):
                    js = rows[c0:c0 + chunk, s]
                    cs = c[c0:c0 + chunk]
                    # a block id repeated within a row is listed at its first slot only
                    first = ~(rows[c0:c0 + chunk, :s] == js[:, None]).any(axis=1)
                    for rr in np.nonzero((js >= 0) & (js < cs) & first)[0]:
                        r = c0 + rr
                        lists[(bi * kv_count + gi) * nb + js[rr]].append((r << 5) | s)
    offs = np.zeros(len(lists) + 1, np.int64)
    offs[1:] = np.cumsum([len(x) for x in lists])
    ent = np.array([e for x in lists for e in x], np.int64)
    return offs, ent


@pytest.mark.parametrize("b,T,hq,hkv,B,k,kv_begin,kv_count", [
    (1, 4096, 8, 2, 256, 4, 0, 2),
    (2, 2048, 4, 1, 64, 9, 0, 1),
    (1, 8192, 32, 8, 512, 3, 3, 4),
    (1, 2048, 4, 4, 16, 33, 1, 2),
    # at least 8 history slots over many short lists: the entries staged in LDS
    (1, 8192, 8, 2, 64, 12, 0, 2),
    (2, 4000, 4, 2, 32, 16, 1, 1),      # and a partial last block
])
def test_inverted_index(moba, b, T, hq, hkv, B, k, kv_begin, kv_count):
    w = small_workload("idx", b, hq, hkv, 64, T, B, k, "iid", seed=B + k)
    inp = make_inputs(w)
    say(f"[index] b={b} T={T} hq={hq} hkv={hkv} B={B} k={k} kv=[{kv_begin},+{kv_count})")
    cent = moba.pool_centroids(dev(inp["k"]), B)
    idx_t = moba.gate_topk(dev(inp["q"]), cent, B, k)
    offs, ent = moba.build_index(idx_t, hkv, B, k, kv_begin, kv_count)
    offs2, ent2 = moba.build_index(idx_t, hkv, B, k, kv_begin, kv_count)
    torch.cuda.synchronize()
    assert torch.equal(offs, offs2) and torch.equal(ent, ent2)        # deterministic
    ref_offs, ref_ent = cpu_index(idx_t.cpu().numpy(), hkv, B, k, kv_begin, kv_count)
    assert np.array_equal(offs.cpu().numpy().astype(np.int64), ref_offs)
    assert np.array_equal(ent.cpu().numpy().astype(np.int64) & 0xFFFFFFFF, ref_ent)


def test_index_repeated_block_ids(moba):
    """A caller-built idx that repeats a block id within a row: the repeat is listed at
    its first slot only, so the lists never hold more than the shape's entry count."""
    b, T, hq, hkv, B, k = 1, 4096, 8, 2, 128, 6
    w = small_workload("dup_idx", b, hq, hkv, 64, T, B, k, "iid", seed=21)
    inp = make_inputs(w)
    cent = moba.pool_centroids(dev(inp["k"]), B)
    idx = moba.gate_topk(dev(inp["q"]), cent, B, k).cpu().numpy()
    rng = np.random.default_rng(5)
    bad = idx.copy()
    rows = rng.integers(0, T, 400)
    for t, h in zip(rows, rng.integers(0, hq, 400)):
        if t // B >= k:                        # rows with k-1 history slots filled
            bad[0, h, t, 1:k - 1] = bad[0, h, t, 0]   # every history slot = slot 0's block
    offs, ent = moba.build_index(dev_i32(bad), hkv, B, k, 0, hkv)
    torch.cuda.synchronize()
    ref_offs, ref_ent = cpu_index(bad, hkv, B, k, 0, hkv)
    assert np.array_equal(offs.cpu().numpy().astype(np.int64), ref_offs)
    # the entry buffer has the shape's capacity; the lists fill its first offs[-1] words
    n = int(ref_offs[-1])
    assert n < ent.numel() == moba.index_entries(b, T, hq, hkv, B, k, hkv)
    assert np.array_equal(ent[:n].cpu().numpy().astype(np.int64) & 0xFFFFFFFF, ref_ent)


def test_stages_ragged_last_block(moba):
    """The stage entry points with T % B != 0 (a partial last block of 104 tokens):
    centroids of every block (the last one the mean of the keys present), the gate's
    selection of every row, and the inverted index."""
    b, T, hq, hkv, d, B, k = 1, 1000, 4, 2, 128, 128, 4
    w = small_workload("ragged_stages", b, hq, hkv, d, T, B, k, "offset", seed=23)
    inp = make_inputs(w)
    cent = moba.pool_centroids(dev(inp["k"]), B)
    assert cent.shape == (b, hkv, 8, d)
    K, Q = bf16_to_f64(inp["k"]), bf16_to_f64(inp["q"])
    C = oracle.centroids(K, B)
    np.testing.assert_allclose(cent.cpu().numpy().astype(np.float64), C, rtol=2e-6, atol=2e-6)
    idx_t = moba.gate_topk(dev(inp["q"]), cent, B, k)
    idx = idx_t.cpu().numpy()
    ref = oracle.select_blocks(Q, C, B, k)
    mism = np.argwhere((idx != ref).any(axis=-1))
    for bi, h, t in mism:
        s_ = oracle.gate_scores_rows(Q, C, B, [(bi, t, h)])[0]
        ok, _, _ = check_selection_row(idx[bi, h, t], s_, t // B, k)
        assert ok, (bi, h, t)
    offs, ent = moba.build_index(idx_t, hkv, B, k)
    torch.cuda.synchronize()
    ref_offs, ref_ent = cpu_index(idx, hkv, B, k, 0, hkv)
    assert np.array_equal(offs.cpu().numpy().astype(np.int64), ref_offs)
    assert np.array_equal(ent.cpu().numpy().astype(np.int64) & 0xFFFFFFFF, ref_ent)


# ------------------------------------------------------------------------- (a4, a5)
SMALL = [
    # name, b, hq, hkv, d, T, B, k, recipe
    ("tiny_2k", None),
    ("gqa4_d128", small_workload("gqa4_d128", 1, 8, 2, 128, 4096, 256, 4, "offset", 7)),
    ("b2_d64", small_workload("b2_d64", 2, 4, 2, 64, 2048, 128, 5, "iid", 8)),
    ("blk16_k33", small_workload("blk16_k33", 1, 2, 1, 128, 1024, 16, 33, "iid", 9)),
    ("blk48", small_workload("blk48", 1, 4, 1, 64, 1536, 48, 3, "offset", 10)),
    ("g8", small_workload("g8", 1, 16, 2, 128, 2048, 128, 6, "iid", 11)),
    ("topk1", small_workload("topk1", 1, 4, 2, 128, 2048, 256, 1, "iid", 12)),
    ("dense", small_workload("dense", 1, 4, 1, 64, 1024, 128, 8, "iid", 13)),
    ("k_over_nb", small_workload("k_over_nb", 1, 2, 2, 128, 768, 256, 9, "iid", 14)),
    # G = 3 (does not divide the eight waves: heads in rounds) and G = 16 (two rounds)
    ("g3", small_workload("g3", 1, 6, 2, 128, 2048, 128, 4, "offset", 16)),
    ("g16_d64", small_workload("g16_d64", 1, 16, 1, 64, 1024, 64, 5, "offset", 17)),
    # top-20 over 24 blocks of 256 keys (the queued chained history kernel): rows with
    # 1-4, 5-8, 9-16 and 19 history parts, every path of the current-block merge
    ("k20_chain", small_workload("k20_chain", 1, 4, 2, 128, 6144, 256, 20, "offset", 18)),
    # top-16 over 125 blocks of 32 keys, the last one partial: the index stages each
    # chunk's entries in LDS
    ("k16_b32_staged", small_workload("k16_b32_staged", 1, 4, 2, 128, 4000, 32, 16, "offset", 19)),
]


@pytest.mark.parametrize("name,w", SMALL, ids=[s[0] for s in SMALL])
def test_forward_small_all_rows(moba, name, w):
    if w is None:
        w = get_workload(name)
    full_compare(moba, w)


def test_forward_dense_equals_sdpa(moba):
    """topk >= nb: the GPU result is full causal attention (torch SDPA, fp32 CPU)."""
    w = small_workload("dense", 1, 4, 2, 128, 2048, 256, 8, "iid", 15)
    inp = make_inputs(w)
    go, gl, gi = run_forward(moba, inp["q"], inp["k"], inp["v"], w)
    q, k, v = (torch.from_numpy(bf16_to_f64(inp[x])).float().permute(0, 2, 1, 3)
               for x in "qkv")
    k = k.repeat_interleave(2, dim=1)
    v = v.repeat_interleave(2, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True,
                                                           scale=w.sm_scale)
    ref = ref.permute(0, 2, 1, 3).double().numpy()
    d = np.abs(go - ref)
    assert d.max() <= OUT_MAX and d.mean() <= OUT_MEAN


def test_forward_zero_query_closed_form(moba):
    """Q = 0: uniform attention, lse = ln|N| and out = mean of V over N."""
    w = small_workload("zq", 1, 4, 2, 128, 2048, 128, 4, "iid", 16)
    inp = make_inputs(w)
    q = np.zeros_like(inp["q"])
    go, gl, gi = run_forward(moba, q, inp["k"], inp["v"], w)
    V = bf16_to_f64(inp["v"])
    B, k = w.block, w.topk
    for t in range(0, w.seqlen, 13):
        c = t // B
        S = list(range(min(k - 1, c))) + [c]
        n = (len(S) - 1) * B + (t - c * B + 1)
        for h in range(w.hq):
            assert gi[0, h, t, :len(S)].tolist() == S
            assert abs(gl[0, h, t] - math.log(n)) <= LSE_MAX
            keys = oracle.attended_keys(S, t, B, w.seqlen)
            assert np.abs(go[0, t, h] - V[0, keys, h // 2].mean(0)).max() <= OUT_MAX


def test_forward_constant_values(moba):
    w = small_workload("cv", 1, 4, 1, 64, 1024, 64, 3, "iid", 17)
    inp = make_inputs(w)
    v = np.full_like(inp["v"], 0x3FC0)        # 1.5
    go, _, _ = run_forward(moba, inp["q"], inp["k"], v, w)
    assert np.abs(go - 1.5).max() <= 1e-2


def test_forward_block_indicator_values(moba):
    """V[u] = e_blk(u): the output is the attention mass per block; it is nonzero
    exactly on the selected blocks and sums to 1 (routing seen through attention)."""
    w = small_workload("ind", 1, 4, 1, 64, 2048, 64, 4, "offset", 18)
    inp = make_inputs(w)
    nb = w.seqlen // w.block
    v = np.zeros_like(inp["v"])
    v[0, np.arange(w.seqlen), 0, np.arange(w.seqlen) // w.block] = 0x3F80   # 1.0
    go, _, gi = run_forward(moba, inp["q"], inp["k"], v, w)
    for h in range(w.hq):
        for t in range(0, w.seqlen, 7):
            S = set(gi[0, h, t][gi[0, h, t] >= 0].tolist())
            nz = set(np.nonzero(go[0, t, h, :nb] > 0)[0].tolist())
            assert nz == S, (h, t, S, nz)
            assert abs(go[0, t, h].sum() - 1) < 2e-2


def test_forward_deterministic_and_chunked(moba):
    """Bitwise identical across runs, and when the workspace only fits one kv-head."""
    w = small_workload("det", 1, 16, 4, 128, 4096, 256, 5, "offset", 19)
    inp = make_inputs(w)
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    a = moba.forward(q, k, v, w.block, w.topk)
    b = moba.forward(q, k, v, w.block, w.topk)
    full, mn = moba.workspace_bytes(1, 4096, 16, 4, 128, 256, 5)
    ws = torch.empty(mn, dtype=torch.uint8, device="cuda")
    c = moba.forward(q, k, v, w.block, w.topk, workspace=ws)
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(x, z)


def test_forward_timed_events(moba):
    """moba_forward_timed gives the same results as moba_forward, and its stage events,
    recorded on the stream without a synchronisation, bracket the whole call."""
    w = small_workload("timed", 1, 8, 2, 128, 4096, 256, 5, "offset", 21)
    inp = make_inputs(w)
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    a = moba.forward(q, k, v, w.block, w.topk)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(moba.STAGES) + 1)]
    for e in evs:
        e.record()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    b = moba.forward(q, k, v, w.block, w.topk, events=evs)
    end.record()
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    stages = [evs[i].elapsed_time(evs[i + 1]) for i in range(len(moba.STAGES))]
    assert all(t >= 0.0 for t in stages) and stages[3] > 0.0   # history ran
    assert sum(stages) <= start.elapsed_time(end) + 0.05
    # top-1 (no history slots): the index and history stages are empty, and every
    # event is still recorded within this call
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    start.record()
    moba.forward(q, k, v, w.block, 1, events=evs)
    end.record()
    torch.cuda.synchronize()
    assert start.elapsed_time(evs[0]) >= 0.0 and evs[-1].elapsed_time(end) >= 0.0
    stages = [evs[i].elapsed_time(evs[i + 1]) for i in range(len(moba.STAGES))]
    assert all(t >= 0.0 for t in stages) and stages[4] > 0.0
    assert stages[2] < 0.05 and stages[3] < 0.05
    assert sum(stages) <= start.elapsed_time(end) + 0.05


@pytest.mark.parametrize("b,hq,hkv,d,T", [(1, 4, 2, 128, 2048), (2, 2, 1, 64, 1024),
                                           (1, 8, 8, 128, 784)])
def test_dense_forward_matches_oracle(moba, b, hq, hkv, d, T):
    """Dense causal attention (the full-attention layers of a hybrid model) against the
    oracle with every block selected (pinned to SDPA), all rows."""
    w = small_workload("dense_causal", b, hq, hkv, d, T, 16, T // 16, "iid", 23)
    inp = make_inputs(w)
    say(f"[dense] b={b} T={T} hq={hq} hkv={hkv} d={d}")
    go, gl = moba.dense_forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), w.sm_scale)
    torch.cuda.synchronize()
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    ro, rl, _, _ = oracle.moba_forward(Q, K, V, w.block, w.topk, w.sm_scale)
    go = go.float().cpu().numpy()
    gl = gl.cpu().numpy()
    err = np.abs(go - ro)
    assert err.max() <= OUT_MAX and err.mean() <= OUT_MEAN, (err.max(), err.mean())
    assert np.abs(gl - rl).max() <= LSE_MAX
    # the hybrid dispatcher's dense branch is the same call
    ho, hl, hi = moba.attention(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), w.block, w.topk,
                                w.sm_scale, dense=True)
    torch.cuda.synchronize()
    assert hi is None and np.array_equal(ho.float().cpu().numpy(), go)


def test_dense_forward_32k_sampled(moba):
    """Dense causal attention at 32K tokens, 32/8 heads, d=128: sampled rows against the
    oracle's one-softmax definition over keys 0..t."""
    w = get_workload("llama8b_32k")
    inp = make_inputs(w)
    go_t, gl_t = moba.dense_forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), w.sm_scale)
    torch.cuda.synchronize()
    K, V = bf16_to_f64(inp["k"]), bf16_to_f64(inp["v"])
    r = np.random.default_rng(7)
    rows = [(0, int(r.integers(w.seqlen)), int(r.integers(w.hq))) for _ in range(160)]
    rows += [(0, 0, 0), (0, w.seqlen - 1, w.hq - 1)]
    G = w.hq // w.hkv
    for bi, t, h in rows:
        o, l = oracle.attend_row(bf16_to_f64(inp["q"][bi, t, h]), K[bi, :, h // G],
                                 V[bi, :, h // G], np.arange(t + 1), w.sm_scale)
        go = go_t[bi, t, h].float().cpu().numpy()
        assert np.abs(go - o).max() <= OUT_MAX, (t, h)
        assert abs(float(gl_t[bi, h, t]) - l) <= LSE_MAX, (t, h)


def test_forward_rejects_small_workspace(moba):
    w = small_workload("ws", 1, 4, 2, 64, 1024, 128, 3, "iid", 20)
    inp = make_inputs(w)
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(moba.MobaError):
        moba.forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), w.block, w.topk,
                     workspace=ws)


# ------------------------------------------------------------------------- full sizes
def big_compare(moba, name, per_block, seed):
    w = get_workload(name)
    say(f"[big] {name}: generating inputs")
    inp = make_inputs(w)
    say(f"[big] {name}: running the GPU path")
    go_t, gl_t, gi_t = moba.forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), w.block,
                                    w.topk, w.sm_scale)
    torch.cuda.synchronize()
    gi = gi_t.cpu().numpy()
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    C = oracle.centroids(K, w.block)
    say(f"[big] {name}: oracle selection for every row")
    ref = oracle.select_blocks(Q, C, w.block, w.topk)
    mism = np.argwhere((gi != ref).any(axis=-1))
    exempt = 0
    for bi, h, t in mism:
        s = oracle.gate_scores_rows(Q, C, w.block, [(bi, t, h)])[0]
        ok, ex, _ = check_selection_row(gi[bi, h, t], s, t // w.block, w.topk)
        assert ok, (bi, h, t, gi[bi, h, t].tolist(), ref[bi, h, t].tolist())
        exempt += ex
    say(f"[big] {name}: {len(mism)} rows differ, all within the near-tie rule "
        f"({exempt} exempt of {gi.shape[1] * gi.shape[2]})")
    rows = sample_rows(w.batch, w.seqlen, w.hq, w.block, per_block=per_block, seed=seed,
                       extra=[(0, w.seqlen - 1, w.hq - 1), (0, 0, 0)])
    bi_, t_, h_ = (np.array(x) for x in zip(*rows))
    ib, it, ih = (torch.as_tensor(x, device="cuda") for x in (bi_, t_, h_))
    go = go_t[ib, it, ih].float().cpu().numpy()
    gl = gl_t[ib, ih, it].cpu().numpy()
    stats = compare_rows(Q, K, V, w.block, w.topk, w.sm_scale, rows, go, gl,
                         gi[bi_, h_, t_], C=C)
    say(f"[big] {name}: {stats}")


def test_llama8b_32k(moba):
    big_compare(moba, "llama8b_32k", per_block=6, seed=2)


def test_llama8b_128k(moba):
    big_compare(moba, "llama8b_128k", per_block=12, seed=3)


def test_llama8b_64k_b128(moba):
    big_compare(moba, "llama8b_64k_b128", per_block=1, seed=4)


class _Bf16Rows:
    """A bf16 bit array that widens to float64 only what is indexed (the oracle's row
    functions index single query rows), so a 1M-token Q need not exist in float64."""

    def __init__(self, bits):
        self.bits = bits
        self.shape = bits.shape

    def __getitem__(self, idx):
        return bf16_to_f64(self.bits[idx])


def check_idx_rows(idx, B, topk):
    """Properties every idx row has, checked on all rows: ascending valid entries,
    min(k, c+1) of them, the last one the current block c, none in the future, then
    -1 padding."""
    b, hq, T, k = idx.shape
    c = (np.arange(T) // B)[None, None, :]
    n_valid = np.minimum(topk, c + 1)
    pos = np.arange(k)[None, None, None, :]
    valid = pos < n_valid[..., None]
    assert np.all(np.where(valid, idx >= 0, idx == -1)), "padding"
    last = np.take_along_axis(idx, (n_valid - 1)[..., None].repeat(b, 0).repeat(hq, 1), -1)
    assert np.all(last[..., 0] == c), "current block"
    assert np.all(np.where(valid, idx <= c[..., None], True)), "future block"
    inc = np.diff(idx, axis=-1) > 0
    assert np.all(np.where(valid[..., 1:], inc, True)), "ascending"


def test_llama8b_1m(moba):
    """1M tokens, B=4096, k=12: every idx row's properties, and sampled rows against the
    oracle (selection with the near-tie rule, out and lse)."""
    w = get_workload("llama8b_1m")
    say(f"[big] {w.name}: generating inputs")
    inp = make_inputs(w)
    say(f"[big] {w.name}: running the GPU path")
    go_t, gl_t, gi_t = moba.forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), w.block,
                                    w.topk, w.sm_scale)
    torch.cuda.synchronize()
    say(f"[big] {w.name}: checking every idx row")
    gi = gi_t.cpu().numpy()
    check_idx_rows(gi, w.block, w.topk)
    rows = sample_rows(w.batch, w.seqlen, w.hq, w.block, per_block=2, seed=5,
                       extra=[(0, w.seqlen - 1, w.hq - 1), (0, 0, 0)])
    say(f"[big] {w.name}: oracle on {len(rows)} sampled rows")
    K = bf16_to_f64(inp["k"])
    V = bf16_to_f64(inp["v"])
    C = oracle.centroids(K, w.block)
    bi_, t_, h_ = (np.array(x) for x in zip(*rows))
    ib, it, ih = (torch.as_tensor(x, device="cuda") for x in (bi_, t_, h_))
    go = go_t[ib, it, ih].float().cpu().numpy()
    gl = gl_t[ib, ih, it].cpu().numpy()
    stats = compare_rows(_Bf16Rows(inp["q"]), K, V, w.block, w.topk, w.sm_scale, rows, go,
                         gl, gi[bi_, h_, t_], C=C)
    say(f"[big] {w.name}: {stats}")


def test_edge_sizes(moba):
    """The largest block count the library accepts (2048 blocks of 16 tokens), every
    row's selection and sampled rows' out/lse; and a one-token sequence."""
    w = small_workload("max_blocks", 1, 2, 1, 64, 32768, 16, 6, "offset", seed=18)
    assert w.num_blocks == 2048
    inp = make_inputs(w)
    say(f"[edge] {w.name}: T={w.seqlen} B={w.block} nb={w.num_blocks} k={w.topk}")
    go_t, gl_t, gi_t = moba.forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), w.block,
                                    w.topk, w.sm_scale)
    torch.cuda.synchronize()
    gi = gi_t.cpu().numpy()
    check_idx_rows(gi, w.block, w.topk)
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    rows = sample_rows(1, w.seqlen, w.hq, w.block, per_block=1, seed=6,
                       extra=[(0, w.seqlen - 1, 1), (0, 0, 0)])
    bi_, t_, h_ = (np.array(x) for x in zip(*rows))
    ib, it, ih = (torch.as_tensor(x, device="cuda") for x in (bi_, t_, h_))
    stats = compare_rows(Q, K, V, w.block, w.topk, w.sm_scale, rows,
                         go_t[ib, it, ih].float().cpu().numpy(), gl_t[ib, ih, it].cpu().numpy(),
                         gi[bi_, h_, t_])
    say(f"       {stats}")
    # one token: it attends itself only
    w1 = small_workload("one_token", 2, 4, 2, 128, 1, 16, 3, "iid", seed=19)
    inp1 = make_inputs(w1)
    o1, l1, i1 = moba.forward(dev(inp1["q"]), dev(inp1["k"]), dev(inp1["v"]), 16, 3)
    torch.cuda.synchronize()
    V1 = bf16_to_f64(inp1["v"])
    Q1, K1 = bf16_to_f64(inp1["q"]), bf16_to_f64(inp1["k"])
    for b in range(2):
        for h in range(4):
            assert i1[b, h, 0].tolist() == [0, -1, -1]
            np.testing.assert_allclose(o1[b, 0, h].float().cpu().numpy(), V1[b, 0, h // 2],
                                       atol=1e-2)
            np.testing.assert_allclose(l1[b, h, 0].item(),
                                       w1.sm_scale * Q1[b, 0, h] @ K1[b, 0, h // 2], atol=1e-3)
