"""The forward run stage by stage through the C ABI, and the tile-order race check.

* pool -> gate -> build_index -> history_partials -> current_merge over kv-head ranges
  reproduces moba_forward bit for bit (out, lse, idx) when topk * block < T (with
  every block selected the forward runs the dense kernel), for every history kernel the
  library dispatches to: blocks of at most 128 keys (resident block), 256 to 4096 keys
  (persistent chained walk fed by the tile queue), 192 keys (one tile per workgroup),
  a partial last block, and two kv-head ranges run separately.
* history_partials with the tiles launched in seeded permuted orders writes the same
  parts, bit for bit, as in list order: each part belongs to one tile, so the result
  may not depend on which tile runs first (a randomised launch-order check for races
  between the inverted index's tiles and the history kernels).
* every history part (o, lse) against the float64 oracle's per-part attention
  (oracle.attend_parts_row: one block's keys, softmax on their own), on the GPU's own
  selection, with the part row read in its stored dimension order; tolerances those
  of tests/parity_util.py.
"""
import sys

import numpy as np
import pytest

import oracle
from workloads import small_workload, make_inputs, bf16_to_f64, to_torch_bf16
from parity_util import OUT_MAX, OUT_MEAN, LSE_MAX

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


def staged_forward(moba, q, k, v, B, topk, scale, ranges):
    b, T, hq, d = q.shape
    hkv = k.shape[2]
    cent = moba.pool_centroids(k, B)
    idx = moba.gate_topk(q, cent, B, topk)
    out = torch.empty_like(q)
    lse = torch.empty((b, hq, T), dtype=torch.float32, device=q.device)
    for kv0, kvn in ranges:
        po = pl = None
        if topk > 1:
            offs, ent = moba.build_index(idx, hkv, B, topk, kv0, kvn)
            po, pl = moba.history_partials(q, k, v, offs, ent, B, topk, scale, kv0, kvn)
        moba.current_merge(q, k, v, po, pl, B, topk, scale, kv0, kvn, out=out, lse=lse)
    return out, lse, idx


# (b, hq, hkv, d, T, B, topk): which history kernel runs is in the comment
CHAIN_SHAPES = [
    (1, 8, 2, 128, 4096, 128, 6, [(0, 2)]),          # resident block (B <= 128)
    (1, 4, 1, 64, 2048, 64, 5, [(0, 1)]),            # resident, d = 64
    (1, 8, 2, 128, 4096, 256, 5, [(0, 2)]),          # chained persistent walk
    (2, 8, 4, 128, 4096, 1024, 3, [(0, 4)]),         # chained, 16 subtiles per tile
    (1, 8, 2, 128, 8192, 2048, 3, [(0, 2)]),         # chained, 32 subtiles per tile
    (1, 8, 2, 128, 4032, 192, 6, [(0, 2)]),          # one tile per workgroup (3 subtiles)
    (1, 8, 4, 128, 4000, 256, 5, [(0, 4)]),          # partial last block
    (1, 16, 4, 128, 4096, 512, 4, [(0, 1), (1, 3)]),  # kv-head ranges run separately
    (1, 4, 2, 128, 1024, 256, 1, [(0, 2)]),          # no history slots
]


@pytest.mark.parametrize("b,hq,hkv,d,T,B,k,ranges", CHAIN_SHAPES)
def test_stage_chain_is_the_forward(moba, b, hq, hkv, d, T, B, k, ranges):
    w = small_workload("stages", b, hq, hkv, d, T, B, k, "offset", 31)
    say("stage chain", (b, hq, hkv, d, T, B, k), ranges)
    inp = make_inputs(w)
    q, kk, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    o1, l1, i1 = moba.forward(q, kk, v, B, k, w.sm_scale)
    o2, l2, i2 = staged_forward(moba, q, kk, v, B, k, w.sm_scale, ranges)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(o1, o2)
    assert torch.equal(l1, l2)


ORDER_SHAPES = [
    (1, 8, 2, 128, 4096, 128, 6),      # resident block
    (1, 8, 2, 128, 4096, 256, 5),      # chained persistent walk
    (1, 8, 2, 128, 8192, 2048, 3),     # chained, 32 subtiles per tile
    (1, 8, 2, 128, 4032, 192, 6),      # one tile per workgroup (3 subtiles)
    (2, 4, 2, 64, 3000, 192, 4),       # d = 64, partial last block, batch 2
]


@pytest.mark.parametrize("b,hq,hkv,d,T,B,k", ORDER_SHAPES)
def test_history_parts_do_not_depend_on_tile_order(moba, b, hq, hkv, d, T, B, k):
    w = small_workload("order", b, hq, hkv, d, T, B, k, "iid", 32)
    say("tile order", (b, hq, hkv, d, T, B, k))
    inp = make_inputs(w)
    q, kk, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    idx = moba.gate_topk(q, moba.pool_centroids(kk, B), B, k)
    offs, ent = moba.build_index(idx, hkv, B, k)
    po0, pl0 = moba.history_partials(q, kk, v, offs, ent, B, k, w.sm_scale)
    for seed in (1, 2, 3, 12345, 2 ** 31 + 7):
        po, pl = moba.history_partials(q, kk, v, offs, ent, B, k, w.sm_scale,
                                       tile_order_seed=seed)
        torch.cuda.synchronize()
        assert torch.equal(po, po0), seed
        assert torch.equal(pl, pl0), seed
    # the parts were written at all: every row of block c >= 1 has a first slot
    assert bool((pl0[0, :, :, B:] != 0).all())


@pytest.mark.parametrize("b,hq,hkv,d,T,B,k", [
    (1, 4, 2, 128, 2048, 256, 4),      # chained walk
    (1, 4, 1, 64, 1024, 128, 5),       # resident block, d = 64
    (1, 2, 1, 128, 4096, 2048, 2),     # chained walk, 32 subtiles per tile
    (1, 2, 1, 128, 1536, 192, 3),      # one tile per workgroup (3 subtiles)
])
def test_history_parts_match_the_oracle(moba, b, hq, hkv, d, T, B, k):
    w = small_workload("parts", b, hq, hkv, d, T, B, k, "offset", 33)
    say("parts vs oracle", (b, hq, hkv, d, T, B, k))
    inp = make_inputs(w)
    q, kk, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    idx = moba.gate_topk(q, moba.pool_centroids(kk, B), B, k)
    offs, ent = moba.build_index(idx, hkv, B, k)
    po, pl = moba.history_partials(q, kk, v, offs, ent, B, k, w.sm_scale)
    torch.cuda.synchronize()
    po = po.float().cpu().numpy()
    pl = pl.cpu().numpy()
    gi = idx.cpu().numpy()
    Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
    G = hq // hkv
    order = np.array(moba.part_dim_order(d))     # the dimension at each stored position
    d_o, d_l = [], []
    n = 0
    for bi in range(b):
        for h in range(hq):
            g = h // G
            for t in range(B, T):
                S = [int(j) for j in gi[bi, h, t] if j >= 0]
                parts = oracle.attend_parts_row(Q[bi, t, h], K[bi, :, g], V[bi, :, g], S, t,
                                                B, T, w.sm_scale)
                hist = [p for p in parts if p[0] == "hist"]
                for slot, (_, j, o_ref, l_ref) in enumerate(hist):
                    assert S[slot] == j
                    d_o.append(np.abs(po[bi, h, t, slot] - o_ref[order]))
                    d_l.append(abs(pl[slot, bi, h, t] - l_ref))
                    n += 1
    d_o = np.concatenate(d_o)
    stats = dict(parts=n, out_max=float(d_o.max()), out_mean=float(d_o.mean()),
                 lse_max=float(max(d_l)))
    say(stats)
    assert stats["out_max"] <= OUT_MAX, stats
    assert stats["out_mean"] <= OUT_MEAN, stats
    assert stats["lse_max"] <= LSE_MAX, stats
