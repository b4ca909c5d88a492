"""The library's forward, backward and decode captured in a HIP graph
(torch.cuda.CUDAGraph).

The library allocates nothing, copies nothing and clears nothing with memset: every
launch goes to the caller's stream and every workspace word it reads is written by an
earlier kernel of the same call, so a captured call replays the eager call exactly.
Each replay is checked bit for bit against the eager result, with other eager work of
the library and a synchronisation between replays.
"""
import sys

import numpy as np
import pytest

from workloads import small_workload, make_inputs, make_output_grad, to_torch_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

REPLAYS = 3


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


def test_forward_graph_replays(moba):
    w = small_workload("graph_fwd", 1, 8, 2, 128, 4096, 256, 4, "offset", seed=91)
    say(f"[graph] forward b=1 T={w.seqlen} hq=8 hkv=2 d=128 B=256 k=4")
    inp = make_inputs(w)
    q, k, v = (dev(inp[x]) for x in "qkv")
    full, _ = moba.workspace_bytes(1, w.seqlen, 8, 2, 128, 256, 4)
    ws = torch.empty(full, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((1, 8, w.seqlen), dtype=torch.float32, device="cuda")
    idx = torch.empty((1, 8, w.seqlen, 4), dtype=torch.int32, device="cuda")
    moba.forward(q, k, v, 256, 4, workspace=ws, out=out, lse=lse, idx=idx)
    torch.cuda.synchronize()
    ref = [x.clone() for x in (out, lse, idx)]
    # other inputs for the eager work between replays
    q2 = torch.flip(q, dims=[1]).contiguous()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moba.forward(q, k, v, 256, 4, workspace=ws, out=out, lse=lse, idx=idx)
    for r in range(REPLAYS):
        out.zero_()
        lse.zero_()
        idx.zero_()
        g.replay()
        torch.cuda.synchronize()
        for name, x, y in zip(("out", "lse", "idx"), (out, lse, idx), ref):
            assert torch.equal(x, y), f"replay {r}: {name} differs from the eager call"
        # eager work of the library on other data, through the same workspace
        moba.forward(q2, k, v, 256, 4, workspace=ws)
        torch.cuda.synchronize()


def test_backward_graph_replays(moba):
    w = small_workload("graph_bwd", 1, 8, 2, 128, 2048, 128, 5, "offset", seed=92)
    say(f"[graph] backward b=1 T={w.seqlen} hq=8 hkv=2 d=128 B=128 k=5")
    inp = make_inputs(w)
    q, k, v = (dev(inp[x]) for x in "qkv")
    dout = dev(make_output_grad(w))
    out, lse, idx = moba.forward(q, k, v, 128, 5)
    full, _ = moba.backward_workspace_bytes(1, w.seqlen, 8, 2, 128, 128, 5)
    ws = torch.empty(full, dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    moba.backward(q, k, v, out, lse, idx, dout, 128, 5, workspace=ws, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    ref = [x.clone() for x in (dq, dk, dv)]
    dout2 = (-dout).contiguous()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moba.backward(q, k, v, out, lse, idx, dout, 128, 5, workspace=ws, dq=dq, dk=dk, dv=dv)
    for r in range(REPLAYS):
        for x in (dq, dk, dv):
            x.zero_()
        g.replay()
        torch.cuda.synchronize()
        for name, x, y in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            assert torch.equal(x, y), f"replay {r}: {name} differs from the eager call"
        moba.backward(q, k, v, out, lse, idx, dout2, 128, 5, workspace=ws)
        torch.cuda.synchronize()
    assert np.isfinite(ref[0].float().cpu().numpy()).all()


def test_decode_graph_replays(moba):
    rng = np.random.default_rng(93)
    from workloads import f32_to_bf16_bits
    say("[graph] decode b=1 n=2 Tk=3000 hq=8 hkv=2 d=128")
    qb = f32_to_bf16_bits(rng.standard_normal((1, 2, 8, 128), dtype=np.float32))
    kb = f32_to_bf16_bits(rng.standard_normal((1, 3000, 2, 128), dtype=np.float32))
    vb = f32_to_bf16_bits(rng.standard_normal((1, 3000, 2, 128), dtype=np.float32))
    q, k, v = dev(qb), dev(kb), dev(vb)
    ws = torch.empty(moba.decode_workspace_bytes(1, 2, 3000, 8, 2, 128), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((1, 8, 2), dtype=torch.float32, device="cuda")
    moba.decode(q, k, v, workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()
    ref = [out.clone(), lse.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moba.decode(q, k, v, workspace=ws, out=out, lse=lse)
    for r in range(REPLAYS):
        out.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), f"replay {r}"
        moba.decode(-q, k, v, workspace=ws)
        torch.cuda.synchronize()
