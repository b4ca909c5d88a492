"""moba_forward_noalloc (the forward for callers that cannot allocate: it runs on the
library's fixed per-GPU scratch) against moba_forward with a caller workspace, through
the C ABI: two calls in a row, the second on a smaller input, each bit for bit equal to
moba_forward (the same kernels, in the same kv-head grouping), and a problem too large
for the scratch rejected on the host before any device work."""
import sys

import numpy as np
import pytest

from workloads import small_workload, make_inputs, to_torch_bf16

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


def run_both(moba, w):
    inp = make_inputs(w)
    q, k, v = (to_torch_bf16(inp[x], "cuda") for x in "qkv")
    ref = moba.forward(q, k, v, w.block, w.topk, w.sm_scale)
    got = moba.forward_noalloc(q, k, v, w.block, w.topk, w.sm_scale)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_forward_twice(moba):
    big = small_workload("na_big", 2, 8, 2, 128, 4096, 256, 5, "offset", seed=61)
    small = small_workload("na_small", 1, 4, 1, 64, 1000, 128, 3, "iid", seed=62)
    for w in (big, small):            # the second call on a smaller input
        say(f"[noalloc] b={w.batch} T={w.seqlen} hq={w.hq} hkv={w.hkv} d={w.head_dim} "
            f"B={w.block} k={w.topk}")
        (ro, rl, ri), (go, gl, gi) = run_both(moba, w)
        assert torch.equal(ri, gi)
        assert torch.equal(rl, gl)
        assert torch.equal(ro.view(torch.int16), go.view(torch.int16))


def test_noalloc_rejects_too_large(moba):
    # one kv-head of the 128K Llama-3.1-8B-shaped forward needs ~1.5 GB of workspace
    full, mn = moba.workspace_bytes(1, 131072, 32, 8, 128, 4096, 12)
    assert mn > 128 << 20
    q = torch.zeros((1, 131072, 32, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 131072, 8, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 7.0)
    with pytest.raises(moba.MobaError) as e:
        moba.forward_noalloc(q, k, k, 4096, 12, out=out)
    assert e.value.status == -3       # MOBA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())   # nothing was written
