"""The short key convolution within blocks on the GPU, against the float64 oracle
(pinned by tests/test_oracle_conv.py).

Bar: the GPU sums the taps in float32 and rounds to bf16; the oracle sums in float64.
Each output may therefore differ from the oracle's value rounded to bf16 by one bf16
step where the two sums straddle a rounding boundary: |gpu - oracle| <= 2^-8 |oracle|
+ 1e-6 elementwise (half a step from the rounding plus the float32 sum's error), and
such elements are rare (checked below).
"""
import sys

import numpy as np
import pytest

import oracle
from workloads import (small_workload, make_inputs, bf16_to_f64, bf16_to_f32,
                       to_torch_bf16, f32_to_bf16_bits)

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


def weights(hkv, d, w, seed):
    r = np.random.default_rng(seed)
    return (r.standard_normal((hkv, d, w)) / np.sqrt(w)).astype(np.float32)


def check(got_bits, ref):
    got = bf16_to_f64(got_bits)
    err = np.abs(got - ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-6), float(err.max())
    # most elements are the oracle's value rounded to bf16 exactly
    exact = got_bits == f32_to_bf16_bits(ref.astype(np.float32))
    assert exact.mean() > 0.995, exact.mean()
    return float(err.max()), float(exact.mean())


@pytest.mark.parametrize("b,T,hkv,d,B,w", [
    (1, 2048, 8, 128, 128, 4), (2, 1000, 2, 64, 64, 8), (1, 777, 1, 128, 16, 3),
    (1, 4096, 8, 128, 4096, 1), (1, 130, 4, 64, 48, 7),
])
def test_key_conv_matches_oracle(moba, b, T, hkv, d, B, w):
    say(f"[conv] b={b} T={T} hkv={hkv} d={d} B={B} w={w}")
    wl = small_workload("conv", b, hkv, hkv, d, T, B, 1, "offset", seed=T + w)
    k = make_inputs(wl)["k"]
    W = weights(hkv, d, w, T)
    out = moba.key_short_conv(to_torch_bf16(k, "cuda"), torch.from_numpy(W).cuda(), B)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    ref = oracle.key_short_conv(bf16_to_f64(k), W.astype(np.float64), B)
    say(f"       max err {check(got, ref)}")


def test_key_conv_packed(moba):
    lengths = (1000, 37, 513, 1, 2000)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    r = np.random.default_rng(9)
    k = f32_to_bf16_bits(r.standard_normal((cu[-1], 4, 128), dtype=np.float32))
    W = weights(4, 128, 5, 9)
    out = moba.key_short_conv(to_torch_bf16(k, "cuda"), torch.from_numpy(W).cuda(), 64,
                              cu_seqlens=cu)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    ref = oracle.key_short_conv(bf16_to_f64(k), W.astype(np.float64), 64, cu)
    say(f"[conv] packed {lengths}: {check(got, ref)}")


def test_key_conv_then_moba_forward(moba):
    """The convolved keys feed moba_forward: routing and attention follow the oracle
    run on the oracle's own convolved keys rounded to bf16 (a key may differ from the
    GPU's by one bf16 step, which moves scores far less than the tolerances)."""
    from parity_util import compare_rows
    w = small_workload("convfwd", 1, 8, 2, 128, 2048, 128, 4, "offset", seed=21)
    inp = make_inputs(w)
    W = weights(2, 128, 4, 21)
    kc = moba.key_short_conv(to_torch_bf16(inp["k"], "cuda"), torch.from_numpy(W).cuda(),
                             w.block)
    out, lse, idx = moba.forward(to_torch_bf16(inp["q"], "cuda"), kc,
                                 to_torch_bf16(inp["v"], "cuda"), w.block, w.topk)
    torch.cuda.synchronize()
    kc_bits = kc.cpu().view(torch.int16).numpy().view(np.uint16)
    ref_kc = oracle.key_short_conv(bf16_to_f64(inp["k"]), W.astype(np.float64), w.block)
    check(kc_bits, ref_kc)
    Kc = bf16_to_f64(f32_to_bf16_bits(ref_kc.astype(np.float32)))
    Q, V = bf16_to_f64(inp["q"]), bf16_to_f64(inp["v"])
    go, gl, gi = out.float().cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy()
    rows = [(0, t, h) for t in range(w.seqlen) for h in range(w.hq)]
    stats = compare_rows(Q, Kc, V, w.block, w.topk, w.sm_scale, rows,
                         np.stack([go[0, t, h] for _, t, h in rows]),
                         np.array([gl[0, h, t] for _, t, h in rows]),
                         np.stack([gi[0, h, t] for _, t, h in rows]))
    say(f"[conv] conv -> forward: {stats}")


def test_key_conv_rejects_bad_width(moba):
    k = torch.zeros(1, 64, 1, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):           # MOBA_ERR_UNSUPPORTED: width 9 > 8
        moba.key_short_conv(k, torch.zeros(1, 64, 9, device="cuda"), 16)
    with pytest.raises(ValueError):           # weight of the wrong shape
        moba.key_short_conv(k, torch.zeros(2, 64, 3, device="cuda"), 16)
