"""Full-attention decode (the hand-off after a MoBA prefill) on the GPU, through the C
ABI, against the float64 oracle ``oracle.decode_attention`` (pinned by
tests/test_oracle_decode.py).  Bar: out max |diff| <= 2e-2 and mean <= 2e-3, lse max
|diff| <= 1e-3, every row (bf16 inputs, fp32 accumulation, P rounded to bf16 for the
PV product, as in the forward).
"""
import sys

import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits, bf16_to_f64, to_torch_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

OUT_MAX, OUT_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def moba():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_sparse_long_pool_amd as m
    return m


def bits(seed, *shape):
    return f32_to_bf16_bits(np.random.default_rng(seed).standard_normal(shape,
                                                                        dtype=np.float32))


def dev(b):
    return to_torch_bf16(b, "cuda")


def check(go, gl, ro, rl, label):
    err = np.abs(go - ro)
    s = {"out_max": float(err.max()), "out_mean": float(err.mean()),
         "lse_max": float(np.abs(gl - rl).max())}
    say(f"       {label}: {s}")
    assert s["out_max"] <= OUT_MAX and s["out_mean"] <= OUT_MEAN and s["lse_max"] <= LSE_MAX, s


@pytest.mark.parametrize("b,n,Tk,hq,hkv,d", [
    (1, 1, 4096, 32, 8, 128),      # one new token, Llama-3.1-8B heads
    (2, 3, 1000, 8, 2, 128),       # three new tokens, a ragged last subtile
    (1, 8, 257, 4, 1, 64),         # G*n = 32 rows, d = 64
    (1, 4, 31, 8, 8, 128),         # a cache shorter than one 32-key subtile
    (1, 1, 1, 4, 2, 128),          # a single key
    (3, 2, 5000, 16, 4, 64),
    (1, 32, 700, 1, 1, 128),       # G = 1, 32 new tokens
    (1, 1, 20000, 32, 1, 128),     # G = 32
    (1, 33, 500, 1, 1, 128),       # 33 rows: two row tiles, the second with one row
    (1, 1, 3000, 64, 1, 128),      # G = 64: two row tiles of one new token
    (2, 16, 2000, 8, 2, 64),       # 128 rows per kv-head: four row tiles
])
def test_decode_all_rows(moba, b, n, Tk, hq, hkv, d):
    say(f"[decode] b={b} n={n} Tk={Tk} hq={hq} hkv={hkv} d={d}")
    qb, kb, vb = bits(Tk + n, b, n, hq, d), bits(Tk + 1, b, Tk, hkv, d), bits(Tk + 2, b, Tk, hkv, d)
    sc = 1.0 / np.sqrt(d)
    out, lse = moba.decode(dev(qb), dev(kb), dev(vb), sc)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_attention(bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb), sc)
    check(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, "all rows")


def test_decode_after_moba_prefill(moba):
    """The hand-off: a MoBA prefill over T tokens, then full-attention decode of two more
    tokens against the same K/V cache extended by their keys.  The decode also equals
    the last rows of dense causal attention over the whole T + 2 tokens."""
    T, n, hq, hkv, d, B, k = 4094, 2, 8, 2, 128, 256, 4   # dense_forward wants 16 | T + n
    Tk = T + n
    qb, kb, vb = bits(1, 1, Tk, hq, d), bits(2, 1, Tk, hkv, d), bits(3, 1, Tk, hkv, d)
    q, kk, v = dev(qb), dev(kb), dev(vb)
    moba.forward(q[:, :T].contiguous(), kk[:, :T].contiguous(), v[:, :T].contiguous(), B, k)
    out, lse = moba.decode(q[:, T:].contiguous(), kk, v)
    dense_out, dense_lse = moba.dense_forward(q, kk, v)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_attention(bf16_to_f64(qb[:, T:]), bf16_to_f64(kb), bf16_to_f64(vb),
                                     1.0 / np.sqrt(d))
    check(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, "decode vs oracle")
    check(out.float().cpu().numpy(), lse.cpu().numpy(),
          dense_out[:, T:].float().cpu().numpy(), dense_lse[:, :, T:].cpu().numpy(),
          "decode vs dense causal prefill")


def test_decode_128k_llama8b(moba):
    """One new token against a 128K cache (Llama-3.1-8B heads), every head's row."""
    Tk, hq, hkv, d = 131072, 32, 8, 128
    say(f"[decode] 128K cache: generating inputs")
    qb, kb, vb = bits(11, 1, 1, hq, d), bits(12, 1, Tk, hkv, d), bits(13, 1, Tk, hkv, d)
    out, lse = moba.decode(dev(qb), dev(kb), dev(vb))
    torch.cuda.synchronize()
    say(f"[decode] 128K cache: oracle")
    ro, rl = oracle.decode_attention(bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb),
                                     1.0 / np.sqrt(d))
    check(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, "128K")


def test_decode_deterministic(moba):
    qb, kb, vb = bits(21, 1, 4, 8, 128), bits(22, 1, 3000, 2, 128), bits(23, 1, 3000, 2, 128)
    a = moba.decode(dev(qb), dev(kb), dev(vb))
    c = moba.decode(dev(qb), dev(kb), dev(vb))
    torch.cuda.synchronize()
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])


def test_decode_rejects_bad_args(moba):
    k = dev(bits(31, 1, 64, 1, 128))
    with pytest.raises(ValueError):            # G * n = 2048 > 1024 rows
        moba.decode(dev(bits(32, 1, 2, 1024, 128)), k, k)
    with pytest.raises(ValueError):            # more new tokens than cached keys
        moba.decode(dev(bits(33, 1, 65, 1, 128)), k, k)
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(moba.MobaError):
        moba.decode(dev(bits(34, 1, 1, 4, 128)), dev(bits(35, 1, 5000, 1, 128)),
                    dev(bits(36, 1, 5000, 1, 128)), workspace=small)
