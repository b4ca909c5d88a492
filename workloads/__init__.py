"""Seeded synthetic inputs for MoBA prefill, shared by the tests, the bench and smoke().

This module only draws random numbers and rounds them to bfloat16.  It holds none of
the method's arithmetic (no pooling for routing, no scoring, no top-k, no softmax),
so neither the CPU oracle nor the HIP path can share a mistake through it.

bfloat16 values are carried as ``numpy.uint16`` bit patterns (numpy has no bf16
dtype).  ``bf16_to_f64`` widens them exactly, ``to_torch_bf16`` hands them to torch.

Workloads follow the attention shape of Llama-3.1-8B (32 query heads in GQA over 8
KV heads, head_dim 128), which the MoBA paper continues to train to 1M tokens (page
"MoBA: Mixture of Block Attention for Long-Context LLMs", atlas.scime.ai, Approach and
Key results).  No weights are used; only the shape.

Random streams: ``numpy.random.default_rng([seed, tensor_id, head])`` with
tensor_id Q=0, K=1, V=2, key offsets=3, planted blocks=4, query noise=5, output gradient=6.  Each head
is drawn on its own, so any head can be regenerated alone.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, asdict

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get_workload", "make_inputs", "f32_to_bf16_bits",
    "bf16_to_f64", "bf16_to_f32", "to_torch_bf16", "small_workload", "make_output_grad",
]

Q_ID, K_ID, V_ID, OFFSET_ID, PLANT_ID, NOISE_ID, DOUT_ID = 0, 1, 2, 3, 4, 5, 6


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    hq: int
    hkv: int
    head_dim: int
    seqlen: int
    block: int
    topk: int
    recipe: str            # "iid" | "offset" | "planted"
    seed: int
    scale: float = field(default=float("nan"))
    description: str = ""

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim) if math.isnan(self.scale) else self.scale

    @property
    def num_blocks(self) -> int:
        return -(-self.seqlen // self.block)

    def as_dict(self) -> dict:
        d = asdict(self)
        d["scale"] = self.sm_scale
        return d


# The five workloads.  Sizes, head layout, block size and top-k are those of the
# benchmark plan; the value recipes are explained in make_inputs.
WORKLOADS = {
    "tiny_2k": Workload(
        "tiny_2k", 1, 1, 1, 64, 2048, 128, 4, "iid", seed=1,
        description="1 q-head / 1 kv-head, d=64, T=2048, B=128 (16 blocks), top-k=4"),
    "llama8b_32k": Workload(
        "llama8b_32k", 1, 32, 8, 128, 32768, 512, 3, "iid", seed=2,
        description="32 q-heads / 8 kv-heads, d=128, T=32768, B=512 (64 blocks), top-k=3"),
    "llama8b_128k": Workload(
        "llama8b_128k", 1, 32, 8, 128, 131072, 4096, 12, "offset", seed=3,
        description="32 q-heads / 8 kv-heads, d=128, T=131072, B=4096 (32 blocks), top-k=12"),
    "llama8b_64k_b128": Workload(
        "llama8b_64k_b128", 1, 32, 8, 128, 65536, 128, 16, "planted", seed=4,
        description="32 q-heads / 8 kv-heads, d=128, T=65536, B=128 (512 blocks), top-k=16"),
    "llama8b_1m": Workload(
        "llama8b_1m", 1, 32, 8, 128, 1048576, 4096, 12, "offset", seed=5,
        description="32 q-heads / 8 kv-heads, d=128, T=1048576, B=4096 (256 blocks), top-k=12"),
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def small_workload(name, batch, hq, hkv, head_dim, seqlen, block, topk, recipe="iid",
                   seed=0, scale=float("nan")) -> Workload:
    """A custom (usually small) workload for tests."""
    return Workload(name, batch, hq, hkv, head_dim, seqlen, block, topk, recipe, seed,
                    scale)


# ----------------------------------------------------------------------------- bf16
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, round-to-nearest-even, returned as uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    return bf16_to_f32(bits).astype(np.float64)


def to_torch_bf16(bits: np.ndarray, device="cpu"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device) if device != "cpu" else t


# ----------------------------------------------------------------------------- draws
def _rng(seed, tensor_id, head):
    return np.random.default_rng([int(seed), int(tensor_id), int(head)])


def _normal_heads(w: Workload, tensor_id: int, nheads: int) -> np.ndarray:
    """[batch, T, nheads, d] float32 N(0,1), one stream per head."""
    out = np.empty((w.batch, w.seqlen, nheads, w.head_dim), np.float32)
    for h in range(nheads):
        out[:, :, h, :] = _rng(w.seed, tensor_id, h).standard_normal(
            (w.batch, w.seqlen, w.head_dim), dtype=np.float32)
    return out


def _bf16_heads(w: Workload, tensor_id: int, nheads: int, mu=None) -> np.ndarray:
    """[batch, T, nheads, d] bf16 bits of N(0,1) draws, one stream per head, the same
    values as rounding _normal_heads(...) (+ the key offsets mu [b, nb, nheads, d] when
    given).  Heads are drawn in parallel threads (numpy's generators and array
    arithmetic run without the interpreter lock), one head's float32 at a time each."""
    out = np.empty((w.batch, w.seqlen, nheads, w.head_dim), np.uint16)

    def one(h):
        x = _rng(w.seed, tensor_id, h).standard_normal(
            (w.batch, w.seqlen, w.head_dim), dtype=np.float32)
        if mu is not None:
            for j in range(w.num_blocks):
                x[:, j * w.block:(j + 1) * w.block] += mu[:, j, h][:, None, :]
        out[:, :, h, :] = f32_to_bf16_bits(x)

    workers = max(1, min(16, os.cpu_count() or 1, nheads))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(one, range(nheads)))
    return out


def _key_offsets(w: Workload) -> np.ndarray:
    """[batch, nb, hkv, d] float32: a per-(kv-head, block) key mean offset, N(0, 0.5^2)."""
    nb = w.num_blocks
    mu = np.empty((w.batch, nb, w.hkv, w.head_dim), np.float32)
    for g in range(w.hkv):
        mu[:, :, g, :] = 0.5 * _rng(w.seed, OFFSET_ID, g).standard_normal(
            (w.batch, nb, w.head_dim), dtype=np.float32)
    return mu


def _distinct_earlier_blocks(rng, c: np.ndarray, m: int) -> np.ndarray:
    """For each row with current block c[i], up to m distinct block ids drawn uniformly
    from [0, c[i]) (all of them when c[i] <= m), padded with -1.  Floyd's sampling,
    vectorised over rows."""
    n = c.shape[0]
    out = np.full((n, m), -1, np.int64)
    # rows with c <= m take every earlier block
    small = c <= m
    ar = np.arange(m)
    out[small] = np.where(ar[None, :] < c[small, None], ar[None, :], -1)
    big = np.nonzero(~small)[0]
    if big.size:
        cb = c[big]
        chosen = np.full((big.size, m), -1, np.int64)
        for i in range(m):
            j = cb - m + i                       # Floyd: j runs over c-m .. c-1
            r = (rng.random(big.size) * (j + 1)).astype(np.int64)
            r = np.minimum(r, j)
            dup = (chosen[:, :i] == r[:, None]).any(axis=1) if i else np.zeros(big.size, bool)
            chosen[:, i] = np.where(dup, j, r)
        out[big] = chosen
    return out


def make_inputs(w: Workload, heads_only=None):
    """Draw the inputs of workload ``w``.

    Returns a dict with uint16 bf16 bit arrays ``q`` [b,T,Hq,d], ``k`` and ``v``
    [b,T,Hkv,d], plus the scalars.

    Recipes:
      iid      Q, K, V i.i.d. N(0,1).
      offset   as iid, and every key gets a mean offset mu[kv-head, block] with
               mu ~ N(0, 0.5^2 I) drawn per (kv-head, block), so gate scores separate.
      planted  K, V i.i.d. N(0,1).  For each query row (t, h) with current block c,
               P = min(8, c) distinct blocks drawn from [0, c); m = mean over P of the
               blocks' mean key (kv-head h's group); q = sqrt(d) m/|m| + N(0, I).
               Rows in block 0 get q = N(0, I).  The routing target P is returned.
    """
    kb = _bf16_heads(w, K_ID, w.hkv, _key_offsets(w) if w.recipe == "offset" else None)
    vb = _bf16_heads(w, V_ID, w.hkv)
    out = {"k": kb, "v": vb, "workload": w}
    if w.recipe in ("iid", "offset"):
        qb = _bf16_heads(w, Q_ID, w.hq)
    elif w.recipe == "planted":
        qb, planted = _planted_queries(w, kb)
        out["planted"] = planted
    else:
        raise ValueError(f"unknown recipe {w.recipe!r}")
    out["q"] = qb
    return out


def _planted_queries(w: Workload, kb: np.ndarray):
    """Queries pointed at 8 earlier blocks (see make_inputs).  Uses the bf16 keys."""
    b, T, hkv, d, B = w.batch, w.seqlen, w.hkv, w.head_dim, w.block
    G = w.hq // w.hkv
    nb = w.num_blocks
    kf = bf16_to_f64(kb)
    # per-block mean key, [b, nb, hkv, d]; the last block may be partial
    bm = np.stack([kf[:, j * B:min((j + 1) * B, T)].mean(axis=1) for j in range(nb)], axis=1)
    del kf
    q = np.empty((b, T, w.hq, d), np.float32)
    planted = np.full((b, w.hq, T, 8), -1, np.int32)
    blk = np.arange(T) // B
    for h in range(w.hq):
        g = h // G
        rng_p = _rng(w.seed, PLANT_ID, h)
        rng_n = _rng(w.seed, NOISE_ID, h)
        for bi in range(b):
            P = _distinct_earlier_blocks(rng_p, blk, 8)            # [T, 8]
            valid = P >= 0
            cnt = valid.sum(axis=1)
            Pc = np.where(valid, P, 0)
            m = np.zeros((T, d))
            for p in range(8):
                m += bm[bi, Pc[:, p], g, :] * valid[:, p, None]
            m /= np.maximum(cnt, 1)[:, None]
            nrm = np.linalg.norm(m, axis=1)
            dirn = np.where((cnt > 0)[:, None], math.sqrt(d) * m / np.maximum(nrm, 1e-30)[:, None], 0.0)
            eps = rng_n.standard_normal((T, d), dtype=np.float32)
            q[bi, :, h, :] = (dirn + eps).astype(np.float32)
            planted[bi, h] = P.astype(np.int32)
    return f32_to_bf16_bits(q), planted


def make_output_grad(w: Workload) -> np.ndarray:
    """The upstream gradient dL/dout of a backward test or benchmark: [b,T,Hq,d] bf16
    bits of i.i.d. N(0,1), one stream per query head (tensor_id 6)."""
    return _bf16_heads(w, DOUT_ID, w.hq)
