"""The plain float64 definition of MoBA prefill forward, its gradient, packed sequences,
the short key convolution and the full-attention decode after a prefill.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the product.

Sources (cited by page and section):

* [Approach] "MoBA: Mixture of Block Attention for Long-Context LLMs", paper summary
  page (atlas.scime.ai), section "Approach": the KV sequence is partitioned into
  blocks, each block is scored by the inner product of the query with the block's
  mean-pooled key, and each query is routed to its top-k blocks together with its own
  current block, causally.
* [Gating] MoBA README (rpkg.in mirror), intro bullet "Parameter-less Gating
  Mechanism": the gate has no learned parameters.
* [Blocks] same README, bullet "Trainable Block Sparse Attention": each query attends
  only the keys/values of the blocks it selected.
* [Sparsity] paper summary page, "Key results": 62.5% sparsity at 128K tokens, which
  with 32 blocks is 1 - 12/32, so the current block counts inside top-k.
* [Switch] README intro bullet "Seamlessly Transition between Full and Sparse
  Attention": with every causal block selected the layer is full causal attention.

Readings where the pages are silent (each is listed with its reason in the design
notes): k counts the current block (k-1 history slots); the gate score is the raw
inner product (no softmax scale, no normalisation); the current block is forced, not
scored; future blocks are never selected; rows whose block index c satisfies
c + 1 <= k take every block 0..c; ties go to the lower block index; query head h uses
kv-head h // (Hq/Hkv); a partial last block is averaged over the tokens present; the
diagonal is included (key u <= query t); lse is the natural log of the sum of
exp(scale * q.k) over the attended keys.

Shapes: Q [b, T, Hq, d], K and V [b, T, Hkv, d] float64; out [b, T, Hq, d];
lse [b, Hq, T]; idx [b, Hq, T, topk] int32, ascending, padded with -1.
"""
from __future__ import annotations

import numpy as np


def num_blocks(T: int, B: int) -> int:
    """Number of key blocks when T tokens are cut into blocks of B [Approach]."""
    return -(-T // B)


def centroids(K: np.ndarray, B: int) -> np.ndarray:
    """Mean-pooled key of every block [Approach: "query-mean-pooled-key"].

    K [b, T, Hkv, d] -> C [b, Hkv, nb, d]; a partial last block is averaged over the
    tokens it has.
    """
    b, T, hkv, d = K.shape
    nb = num_blocks(T, B)
    C = np.empty((b, hkv, nb, d), np.float64)
    for j in range(nb):
        C[:, :, j, :] = K[:, j * B:min((j + 1) * B, T)].mean(axis=1)
    return C


def gate_scores_rows(Q: np.ndarray, C: np.ndarray, B: int, rows) -> list:
    """Gate scores of the given rows [Approach, Gating].

    For a row (bi, t, h) with current block c = t // B the score of history block
    j < c is the plain inner product <Q[bi,t,h], C[bi, h // G, j]>.  Returns a list of
    1-D arrays (length c each).
    """
    G = Q.shape[2] // C.shape[1]
    out = []
    for bi, t, h in rows:
        c = t // B
        out.append(C[bi, h // G, :c, :] @ Q[bi, t, h, :])
    return out


def select_rows(scores: list, cs, topk: int) -> list:
    """Block set S of every row [Approach, Sparsity].

    The current block c is always in S.  The other k-1 members are the history blocks
    j < c ranked by (score descending, block index ascending); when c + 1 <= k every
    block 0..c is taken.  Returns sorted lists.
    """
    sel = []
    for s, c in zip(scores, cs):
        if c + 1 <= topk:
            sel.append(list(range(c + 1)))
            continue
        j = np.arange(c)
        order = np.lexsort((j, -s))          # primary: -score, secondary: block id
        hist = sorted(int(x) for x in j[order[:topk - 1]])
        sel.append(hist + [c])
    return sel


def select_blocks(Q: np.ndarray, C: np.ndarray, B: int, topk: int) -> np.ndarray:
    """idx [b, Hq, T, topk] for every row: sorted S then -1 padding."""
    b, T, hq, d = Q.shape
    idx = np.full((b, hq, T, topk), -1, np.int32)
    G = hq // C.shape[1]
    nb = num_blocks(T, B)
    for bi in range(b):
        for h in range(hq):
            Cg = C[bi, h // G]
            for c in range(nb):
                t0, t1 = c * B, min((c + 1) * B, T)
                if c + 1 <= topk:
                    idx[bi, h, t0:t1, :c + 1] = np.arange(c + 1)
                    continue
                s = Q[bi, t0:t1, h, :] @ Cg[:c].T                # [rows, c]
                j = np.broadcast_to(np.arange(c), s.shape)
                order = np.lexsort((j, -s), axis=-1)[:, :topk - 1]
                hist = np.sort(order, axis=1)                    # ids == positions
                idx[bi, h, t0:t1, :topk - 1] = hist
                idx[bi, h, t0:t1, topk - 1] = c
    return idx


def attended_keys(S, t: int, B: int, T: int) -> np.ndarray:
    """Key positions N(t) a row attends [Blocks, Approach "(causal)"]:
    every key of each selected history block j < c, then the current block's keys
    c*B .. t (the diagonal included)."""
    c = t // B
    parts = [np.arange(j * B, min((j + 1) * B, T)) for j in S if j < c]
    parts.append(np.arange(c * B, t + 1))
    return np.concatenate(parts)


def attend_row(q: np.ndarray, Kg: np.ndarray, Vg: np.ndarray, keys: np.ndarray,
               scale: float, return_p: bool = False):
    """One softmax over the attended keys [Blocks].

    z_u = scale * q.K[u]; p = exp(z - max z) / sum; out = sum_u p_u V[u];
    lse = max z + ln sum exp(z - max z).
    """
    z = scale * (Kg[keys] @ q)
    m = z.max()
    e = np.exp(z - m)
    ssum = e.sum()
    out = (e @ Vg[keys]) / ssum
    lse = m + np.log(ssum)
    if return_p:
        return out, lse, e / ssum
    return out, lse


def attend_rows(Q, K, V, B: int, scale: float, rows, sels):
    """out [n, d] and lse [n] for the given rows and their block sets."""
    hq, hkv = Q.shape[2], K.shape[2]
    G = hq // hkv
    T = Q.shape[1]
    n = len(rows)
    out = np.empty((n, Q.shape[3]))
    lse = np.empty(n)
    for i, ((bi, t, h), S) in enumerate(zip(rows, sels)):
        keys = attended_keys(S, t, B, T)
        out[i], lse[i] = attend_row(Q[bi, t, h], K[bi, :, h // G], V[bi, :, h // G],
                                    keys, scale)
    return out, lse


def attend_parts_row(q, Kg, Vg, S, t: int, B: int, T: int, scale: float):
    """The (out, lse) of each part of a row separately: one per selected history block
    and one for the causal current block.  Used to check partial results and the
    log-sum-exp merge identity."""
    c = t // B
    parts = []
    for j in S:
        if j < c:
            keys = np.arange(j * B, min((j + 1) * B, T))
            parts.append(("hist", j) + attend_row(q, Kg, Vg, keys, scale))
    keys = np.arange(c * B, t + 1)
    parts.append(("cur", c) + attend_row(q, Kg, Vg, keys, scale))
    return parts


def merge_parts(outs, lses):
    """Log-sum-exp merge of softmax parts over disjoint key sets:
    L = ln sum_i exp(lse_i); out = sum_i exp(lse_i - L) out_i."""
    lses = np.asarray(lses, np.float64)
    m = lses.max()
    L = m + np.log(np.exp(lses - m).sum())
    w = np.exp(lses - L)
    return (w[:, None] * np.asarray(outs)).sum(axis=0), L


def moba_forward(Q, K, V, B: int, topk: int, scale: float):
    """The whole forward for small inputs: (out, lse, idx, C)."""
    b, T, hq, d = Q.shape
    C = centroids(K, B)
    idx = select_blocks(Q, C, B, topk)
    out = np.empty_like(Q)
    lse = np.empty((b, hq, T))
    G = hq // K.shape[2]
    for bi in range(b):
        for h in range(hq):
            Kg, Vg = K[bi, :, h // G], V[bi, :, h // G]
            for t in range(T):
                S = [int(j) for j in idx[bi, h, t] if j >= 0]
                keys = attended_keys(S, t, B, T)
                out[bi, t, h], lse[bi, h, t] = attend_row(Q[bi, t, h], Kg, Vg, keys, scale)
    return out, lse, idx, C


def moba_rows(Q, K, V, B: int, topk: int, scale: float, rows, C=None):
    """The forward on a sample of rows [(bi, t, h), ...]:
    returns (out [n,d], lse [n], sels (list of sorted S), scores (list))."""
    if C is None:
        C = centroids(K, B)
    scores = gate_scores_rows(Q, C, B, rows)
    sels = select_rows(scores, [t // B for _, t, _ in rows], topk)
    out, lse = attend_rows(Q, K, V, B, scale, rows, sels)
    return out, lse, sels, scores


def attended_pairs(T: int, B: int, topk: int) -> int:
    """Number of (query, key) pairs one query head attends, from the definition:
    min(c, k-1) full history blocks plus the causal part of the current block.
    (The last block may be partial.)"""
    total = 0
    nb = num_blocks(T, B)
    for c in range(nb):
        t0, t1 = c * B, min((c + 1) * B, T)
        n = t1 - t0
        hist = min(c, topk - 1)
        total += n * hist * B + n * (n + 1) // 2
    return total


# ----------------------------------------------------------------------------- backward
# The gradient of the layer's output with respect to Q, K and V, for the training use of
# MoBA ("Trainable Block Sparse Attention", README).  The block selection is a
# piecewise-constant function of Q and K (a top-k over inner products with mean keys,
# [Gating]: no parameters), so it contributes no gradient: the selection S of every row
# is held fixed, and each row's output is ordinary softmax attention over its attended
# keys N.  With z_u = scale q.k_u, p = softmax(z), o = sum_u p_u v_u and an upstream
# gradient g = dL/do (the lse output is taken to carry no gradient):
#   dv_u += p_u g,  dp_u = g.v_u,  dz_u = p_u (dp_u - g.o),
#   dq = scale sum_u dz_u k_u,  dk_u += scale dz_u q.

def attend_row_grad(q, Kg, Vg, keys, scale: float, g):
    """(dq [d], dk [len(keys), d], dv [len(keys), d]) of one row's attention."""
    z = scale * (Kg[keys] @ q)
    e = np.exp(z - z.max())
    p = e / e.sum()
    o = p @ Vg[keys]
    dp = Vg[keys] @ g
    dz = p * (dp - g @ o)
    dq = scale * (dz @ Kg[keys])
    dk = scale * np.outer(dz, q)
    dv = np.outer(p, g)
    return dq, dk, dv


def moba_backward(Q, K, V, dO, B: int, topk: int, scale: float, idx=None):
    """dQ, dK, dV (float64, shapes of Q, K, V) of sum(dO * out) with each row's block set
    fixed: the oracle's own selection, or ``idx`` [b, Hq, T, topk] when given."""
    b, T, hq, d = Q.shape
    hkv = K.shape[2]
    G = hq // hkv
    if idx is None:
        idx = select_blocks(Q, centroids(K, B), B, topk)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for bi in range(b):
        for h in range(hq):
            g = h // G
            Kg, Vg = K[bi, :, g], V[bi, :, g]
            for t in range(T):
                S = [int(j) for j in idx[bi, h, t] if j >= 0]
                keys = attended_keys(S, t, B, T)
                dq, dk, dv = attend_row_grad(Q[bi, t, h], Kg, Vg, keys, scale, dO[bi, t, h])
                dQ[bi, t, h] = dq
                dK[bi, keys, g] += dk
                dV[bi, keys, g] += dv
    return dQ, dK, dV


# --------------------------------------------------------------------- packed sequences
# Several sequences of different lengths packed along the token axis (cu = cumulative
# lengths).  Each sequence is its own MoBA problem ("Approach" of the paper summary,
# applied per sequence): its blocks start at its first token, its last block may be
# partial, and it routes and attends only within itself.

def moba_forward_varlen(Q, K, V, cu, B: int, topk: int, scale: float):
    """Q [total, Hq, d], K/V [total, Hkv, d] float64, cu [nseq + 1] ->
    (out [total, Hq, d], lse [Hq, total], idx [Hq, total, topk]), block ids counted
    within each sequence."""
    total, hq, d = Q.shape
    out = np.empty_like(Q)
    lse = np.empty((hq, total))
    idx = np.full((hq, total, topk), -1, np.int32)
    for s in range(len(cu) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        if e == a:
            continue
        o, l, i, _ = moba_forward(Q[None, a:e], K[None, a:e], V[None, a:e], B, topk, scale)
        out[a:e] = o[0]
        lse[:, a:e] = l[0]
        idx[:, a:e] = i[0]
    return out, lse, idx


# ------------------------------------------------------------------- key short convolution
# A short convolution of the keys inside each block before pooling (FlashMoBA story,
# paragraph on short convolutions).  Reading: depthwise and causal along tokens, per
# kv-head channel, with no tap reaching into the previous block.

def key_short_conv(K, W, B: int, cu=None):
    """K [b, T, Hkv, d] (or packed [total, Hkv, d] with cu), W [Hkv, d, w] float64 ->
    out like K: out[t, g, c] = sum over taps i with t - i in t's block of
    W[g, c, i] * K[t - i, g, c] (t counted within its sequence)."""
    if cu is not None:
        out = np.empty_like(K)
        for s in range(len(cu) - 1):
            a, e = int(cu[s]), int(cu[s + 1])
            if e > a:
                out[a:e] = key_short_conv(K[None, a:e], W, B)[0]
        return out
    b, T, hkv, d = K.shape
    w = W.shape[2]
    out = np.zeros_like(K)
    for t in range(T):
        start = (t // B) * B
        for i in range(w):
            if t - i < start:
                break
            out[:, t] += W[None, :, :, i] * K[:, t - i]
    return out


def moba_backward_varlen(Q, K, V, dO, cu, B: int, topk: int, scale: float):
    """dQ, dK, dV (float64, packed like Q, K, V) of packed sequences, each one the batch-1
    backward of its own sequence with the oracle's own selection."""
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for s in range(len(cu) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        if e == a:
            continue
        gq, gk, gv = moba_backward(Q[None, a:e], K[None, a:e], V[None, a:e], dO[None, a:e],
                                   B, topk, scale)
        dQ[a:e], dK[a:e], dV[a:e] = gq[0], gk[0], gv[0]
    return dQ, dK, dV


# ------------------------------------------------------------- full-attention decode
# After a MoBA prefill, generation switches to full attention (paper summary page,
# "Limitations"; README bullet "Seamlessly Transition between Full and Sparse
# Attention").  Reading: the n new query tokens are the last n positions of the key
# sequence, and each attends every key up to its own position.

def decode_attention(Q, K, V, scale: float):
    """Q [b, n, Hq, d], K and V [b, Tk, Hkv, d] float64 (Tk >= n): query i sits at
    position Tk - n + i and attends keys 0 .. Tk - n + i.  Returns out [b, n, Hq, d]
    and lse [b, Hq, n]."""
    b, n, hq, d = Q.shape
    Tk, hkv = K.shape[1], K.shape[2]
    G = hq // hkv
    out = np.empty_like(Q)
    lse = np.empty((b, hq, n))
    for bi in range(b):
        for h in range(hq):
            Kg, Vg = K[bi, :, h // G], V[bi, :, h // G]
            for i in range(n):
                keys = np.arange(Tk - n + i + 1)
                out[bi, i, h], lse[bi, h, i] = attend_row(Q[bi, i, h], Kg, Vg, keys, scale)
    return out, lse
