"""Attention-mask formulation of MoBA, for tiny inputs (T up to a few thousand).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The MoBA radar page (vibecrowd.fund, "How it works" and "Getting started") names a
naive variant built on attention masks next to the efficient one.  This module is our
own version of that idea, written independently of ``moba_oracle``: it forms the full
T x nb gate matrix, pins the current block with +inf and bans future blocks with -inf,
picks blocks with one stable argsort, expands the choice into a T x T boolean mask
and runs one dense masked softmax.  It shares no helper with ``moba_oracle``.
"""
from __future__ import annotations

import numpy as np


def moba_bruteforce(Q, K, V, B: int, topk: int, scale: float):
    """Q [b,T,Hq,d], K/V [b,T,Hkv,d] float64 -> (out, lse, idx) like moba_forward."""
    b, T, hq, d = Q.shape
    hkv = K.shape[2]
    G = hq // hkv
    nb = (T + B - 1) // B
    blk = np.arange(T) // B
    # block means through an indicator matrix: M[j, u] = 1/n_j if u in block j
    M = np.zeros((nb, T))
    M[blk, np.arange(T)] = 1.0
    M /= M.sum(axis=1, keepdims=True)
    out = np.empty_like(Q)
    lse = np.empty((b, hq, T))
    idx = np.full((b, hq, T, topk), -1, np.int32)
    jj = np.arange(nb)
    for bi in range(b):
        for h in range(hq):
            Kh, Vh = K[bi, :, h // G], V[bi, :, h // G]
            C = M @ Kh                                  # [nb, d]
            gate = Q[bi, :, h] @ C.T                    # [T, nb]
            gate = np.where(jj[None, :] == blk[:, None], np.inf, gate)
            gate = np.where(jj[None, :] > blk[:, None], -np.inf, gate)
            order = np.argsort(-gate, axis=1, kind="stable")
            keep = np.minimum(topk, blk + 1)            # causal blocks available
            chosen = np.zeros((T, nb), bool)
            for t in range(T):
                chosen[t, order[t, :keep[t]]] = True
                sel = np.nonzero(chosen[t])[0]
                idx[bi, h, t, :sel.size] = sel
            mask = chosen[:, blk] & (np.arange(T)[None, :] <= np.arange(T)[:, None])
            z = scale * (Q[bi, :, h] @ Kh.T)
            z = np.where(mask, z, -np.inf)
            zmax = z.max(axis=1, keepdims=True)
            e = np.exp(z - zmax)
            den = e.sum(axis=1, keepdims=True)
            out[bi, :, h] = (e / den) @ Vh
            lse[bi, h] = zmax[:, 0] + np.log(den[:, 0])
    return out, lse, idx


def moba_bruteforce_packed(Q, K, V, cu, B: int, topk: int, scale: float):
    """Packed sequences, Q [total,Hq,d], K/V [total,Hkv,d], cu [nseq+1] -> (out
    [total,Hq,d], lse [Hq,total], idx [Hq,total,topk]) from one mask over the packed
    tokens: one gate matrix over the blocks of every sequence, with the blocks of other
    sequences banned like future ones."""
    total, hq, d = Q.shape
    hkv = K.shape[1]
    G = hq // hkv
    cu = np.asarray(cu, dtype=np.int64)
    seq = np.searchsorted(cu, np.arange(total), side="right") - 1   # sequence of a token
    pos = np.arange(total) - cu[seq]                                 # position in it
    # global blocks: (sequence, local block), numbered in token order
    key = seq * (total + 1) + pos // B
    uniq, gblk = np.unique(key, return_inverse=True)
    nbg = uniq.size
    gseq = uniq // (total + 1)
    glocal = uniq % (total + 1)
    M = np.zeros((nbg, total))
    M[gblk, np.arange(total)] = 1.0
    M /= M.sum(axis=1, keepdims=True)
    out = np.empty_like(Q)
    lse = np.empty((hq, total))
    idx = np.full((hq, total, topk), -1, np.int32)
    same = seq[:, None] == seq[None, :]
    for h in range(hq):
        Kh, Vh = K[:, h // G], V[:, h // G]
        gate = Q[:, h] @ (M @ Kh).T                                   # [total, nbg]
        own = gseq[None, :] == seq[:, None]
        cur = gblk[:, None] == np.arange(nbg)[None, :]
        later = glocal[None, :] > (pos // B)[:, None]
        gate = np.where(cur, np.inf, gate)
        gate = np.where(~own | (own & later), -np.inf, gate)
        order = np.argsort(-gate, axis=1, kind="stable")
        keep = np.minimum(topk, pos // B + 1)
        chosen = np.zeros((total, nbg), bool)
        for t in range(total):
            chosen[t, order[t, :keep[t]]] = True
            sel = np.sort(glocal[np.nonzero(chosen[t])[0]])
            idx[h, t, :sel.size] = sel
        mask = chosen[:, gblk] & same & (pos[None, :] <= pos[:, None])
        z = scale * (Q[:, h] @ Kh.T)
        z = np.where(mask, z, -np.inf)
        zmax = z.max(axis=1, keepdims=True)
        e = np.exp(z - zmax)
        den = e.sum(axis=1, keepdims=True)
        out[:, h] = (e / den) @ Vh
        lse[h] = zmax[:, 0] + np.log(den[:, 0])
    return out, lse, idx
