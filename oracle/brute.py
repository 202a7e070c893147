"""Token-level brute force of SLA for tiny N (numpy / Python, fp64).

TEST INFRASTRUCTURE ONLY.  A second, independent evaluation of the method of
the SLA article (techwalker.com, section 3): every (query token, key token)
pair is given the label of its (query block, key block) pair and handled by
that label.  Unlike the C oracle it

  - pools with math.fsum (the correctly rounded sum) and Fraction-free fp64;
  - scores blocks with math.fsum of the exact products;
  - ranks with Python's stable sorted() on the key (-score, block index);
  - evaluates the linear part in its quadratic form
        sum_u (phi(q).phi(k_u)) v_u / sum_u phi(q).phi(k_u)
    over marginal key tokens u, never forming phi(K)^T V.

It is O(N^2 d) and meant for N of a few hundred at most.
"""
from __future__ import annotations

import math

import numpy as np


def counts(Nb: int, rho_c: float, rho_n: float):
    kc = min(Nb, max(0, math.ceil(rho_c * Nb - 1e-9)))
    kn = min(Nb - kc, max(0, math.floor(rho_n * Nb + 1e-9)))
    return kc, kn


def pool(x: np.ndarray, blk: int) -> np.ndarray:
    N, d = x.shape
    Nb = -(-N // blk)
    out = np.empty((Nb, d), np.float32)
    for i in range(Nb):
        seg = x[i * blk:min(N, (i + 1) * blk)].astype(np.float64)
        for c in range(d):
            out[i, c] = np.float32(math.fsum(seg[:, c]) / seg.shape[0])
    return out


def labels(qp: np.ndarray, kp: np.ndarray, kc: int, kn: int) -> np.ndarray:
    Nb = qp.shape[0]
    lab = np.zeros((Nb, Nb), np.int8)
    for i in range(Nb):
        s = [math.fsum(float(a) * float(b) for a, b in zip(qp[i], kp[j])) for j in range(Nb)]
        order = sorted(range(Nb), key=lambda j: (-s[j], j))
        for j in order[:kc]:
            lab[i, j] = 1
        for j in order[Nb - kn:]:
            lab[i, j] = -1
    return lab


def softmax_rows(x: np.ndarray) -> np.ndarray:
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def forward_head(q, k, v, w, blk: int, rho_c: float, rho_n: float):
    """One head: q, k, v [N, d] -> (o, o_s, o_l, labels), o [N, d] fp64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    w = np.asarray(w, np.float64)
    N, d = q.shape
    Nb = -(-N // blk)
    kc, kn = counts(Nb, rho_c, rho_n)
    lab = labels(pool(q.astype(np.float32), blk), pool(k.astype(np.float32), blk), kc, kn)
    tok_lab = np.repeat(np.repeat(lab, blk, axis=0), blk, axis=1)[:N, :N]
    logits = q @ k.T / math.sqrt(d)
    phq = softmax_rows(q)
    phk = softmax_rows(k)
    kern = phq @ phk.T                                   # phi(q_r) . phi(k_u)
    o_s = np.zeros((N, d))
    o_l = np.zeros((N, d))
    for r in range(N):
        crit = tok_lab[r] == 1
        if crit.any():
            lg = logits[r, crit]
            p = np.exp(lg - lg.max())
            o_s[r] = (p / p.sum()) @ v[crit]
        marg = tok_lab[r] == 0
        if marg.any():
            a = kern[r, marg]
            o_l[r] = (a @ v[marg]) / a.sum()
    o = o_s + o_l @ w.T
    return o, o_s, o_l, lab


def forward(q, k, v, w, blk: int, rho_c: float, rho_n: float):
    """q, k, v [B, H, N, d] -> o [B, H, N, d] and labels [B, H, Nb, Nb]."""
    B, H, N, d = q.shape
    Nb = -(-N // blk)
    o = np.zeros((B, H, N, d))
    lab = np.zeros((B, H, Nb, Nb), np.int8)
    for b in range(B):
        for h in range(H):
            o[b, h], _, _, lab[b, h] = forward_head(q[b, h], k[b, h], v[b, h], w, blk, rho_c, rho_n)
    return o, lab
