"""Sparse attention over key-block lists given per query-block row, from the
definition in fp64 (the block-sparse softmax of the LVSA page's method
steps: one softmax over the union of the listed blocks' keys, scale
1/sqrt(d), keys past N excluded, no linear branch).

TEST INFRASTRUCTURE ONLY: imported by tests/ and the CPU baseline of the
measurements, never by the product path.  Shares nothing with the GPU library.
"""
from __future__ import annotations

import numpy as np


def row_blocks(lists: np.ndarray, counts: np.ndarray, bh: int, i: int, Nb: int) -> list:
    """The distinct valid key blocks of row (bh, i): the first counts entries,
    those in [0, Nb), each once, ascending."""
    c = int(max(0, min(int(counts[bh, i]), lists.shape[-1])))
    return sorted({int(j) for j in lists[bh, i, :c] if 0 <= int(j) < Nb})


def attention_lists(q, k, v, lists, counts, blk: int = 64, rows=None) -> np.ndarray:
    """q, k, v: [B, H, N, d]; lists: [B, H, Nb, kmax]; counts: [B, H, Nb].
    Returns out [B, H, N, d] fp64, or with rows = [(bh, i), ...] an array
    [len(rows), blk, d] holding those query blocks (pad rows zero)."""
    B, H, N, d = q.shape
    Nb = -(-N // blk)
    qf = np.asarray(q, np.float64).reshape(B * H, N, d)
    kf = np.asarray(k, np.float64).reshape(B * H, N, d)
    vf = np.asarray(v, np.float64).reshape(B * H, N, d)
    L = np.asarray(lists).reshape(B * H, Nb, -1)
    C = np.asarray(counts).reshape(B * H, Nb)
    want = rows if rows is not None else [(bh, i) for bh in range(B * H) for i in range(Nb)]
    res = np.zeros((len(want), blk, d))
    for x, (bh, i) in enumerate(want):
        r0, r1 = blk * i, min(N, blk * (i + 1))
        keys = [u for j in row_blocks(L, C, bh, i, Nb) for u in range(blk * j, min(N, blk * (j + 1)))]
        if not keys:
            continue
        s = qf[bh, r0:r1] @ kf[bh, keys].T / np.sqrt(d)
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        res[x, :r1 - r0] = p @ vf[bh, keys]
    if rows is not None:
        return res
    out = np.zeros((B * H, Nb * blk, d))
    for x, (bh, i) in enumerate(want):
        out[bh, blk * i:blk * (i + 1)] = res[x]
    return out[:, :N].reshape(B, H, N, d)
