"""Mask-quality diagnostics, computed from the definitions in fp64.

TEST INFRASTRUCTURE ONLY: imported by tests/ (and the CPU baseline of the
diagnostics measurement), never by the product path.  Shares nothing with the
GPU library.

What is measured (synthetic analogues of the pages' observations):
  * block attention mass (SLA article, section 2: a few attention weights
    carry most of the mass, the "three worlds"): for query block i and key
    block j, the mean over the valid rows r of block i of the full softmax
    probability (over all N keys, scale 1/sqrt(d)) that row r puts on the
    valid keys of block j.  Each row of the matrix sums to 1.
  * per row of blocks, from the mass and the three-way labels: the mass on
    the critical blocks (recall), on the marginal and on the negligible ones;
  * the 95 % density (SVOO page, offline profiling: the smallest share of
    entries that covers 95 % of the cumulative attention mass), here at block
    granularity: the smallest number of key blocks, taken by decreasing
    mass, whose mass reaches 0.95, divided by Nb;
  * numerical rank of a row-softmax matrix and of what is left after its
    largest entries are removed (SLA article, section 2), by SVD.
"""
from __future__ import annotations

import numpy as np


def block_mass(q: np.ndarray, k: np.ndarray, blk: int = 64, blocks=None) -> np.ndarray:
    """q, k: [B, H, N, d].  Returns mass [B, H, Nb, Nb] (fp64), or, with
    `blocks` a list of (bh, i), an array [len(blocks), Nb] of those rows."""
    B, H, N, d = q.shape
    Nb = -(-N // blk)
    qf = np.asarray(q, dtype=np.float64).reshape(B * H, N, d)
    kf = np.asarray(k, dtype=np.float64).reshape(B * H, N, d)
    want = blocks if blocks is not None else [(bh, i) for bh in range(B * H) for i in range(Nb)]
    out = np.zeros((len(want), Nb))
    scale = 1.0 / np.sqrt(d)
    for x, (bh, i) in enumerate(want):
        r0, r1 = blk * i, min(N, blk * (i + 1))
        s = qf[bh, r0:r1] @ kf[bh].T * scale                  # [n_i, N] scores of the valid rows
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)                     # full softmax over the N keys
        per_block = np.add.reduceat(p, np.arange(0, N, blk), axis=1)   # [n_i, Nb]
        out[x] = per_block.mean(axis=0)
    if blocks is None:
        return out.reshape(B, H, Nb, Nb)
    return out


def row_quality(mass_row: np.ndarray, labels_row: np.ndarray) -> dict:
    """One row of blocks: mass on each class and the 95 % block density."""
    crit = float(mass_row[labels_row == 1].sum())
    marg = float(mass_row[labels_row == 0].sum())
    negl = float(mass_row[labels_row == -1].sum())
    order = np.sort(mass_row)[::-1]
    csum = np.cumsum(order)
    need = int(np.searchsorted(csum, 0.95 * csum[-1]) + 1)
    return {"critical": crit, "marginal": marg, "negligible": negl, "density95": need / len(mass_row)}


def numerical_rank(a: np.ndarray, rtol: float = 1e-6) -> int:
    """Number of singular values above rtol times the largest."""
    s = np.linalg.svd(np.asarray(a, dtype=np.float64), compute_uv=False)
    return int((s > rtol * s[0]).sum()) if s.size and s[0] > 0 else 0


def rank_split(q: np.ndarray, k: np.ndarray, top_share: float, rtol: float = 1e-6) -> dict:
    """q, k: [N, d] of one head.  Rank of P = softmax(q k^T / sqrt(d)) and of
    P with its largest top_share of entries set to zero."""
    s = np.asarray(q, np.float64) @ np.asarray(k, np.float64).T / np.sqrt(q.shape[1])
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    cut = np.quantile(p, 1.0 - top_share)
    rest = np.where(p > cut, 0.0, p)
    return {"rank_full": numerical_rank(p, rtol), "rank_rest": numerical_rank(rest, rtol)}
