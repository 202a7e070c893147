"""Dense softmax attention over the N valid tokens, in fp64 with torch on the
CPU: what the SLA forward computes when every key block is critical (SLA
article, section 三, with the critical share at 100 %: the sparse branch
attends every key, the marginal and negligible sets are empty, so the
linear branch and its projection contribute nothing).

TEST INFRASTRUCTURE ONLY: imported by tests/, never by the product path.
Shares nothing with the GPU library.  It exists because the plain C oracle
(sla_oracle.c) evaluates the same quantity one key at a time, which at the
HunyuanVideo shape (N = 118800) takes minutes per head on a sample of query
blocks; here the two products are library matrix products (fp64), the
softmax one library call per row.  Pinned to sla_oracle.c at rho_c = 1 in
tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def attention_rows(q, k, v, rows, blk: int = 64, chunk: int = 1024) -> np.ndarray:
    """q, k, v: [B, H, N, d] (any float dtype); rows: [n, 2] (b*H + h, query
    block) pairs.  Returns [n, blk, d] fp64: for each valid query token r of
    each listed block, sum_u softmax_u(q_r . k_u / sqrt(d)) v_u over all N
    keys; rows of a ragged last block past N are zero."""
    B, H, N, d = q.shape
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
    out = np.zeros((rows.shape[0], blk, d))
    scale = 1.0 / math.sqrt(d)
    for bh in np.unique(rows[:, 0]):
        b, h = divmod(int(bh), H)
        sel = np.nonzero(rows[:, 0] == bh)[0]
        qh = torch.from_numpy(np.asarray(q[b, h], np.float64))
        kh = torch.from_numpy(np.asarray(k[b, h], np.float64))
        vh = torch.from_numpy(np.asarray(v[b, h], np.float64))
        # the valid query tokens of the listed blocks, and where each one goes
        toks, dest = [], []
        for x in sel:
            i = int(rows[x, 1])
            r0, r1 = blk * i, min(N, blk * (i + 1))
            toks.append(np.arange(r0, r1))
            dest.append(np.stack([np.full(r1 - r0, x), np.arange(r1 - r0)], axis=1))
        toks = np.concatenate(toks)
        dest = np.concatenate(dest)
        for c in range(0, toks.size, chunk):
            t = torch.from_numpy(toks[c:c + chunk])
            p = torch.softmax((qh[t] @ kh.T) * scale, dim=-1)
            o = (p @ vh).numpy()
            dd = dest[c:c + chunk]
            out[dd[:, 0], dd[:, 1]] = o
    return out
