"""Gradients of the SLA forward pass (dQ, dK, dV, dW), in fp64 with torch
autograd on the CPU.

TEST INFRASTRUCTURE ONLY: imported by tests/ and by the CPU baseline of the
measurements, never by the product path.  Shares nothing with the GPU library.

Source: the SLA article, section 三 (the backward pass splits like the
forward: FlashAttention gradients for the sparse part, linear-attention
gradients for the linear part).  The forward is written here at token
level, from the same definitions as oracle/sla_oracle.c (and pinned to it):
  O_s[r] = softmax over the keys u of the critical blocks of r's row of
           (q_r . k_u / sqrt(d)), applied to V;
  O_l[r] = sum_u m(r,u) (phi(q_r) . phi(k_u)) v_u / sum_u m(r,u) phi(q_r) . phi(k_u),
           m(r,u) = 1 when u's block is marginal for r's row (0 when the row
           has no marginal block: O_l = 0), phi = softmax over channels;
  O = O_s + O_l W^T.
The block labels come from the pooled scores and are held fixed: the
gradient flows through the attention and the linear branch, not through
the selection (reading: the article's backward treats the mask as given).
"""
from __future__ import annotations

import math

import numpy as np
import torch


def token_masks(mask: np.ndarray, N: int, blk: int = 64):
    """mask [BH, Nb, Nb] int8 labels -> (critical, marginal) [BH, N, N] bool."""
    blkid = np.arange(N) // blk
    m = np.asarray(mask).reshape(-1, mask.shape[-2], mask.shape[-1])
    lab = m[:, blkid][:, :, blkid]
    return torch.from_numpy(lab == 1), torch.from_numpy(lab == 0)


def forward_tokens(q, k, v, w, crit, marg):
    """q, k, v [BH, N, d] and w [d, d] fp64 torch tensors (may require grad);
    crit, marg [BH, N, N] bool.  Returns O [BH, N, d]."""
    d = q.shape[-1]
    s = q @ k.transpose(-1, -2) / math.sqrt(d)
    s = s.masked_fill(~crit, float("-inf"))
    has = crit.any(dim=-1, keepdim=True)
    p = torch.softmax(torch.where(has, s, torch.zeros_like(s)), dim=-1) * has
    o_s = p @ v
    a = (torch.softmax(q, dim=-1) @ torch.softmax(k, dim=-1).transpose(-1, -2)) * marg
    den = a.sum(dim=-1, keepdim=True)
    o_l = torch.where(den > 0, (a @ v) / torch.where(den > 0, den, torch.ones_like(den)), torch.zeros_like(den))
    return o_s + o_l @ w.transpose(0, 1)


def gradients(q, k, v, w, mask, dout, blk: int = 64):
    """q, k, v, dout [B, H, N, d], w [d, d] (numpy, any float), mask [B, H, Nb, Nb]
    int8.  Returns (out, dq, dk, dv, dw) as fp64 numpy arrays."""
    B, H, N, d = q.shape
    t = lambda x: torch.tensor(np.asarray(x, np.float64).reshape(B * H, N, d), requires_grad=True)
    tq, tk, tv = t(q), t(k), t(v)
    tw = torch.tensor(np.asarray(w, np.float64), requires_grad=True)
    crit, marg = token_masks(mask, N, blk)
    out = forward_tokens(tq, tk, tv, tw, crit, marg)
    g = torch.from_numpy(np.asarray(dout, np.float64).reshape(B * H, N, d))
    dq, dk, dv, dw = torch.autograd.grad(out, (tq, tk, tv, tw), g)
    shape = (B, H, N, d)
    return (out.detach().numpy().reshape(shape), dq.numpy().reshape(shape), dk.numpy().reshape(shape),
            dv.numpy().reshape(shape), dw.numpy())


def gradients_blocks(q, k, v, w, mask, dout, qblocks, kblocks, blk: int = 64):
    """Exact gradients of the SLA forward of ONE head at any N, on selected
    blocks.  q, k, v, dout: [N, d] (numpy, any float); w [d, d]; mask
    [Nb, Nb] int8 labels of this head.  Returns (dq_rows, dk_rows, dv_rows,
    dw_head): dq of the tokens of the query blocks `qblocks`, dk and dv of
    the tokens of the key blocks `kblocks` (each [len(rows), d], rows in
    ascending block order, a ragged last block shorter), and this head's dW.

    The same forward as forward_tokens, arranged so that only what these
    gradients depend on is built: the sparse softmax at token level for the
    query blocks in `qblocks` and for every query block that has one of
    `kblocks` critical (no other row's sparse output involves those keys),
    and the linear branch for all rows with its sums grouped by key block,
    H_i = sum over marginal j of phi(K_j)^T (V_j W^T), Z_i = sum of phi(K_j)
    (the token sums of forward_tokens, added block by block)."""
    N, d = q.shape
    Nb = -(-N // blk)
    Np = Nb * blk
    f64 = lambda x: torch.tensor(np.asarray(x, np.float64))
    pad = lambda x: torch.cat([x, torch.zeros(Np - N, d, dtype=torch.float64)]) if Np > N else x
    tq, tk, tv, tw = f64(q).requires_grad_(), f64(k).requires_grad_(), f64(v).requires_grad_(), f64(w).requires_grad_()
    g = pad(f64(dout))
    lab = torch.from_numpy(np.asarray(mask).astype(np.int64))
    crit = lab == 1
    marg = (lab == 0).to(torch.float64)

    # linear branch, all rows
    phq = torch.softmax(pad(tq), dim=-1).reshape(Nb, blk, d)
    valid = (torch.arange(Np) < N).to(torch.float64).reshape(Nb, blk, 1)
    phk = torch.softmax(pad(tk), dim=-1).reshape(Nb, blk, d) * valid
    vp = (pad(tv) @ tw.transpose(0, 1)).reshape(Nb, blk, d)
    hj = phk.transpose(1, 2) @ vp                        # [Nb, d, d]
    zj = phk.sum(dim=1)                                  # [Nb, d]
    Hi = (marg @ hj.reshape(Nb, d * d)).reshape(Nb, d, d)
    Zi = marg @ zj
    num = phq @ Hi                                       # [Nb, blk, d]
    den = (phq * Zi[:, None, :]).sum(dim=-1, keepdim=True)
    has = marg.sum(dim=1).reshape(Nb, 1, 1) > 0
    o_l = torch.where(has, num / torch.where(has, den, torch.ones_like(den)), torch.zeros_like(num))
    loss = (o_l.reshape(Np, d) * g).sum()

    # sparse branch, the query blocks that matter
    kset = set(int(j) for j in kblocks)
    rows_i = sorted(set(int(i) for i in qblocks) |
                    {i for i in range(Nb) if any(bool(crit[i, j]) for j in kset)})
    scale = 1.0 / math.sqrt(d)
    for i in rows_i:
        keys = [j for j in range(Nb) if bool(crit[i, j])]
        if not keys:
            continue
        r0, r1 = i * blk, min(N, (i + 1) * blk)
        ku = torch.cat([tk[j * blk:min(N, (j + 1) * blk)] for j in keys])
        vu = torch.cat([tv[j * blk:min(N, (j + 1) * blk)] for j in keys])
        p = torch.softmax(tq[r0:r1] @ ku.transpose(0, 1) * scale, dim=-1)
        loss = loss + ((p @ vu) * g[r0:r1]).sum()

    dq, dk, dv, dw = torch.autograd.grad(loss, (tq, tk, tv, tw))
    take = lambda x, blocks: np.concatenate([x[b * blk:min(N, (b + 1) * blk)].numpy() for b in sorted(blocks)])
    return take(dq, qblocks), take(dk, kblocks), take(dv, kblocks), dw.numpy()
