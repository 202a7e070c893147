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
