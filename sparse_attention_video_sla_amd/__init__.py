"""SLA sparse-linear attention forward for MI355X (gfx950).

Thin binding over the C ABI of libsla.so (include/sla.h): it checks tensor
placement and layout, allocates outputs and workspace with torch on the
current device, and passes raw pointers plus the current HIP stream.  Every
step of the computation runs in the library's HIP kernels.

    out = forward(q, k, v, w, crit_frac=0.05, negl_frac=0.10)

q, k, v: [B, H, N, d] bf16 or float32 on the GPU; w: [d, d] float32.
"""
from __future__ import annotations

import ctypes
from typing import Optional

from . import _lib

__all__ = ["counts", "workspace_size", "pool", "classify", "forward", "forward_lists", "lvsa_plan", "lvsa_sets", "forward_lvsa", "sta_tile_order", "forward_sta", "backward", "forward_save", "backward_saved", "SavedForward",
           "block_mass", "mask_stats", "version",
           "SlaError"]

SlaError = _lib.SlaError


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return _lib.SLA_BF16
    if t.dtype == torch.float32:
        return _lib.SLA_F32
    raise TypeError("unsupported dtype %s (bfloat16 or float32)" % t.dtype)


def _stream_ptr(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _check_gpu(*ts) -> None:
    dev = ts[0].device
    for t in ts:
        if t.device.type != "cuda":
            raise ValueError("tensors must be on the GPU")
        if t.device != dev:
            raise ValueError("tensors must be on one device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def version() -> int:
    return _lib.load().sla_version()


def counts(Nb: int, crit_frac: float, negl_frac: float):
    """(k_c, k_n): critical and negligible key blocks per query-block row."""
    kc, kn = ctypes.c_int(), ctypes.c_int()
    _lib.check(_lib.load().sla_counts(Nb, crit_frac, negl_frac, ctypes.byref(kc), ctypes.byref(kn)))
    return kc.value, kn.value


def workspace_size(B: int, H: int, N: int, d: int, dtype: str = "bf16", crit_frac: float = 0.05,
                   negl_frac: float = 0.10, block: int = 64) -> int:
    code = {"bf16": _lib.SLA_BF16, "f32": _lib.SLA_F32}[dtype]
    n = ctypes.c_size_t()
    _lib.check(_lib.load().sla_workspace_size(B, H, N, d, block, code, crit_frac, negl_frac, ctypes.byref(n)))
    return n.value


def pool(q, k, block: int = 64):
    """Block means of q and k: two [B, H, Nb, d] float32 tensors."""
    torch = _torch()
    _check_gpu(q, k)
    if q.shape != k.shape or q.dtype != k.dtype:
        raise ValueError("q and k must have one shape and dtype")
    B, H, N, d = q.shape
    Nb = -(-N // block)
    qp = torch.empty((B, H, Nb, d), dtype=torch.float32, device=q.device)
    kp = torch.empty_like(qp)
    _lib.check(_lib.load().sla_pool(q.data_ptr(), k.data_ptr(), _dtype_code(q), B, H, N, d, block,
                                    qp.data_ptr(), kp.data_ptr(), _stream_ptr(q.device)))
    return qp, kp


def classify(qp, kp, crit_frac: float = 0.05, negl_frac: float = 0.10, want_excl: bool = False,
             want_pc: bool = False) -> dict:
    """Labels of the compressed map: mask [B,H,Nb,Nb] int8 (+1/0/-1), the
    ascending critical list [B,H,Nb,k_c] and optionally the excluded list and P_c."""
    torch = _torch()
    _check_gpu(qp, kp)
    if qp.dtype != torch.float32 or kp.dtype != torch.float32 or qp.shape != kp.shape:
        raise ValueError("pooled inputs must be float32 of one shape")
    B, H, Nb, d = qp.shape
    kc, kn = counts(Nb, crit_frac, negl_frac)
    dev = qp.device
    mask = torch.empty((B, H, Nb, Nb), dtype=torch.int8, device=dev)
    crit = torch.empty((B, H, Nb, kc), dtype=torch.int32, device=dev)
    excl = torch.empty((B, H, Nb, kc + kn), dtype=torch.int32, device=dev) if want_excl else None
    pc = torch.empty((B, H, Nb, Nb), dtype=torch.float32, device=dev) if want_pc else None
    _lib.check(_lib.load().sla_classify(qp.data_ptr(), kp.data_ptr(), B, H, Nb, d, crit_frac, negl_frac,
                                        mask.data_ptr(), crit.data_ptr() if kc > 0 else None,
                                        excl.data_ptr() if excl is not None and excl.numel() else None,
                                        pc.data_ptr() if pc is not None else None, _stream_ptr(dev)))
    out = dict(mask=mask, crit=crit, k_c=kc, k_n=kn)
    if want_excl:
        out["excl"] = excl
    if want_pc:
        out["pc"] = pc
    return out


def forward(q, k, v, w, crit_frac: float = 0.05, negl_frac: float = 0.10, block: int = 64,
            out_dtype=None, return_mask: bool = False, workspace=None, out=None):
    """SLA forward: O = sparse softmax attention over the critical blocks +
    (linear attention over the marginal blocks) W^T.  Returns out [B,H,N,d]
    (float32 by default) or (out, mask) with return_mask."""
    torch = _torch()
    _check_gpu(q, k, v, w)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must have one shape and dtype")
    B, H, N, d = q.shape
    if w.dtype != torch.float32 or tuple(w.shape) != (d, d):
        raise ValueError("w must be float32 [d, d]")
    in_code = _dtype_code(q)
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    out_code = _lib.SLA_F32 if out_dtype == torch.float32 else _dtype_code(torch.empty(0, dtype=out_dtype))
    dev = q.device
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=dev)
    elif out.shape != q.shape or out.dtype != out_dtype or not out.is_contiguous() or out.device != dev:
        raise ValueError("out must be a contiguous [B,H,N,d] tensor of out_dtype on q's device")
    Nb = -(-N // block)
    mask = torch.empty((B, H, Nb, Nb), dtype=torch.int8, device=dev) if return_mask else None
    need = workspace_size(B, H, N, d, "bf16" if in_code == _lib.SLA_BF16 else "f32", crit_frac, negl_frac, block)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _lib.check(_lib.load().sla_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), w.data_ptr(), in_code, out_code,
                                       B, H, N, d, block, crit_frac, negl_frac, _lib.SLA_PHI_SOFTMAX,
                                       out.data_ptr(), mask.data_ptr() if mask is not None else None,
                                       workspace.data_ptr(), workspace.numel(), _stream_ptr(dev)))
    return (out, mask) if return_mask else out


def forward_noalloc(q, k, v, w, out, crit_frac: float = 0.05, negl_frac: float = 0.10, block: int = 64,
                    mask_out=None):
    """sla_forward_noalloc: the forward pass of `forward` into the caller's
    `out` (and optional int8 `mask_out` [B,H,Nb,Nb]), with the library's
    static scratch array instead of a workspace; nothing is allocated."""
    torch = _torch()
    _check_gpu(q, k, v, w, out)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must have one shape and dtype")
    B, H, N, d = q.shape
    if w.dtype != torch.float32 or tuple(w.shape) != (d, d):
        raise ValueError("w must be float32 [d, d]")
    if out.shape != q.shape or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous [B,H,N,d] tensor on q's device")
    Nb = -(-N // block)
    if mask_out is not None and (tuple(mask_out.shape) != (B, H, Nb, Nb) or mask_out.dtype != torch.int8
                                 or not mask_out.is_contiguous()):
        raise ValueError("mask_out must be a contiguous int8 [B,H,Nb,Nb] tensor")
    out_code = _lib.SLA_F32 if out.dtype == torch.float32 else _dtype_code(out)
    _lib.check(_lib.load().sla_forward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), w.data_ptr(),
                                               _dtype_code(q), out_code, B, H, N, d, block, crit_frac, negl_frac,
                                               _lib.SLA_PHI_SOFTMAX, out.data_ptr(),
                                               mask_out.data_ptr() if mask_out is not None else None,
                                               _stream_ptr(q.device)))
    return out


def lvsa_plan(T: int, C: int, W: int):
    """(T_per, |G_s|, frames per set) of the LVSA frame sets (host arithmetic)."""
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _lib.check(_lib.load().sla_lvsa_plan(T, C, W, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def lvsa_sets(T: int, C: int, W: int, step: int, device="cuda"):
    """LVSA frame sets A(t) built on the device: (sets [T, F] int32, counts
    [T] int32), frame t's set ascending in its first counts[t] entries."""
    torch = _torch()
    F = lvsa_plan(T, C, W)[2]
    sets = torch.full((T, F), -1, dtype=torch.int32, device=device)
    cnt = torch.empty(T, dtype=torch.int32, device=device)
    _lib.check(_lib.load().sla_lvsa_sets(T, C, W, step, sets.data_ptr(), cnt.data_ptr(), F,
                                         _stream_ptr(torch.device(device))))
    return sets, cnt


def forward_lvsa(q, k, v, T: int, C: int, W: int, step: int, out_dtype=None, out=None, workspace=None,
                 block: int = 64):
    """LVSA frame-level sparse attention (linear branch off): the sequence is
    T frames of N / T tokens; every query token of frame t attends the tokens
    of the frames in A(t) = G_step U W(t)."""
    torch = _torch()
    _check_gpu(q, k, v)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must have one shape and dtype")
    B, H, N, d = q.shape
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    out_code = _lib.SLA_F32 if out_dtype == torch.float32 else _dtype_code(torch.empty(0, dtype=out_dtype))
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    L = _lib.load()
    n = ctypes.c_size_t()
    _lib.check(L.sla_lvsa_workspace_size(B, H, N, T, C, W, ctypes.byref(n)))
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=q.device)
    _lib.check(L.sla_forward_lvsa(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), out_code, B, H, N, d,
                                  block, T, C, W, step, out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                  _stream_ptr(q.device)))
    return out


def lvsa_workspace_size(B: int, H: int, N: int, T: int, C: int, W: int) -> int:
    n = ctypes.c_size_t()
    _lib.check(_lib.load().sla_lvsa_workspace_size(B, H, N, T, C, W, ctypes.byref(n)))
    return n.value


def sta_tile_order(grid, tile):
    """numpy int32 [N]: perm[m] = raster index of the m-th token in the
    tile-major order sla_forward_sta takes (host arithmetic)."""
    import numpy as np
    F, Hh, Ww = grid
    perm = np.empty(F * Hh * Ww, dtype=np.int32)
    _lib.check(_lib.load().sla_sta_tile_order(F, Hh, Ww, *tile, perm.ctypes.data))
    return perm


def forward_sta(q, k, v, grid, tile, window, out_dtype=None, out=None, workspace=None, block: int = 64):
    """Sliding tile attention (linear branch off) over q, k, v [B, H, N, d]
    in tile-major order (sta_tile_order); grid (F, Hh, Ww), tile and window
    per axis.  Returns out [B, H, N, d] in the same order."""
    torch = _torch()
    _check_gpu(q, k, v)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must have one shape and dtype")
    B, H, N, d = q.shape
    if N != grid[0] * grid[1] * grid[2]:
        raise ValueError("N must equal F * Hh * Ww")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    out_code = _lib.SLA_F32 if out_dtype == torch.float32 else _dtype_code(torch.empty(0, dtype=out_dtype))
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    L = _lib.load()
    n = ctypes.c_size_t()
    _lib.check(L.sla_sta_workspace_size(B, H, *grid, *tile, *window, ctypes.byref(n)))
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=q.device)
    _lib.check(L.sla_forward_sta(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), out_code, B, H, d, block,
                                 *grid, *tile, *window, out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                 _stream_ptr(q.device)))
    return out


def sta_workspace_size(B: int, H: int, grid, tile, window) -> int:
    n = ctypes.c_size_t()
    _lib.check(_lib.load().sla_sta_workspace_size(B, H, *grid, *tile, *window, ctypes.byref(n)))
    return n.value


def backward(q, k, v, w, dout, crit_frac: float = 0.05, negl_frac: float = 0.10, workspace=None, block: int = 64):
    """Gradients (dq, dk, dv [B, H, N, d] float32, dw [d, d] float32) of
    forward(q, k, v, w, crit_frac, negl_frac) for the output gradient dout,
    with the block labels held fixed.  bf16 inputs."""
    torch = _torch()
    _check_gpu(q, k, v, w, dout)
    if not (q.shape == k.shape == v.shape == dout.shape) or not (q.dtype == k.dtype == v.dtype == dout.dtype):
        raise ValueError("q, k, v, dout must have one shape and dtype")
    B, H, N, d = q.shape
    if w.dtype != torch.float32 or tuple(w.shape) != (d, d):
        raise ValueError("w must be float32 [d, d]")
    L = _lib.load()
    n = ctypes.c_size_t()
    _lib.check(L.sla_backward_workspace_size(B, H, N, d, block, crit_frac, negl_frac, ctypes.byref(n)))
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=q.device)
    dq = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    dw = torch.empty((d, d), dtype=torch.float32, device=q.device)
    _lib.check(L.sla_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), w.data_ptr(), dout.data_ptr(), _dtype_code(q),
                              B, H, N, d, block, crit_frac, negl_frac, _lib.SLA_PHI_SOFTMAX, dq.data_ptr(),
                              dk.data_ptr(), dv.data_ptr(), dw.data_ptr(), workspace.data_ptr(), workspace.numel(),
                              _stream_ptr(q.device)))
    return dq, dk, dv, dw


class SavedForward:
    """What sla_forward_save leaves for sla_backward_saved: the device buffer
    and the arguments it was made with."""

    def __init__(self, buffer, shape, crit_frac, negl_frac, block):
        self.buffer, self.shape = buffer, tuple(shape)
        self.crit_frac, self.negl_frac, self.block = crit_frac, negl_frac, block


def forward_save(q, k, v, w, crit_frac: float = 0.05, negl_frac: float = 0.10, block: int = 64, out_dtype=None,
                 return_mask: bool = False, saved=None):
    """sla_forward_save: the output of `forward` (bf16 inputs) and a
    SavedForward for backward_saved.  `saved` may be an earlier SavedForward
    of the same sizes, whose buffer is then reused."""
    torch = _torch()
    _check_gpu(q, k, v, w)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must have one shape and dtype")
    B, H, N, d = q.shape
    if w.dtype != torch.float32 or tuple(w.shape) != (d, d):
        raise ValueError("w must be float32 [d, d]")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    out_code = _lib.SLA_F32 if out_dtype == torch.float32 else _dtype_code(torch.empty(0, dtype=out_dtype))
    dev = q.device
    out = torch.empty((B, H, N, d), dtype=out_dtype, device=dev)
    Nb = -(-N // block)
    mask = torch.empty((B, H, Nb, Nb), dtype=torch.int8, device=dev) if return_mask else None
    L = _lib.load()
    n = ctypes.c_size_t()
    _lib.check(L.sla_backward_workspace_size(B, H, N, d, block, crit_frac, negl_frac, ctypes.byref(n)))
    buf = saved.buffer if saved is not None and saved.buffer.numel() >= n.value else \
        torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
    _lib.check(L.sla_forward_save(q.data_ptr(), k.data_ptr(), v.data_ptr(), w.data_ptr(), _dtype_code(q), out_code,
                                  B, H, N, d, block, crit_frac, negl_frac, _lib.SLA_PHI_SOFTMAX, out.data_ptr(),
                                  mask.data_ptr() if mask is not None else None, buf.data_ptr(), buf.numel(),
                                  _stream_ptr(dev)))
    ctx = SavedForward(buf, q.shape, crit_frac, negl_frac, block)
    return (out, mask, ctx) if return_mask else (out, ctx)


def backward_saved(saved, q, k, v, w, dout):
    """sla_backward_saved: the gradients of `backward` (dq, dk, dv, dw) from
    the state forward_save left in `saved` for these same q, k, v, w."""
    torch = _torch()
    _check_gpu(q, k, v, w, dout)
    if not (q.shape == k.shape == v.shape == dout.shape) or not (q.dtype == k.dtype == v.dtype == dout.dtype):
        raise ValueError("q, k, v, dout must have one shape and dtype")
    if tuple(q.shape) != saved.shape:
        raise ValueError("the saved forward state is for shape %s, not %s" % (saved.shape, tuple(q.shape)))
    B, H, N, d = q.shape
    if w.dtype != torch.float32 or tuple(w.shape) != (d, d):
        raise ValueError("w must be float32 [d, d]")
    dq = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    dw = torch.empty((d, d), dtype=torch.float32, device=q.device)
    _lib.check(_lib.load().sla_backward_saved(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), w.data_ptr(), dout.data_ptr(), _dtype_code(q), B, H, N, d,
        saved.block, saved.crit_frac, saved.negl_frac, _lib.SLA_PHI_SOFTMAX, dq.data_ptr(), dk.data_ptr(),
        dv.data_ptr(), dw.data_ptr(), saved.buffer.data_ptr(), saved.buffer.numel(), _stream_ptr(q.device)))
    return dq, dk, dv, dw


def backward_workspace_size(B: int, H: int, N: int, d: int, crit_frac: float = 0.05, negl_frac: float = 0.10) -> int:
    n = ctypes.c_size_t()
    _lib.check(_lib.load().sla_backward_workspace_size(B, H, N, d, 64, crit_frac, negl_frac, ctypes.byref(n)))
    return n.value


def block_mass(q, k, block: int = 64):
    """Exact block attention mass [B, H, Nb, Nb] float32 (diagnostic): row i,
    column j is the mean over the valid rows of query block i of the full
    softmax mass on key block j.  q, k: [B, H, N, d] bf16 on the GPU."""
    torch = _torch()
    _check_gpu(q, k)
    if q.shape != k.shape or q.dtype != k.dtype:
        raise ValueError("q and k must have one shape and dtype")
    B, H, N, d = q.shape
    Nb = -(-N // block)
    mass = torch.empty((B, H, Nb, Nb), dtype=torch.float32, device=q.device)
    _lib.check(_lib.load().sla_block_mass(q.data_ptr(), k.data_ptr(), _dtype_code(q), B, H, N, d, block,
                                          mass.data_ptr(), _stream_ptr(q.device)))
    return mass


def mask_stats(mass, mask):
    """Per row of blocks: [..., 4] float32 = mass on the critical, marginal and
    negligible blocks and the 95 % block density.  mass: [B, H, Nb, Nb]
    float32, mask: [B, H, Nb, Nb] int8 (from classify or forward)."""
    torch = _torch()
    _check_gpu(mass, mask)
    if mass.shape != mask.shape or mass.dtype != torch.float32 or mask.dtype != torch.int8:
        raise ValueError("mass (float32) and mask (int8) must have one shape")
    Nb = mass.shape[-1]
    rows = mass.numel() // Nb
    stats = torch.empty(tuple(mass.shape[:-1]) + (4,), dtype=torch.float32, device=mass.device)
    _lib.check(_lib.load().sla_mask_stats(mass.data_ptr(), mask.data_ptr(), rows, Nb, stats.data_ptr(),
                                          _stream_ptr(mass.device)))
    return stats


def forward_lists(q, k, v, lists, counts, out_dtype=None, out=None, block: int = 64):
    """Sparse attention over the key-block lists given per query-block row
    (linear branch off).  lists: [B, H, Nb, kmax] int32 (ascending in the
    first counts entries), counts: [B, H, Nb] int32, on q's device."""
    torch = _torch()
    _check_gpu(q, k, v, lists, counts)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must have one shape and dtype")
    B, H, N, d = q.shape
    Nb = -(-N // block)
    if lists.dtype != torch.int32 or counts.dtype != torch.int32:
        raise ValueError("lists and counts must be int32")
    if lists.dim() != 4 or tuple(lists.shape[:3]) != (B, H, Nb) or tuple(counts.shape) != (B, H, Nb):
        raise ValueError("lists must be [B, H, Nb, kmax] and counts [B, H, Nb]")
    kmax = lists.shape[3]
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    out_code = _lib.SLA_F32 if out_dtype == torch.float32 else _dtype_code(torch.empty(0, dtype=out_dtype))
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    n = ctypes.c_size_t()
    L = _lib.load()
    _lib.check(L.sla_lists_workspace_size(B, H, N, kmax, ctypes.byref(n)))
    ws = torch.empty(max(n.value, 1), dtype=torch.uint8, device=q.device)
    _lib.check(L.sla_forward_lists(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), out_code, B, H, N, d,
                                   block, lists.data_ptr(), counts.data_ptr(), kmax, out.data_ptr(), ws.data_ptr(),
                                   ws.numel(), _stream_ptr(q.device)))
    return out
