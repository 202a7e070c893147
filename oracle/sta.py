"""Sliding tile attention (STA) mask and the attention it defines, in fp64.

TEST INFRASTRUCTURE ONLY: imported by tests/ and by the CPU baseline of the
measurements, never by the product path.  Shares nothing with the GPU library.

Source: the VORTA page (sparse attention variants for video diffusion
transformers), "Key designs", item 1 (sliding window attention for local
heads): per axis, the mask keeps key j of query i when j lies in
(tau(i) - w, tau(i) + w], tau(i) = floor(i / t) * t + ceil(t / 2) being the
centre of i's tile, with window (18, 27, 24) for (frames, height, width).

Readings where the page leaves a step open (each also listed in the design doc):
  * the test is applied per axis to the key's tile centre tau(j) (so whole
    key tiles are in or out: the page's point is a block-dense mask), with
    w = W / 2 for the window W of that axis;
  * a key is kept when all three axes keep it; no shift of the window at
    the borders (tiles past the grid do not exist);
  * tokens are in raster order (frames slowest) for this oracle; the GPU
    path takes them tile-major (tile_order below), the layout STA computes
    in, and the tests permute between the two.
"""
from __future__ import annotations

import math

import numpy as np


def centre(i, t: int):
    """tau(i) = floor(i / t) * t + ceil(t / 2) (numpy arrays or ints)."""
    return (np.asarray(i) // t) * t + (t + 1) // 2


def axis_keep(i, j, t: int, W: int) -> np.ndarray:
    """Per axis: key j kept for query i when tau(j) lies in (tau(i) - W/2, tau(i) + W/2]."""
    d = centre(j, t) - centre(i, t)
    return (2 * d > -W) & (2 * d <= W)


def coords(grid) -> np.ndarray:
    """[N, 3] (f, h, w) of each token in raster order."""
    F, Hh, Ww = grid
    f, h, w = np.meshgrid(np.arange(F), np.arange(Hh), np.arange(Ww), indexing="ij")
    return np.stack([f.ravel(), h.ravel(), w.ravel()], axis=1)


def mask(grid, tile, window) -> np.ndarray:
    """[N, N] bool, raster order: mask[n, u] = key u kept for query n."""
    c = coords(grid)
    keep = np.ones((len(c), len(c)), bool)
    for a in range(3):
        keep &= axis_keep(c[:, a][:, None], c[:, a][None, :], tile[a], window[a])
    return keep


def tile_order(grid, tile) -> np.ndarray:
    """perm[m] = raster index of the m-th token in tile-major order: tiles in
    raster order over the tile grid, tokens in raster order inside a tile."""
    F, Hh, Ww = grid
    tf, th, tw = tile
    c = coords(grid)
    tid = ((c[:, 0] // tf) * (Hh // th) + c[:, 1] // th) * (Ww // tw) + c[:, 2] // tw
    inner = ((c[:, 0] % tf) * th + c[:, 1] % th) * tw + c[:, 2] % tw
    return np.lexsort((inner, tid))


def attention_sta(q, k, v, grid, tile, window, rows=None) -> np.ndarray:
    """q, k, v: [B, H, N, d] in raster order.  Every query attends the keys
    the mask keeps, one softmax, scale 1/sqrt(d).  Returns out [B, H, N, d]
    fp64, or with rows = [(bh, n), ...] an array [len(rows), d]."""
    B, H, N, d = q.shape
    c = coords(grid)
    qf = np.asarray(q, np.float64).reshape(B * H, N, d)
    kf = np.asarray(k, np.float64).reshape(B * H, N, d)
    vf = np.asarray(v, np.float64).reshape(B * H, N, d)
    scale = 1.0 / math.sqrt(d)

    def keys_of(n):
        keep = np.ones(N, bool)
        for a in range(3):
            keep &= axis_keep(c[n, a], c[:, a], tile[a], window[a])
        return np.nonzero(keep)[0]

    def one(bh, n, keys):
        s = kf[bh, keys] @ qf[bh, n] * scale
        s -= s.max()
        p = np.exp(s)
        return (p / p.sum()) @ vf[bh, keys]

    if rows is not None:
        return np.stack([one(bh, n, keys_of(n)) for bh, n in rows]) if len(rows) else np.zeros((0, d))
    out = np.zeros((B * H, N, d))
    for n in range(N):
        keys = keys_of(n)
        s = qf[:, n:n + 1] @ kf[:, keys].transpose(0, 2, 1) * scale
        s -= s.max(axis=2, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=2, keepdims=True)
        out[:, n] = (p @ vf[:, keys])[:, 0]
    return out.reshape(B, H, N, d)


def kept_pairs(grid, tile, window) -> int:
    """Number of (query, key) pairs the mask keeps (per head)."""
    total = 1
    for a in range(3):
        n = grid[a]
        i = np.arange(n)
        total *= int(axis_keep(i[:, None], i[None, :], tile[a], window[a]).sum())
    return total
