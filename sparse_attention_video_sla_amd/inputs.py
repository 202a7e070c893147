"""Seeded synthetic inputs for sparse-linear attention over 3D video tokens.

This module only *builds inputs*; it holds none of the attention method's
arithmetic, so both the CPU oracle and the GPU path can consume what it
produces without sharing any computation.

Token layout: a latent video of T x Hg x Wg positions flattened in raster order
with t slowest, token n = (t * Hg + h) * Wg + w.  The shapes of the named
workloads come from the latent grids of the pages' video models: Wan2.1 at
81 frames -> 21 latent frames, HunyuanVideo at 129 frames -> 33, with
480x832 and 720x1280 pixels at stride 16 (LVSA page, "training temporal
length" glossary entry and the reproducibility section).

Q and K are 0.5 * N(0,1) noise plus low-frequency sinusoids of (t, h, w) that
Q and K of one head share, so that q.k peaks at nearby positions and attention
is local.  V ~ N(0,1); the d x d projection W ~ N(0, 1/d).

Random streams (numpy PCG64; seed = 1000 + config id for the named workloads):
  root = PCG64(SeedSequence(seed)):
    1. frequencies  omega[h, axis, f] ~ U[0, 0.3)  (shape [H, 3, 8])
    2. W            [d, d] ~ N(0, 1/d)
  head (b, h) = PCG64(SeedSequence(seed).spawn(B*H)[b*H + h]):
    eps_Q [N,d], eps_K [N,d], V [N,d], each standard_normal(dtype=float32)
Heads are independent streams, so they are generated in parallel threads.
Q and K are formed in float64 from the float32 draws, rounded once to float32
and then (bf16 workloads) rounded to bfloat16 with round-to-nearest-even.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Optional, Sequence, Tuple

import numpy as np

N_FREQ = 8            # random frequencies per axis
FREQ_MAX = 0.3        # rad per grid step
NOISE = 0.5           # noise amplitude on Q and K
ROPE_SPLIT = (44, 42, 42)   # channels for t, h, w (d = 128)
ROPE_BASE = 10000.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtype, RoPE switch and fraction sweep."""
    cid: int
    name: str
    B: int
    H: int
    grid: Tuple[int, int, int]
    d: int
    dtype: str                       # "f32" or "bf16"
    rope: bool
    fracs: Tuple[Tuple[float, float], ...]   # (critical, negligible) settings
    block: int = 64

    @property
    def N(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def seed(self) -> int:
        return 1000 + self.cid


WORKLOADS = {
    0: Workload(0, "tiny-4x32x32-d64-f32", 1, 2, (4, 32, 32), 64, "f32", False,
                ((0.05, 0.10),)),
    1: Workload(1, "wan2.1-1.3b-480p-21x30x52", 1, 12, (21, 30, 52), 128, "bf16",
                False, ((0.05, 0.10),)),
    2: Workload(2, "wan2.1-480p-rope-cfg-pair", 2, 12, (21, 30, 52), 128, "bf16",
                True, ((0.025, 0.10), (0.05, 0.10), (0.10, 0.10))),
    3: Workload(3, "wan2.1-720p-21x45x80-rope", 1, 40, (21, 45, 80), 128, "bf16",
                True, ((0.05, 0.10),)),
    4: Workload(4, "hunyuanvideo-720p-33x45x80", 1, 24, (33, 45, 80), 128, "bf16",
                False, ((0.05, 0.10), (1.0, 0.0))),
}


@dataclasses.dataclass(frozen=True)
class LvsaWorkload:
    """A long-video workload for the LVSA frame-level sets: grid (T latent
    frames, h, w), budget C frames, half window W, denoising step."""
    name: str
    B: int
    H: int
    grid: Tuple[int, int, int]
    d: int
    C: int
    W: int
    step: int
    seed: int

    @property
    def T(self) -> int:
        return self.grid[0]

    @property
    def P(self) -> int:
        return self.grid[1] * self.grid[2]

    @property
    def N(self) -> int:
        return self.T * self.P


# Wan2.1 1.3B at 6x its training length: 481 video frames are 121 latent
# frames of 30 x 52 tokens (480 x 832); budget C = 21 latent frames (the
# training length), W = 3 so that every set holds exactly C frames.
LVSA_WORKLOADS = {
    "wan6x": LvsaWorkload("wan2.1-1.3b-480p-6x-121x30x52-lvsa", 1, 12, (121, 30, 52), 128, 21, 3, 0, 2001),
}


def make_lvsa_workload(key: str, heads: Optional[int] = None) -> Inputs:
    wl = LVSA_WORKLOADS[key]
    return make_inputs(wl.B, heads or wl.H, wl.grid, wl.d, "bf16", False, wl.seed)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32 values.
    Finite inputs below the largest bfloat16 only."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    bias = (u >> 16) & 1
    bias += 0x7FFF
    u += bias
    u &= 0xFFFF0000
    return u.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16-representable float32 values -> their uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def grid_positions(grid: Tuple[int, int, int]) -> np.ndarray:
    """[N, 3] integer (t, h, w) of each token in raster order, t slowest."""
    t, h, w = grid
    tt, hh, ww = np.meshgrid(np.arange(t), np.arange(h), np.arange(w), indexing="ij")
    return np.stack([tt.ravel(), hh.ravel(), ww.ravel()], axis=1).astype(np.float64)


def positional_features(pos: np.ndarray, omega: np.ndarray) -> np.ndarray:
    """F(n) in R^48: (cos(omega_af p_a), sin(omega_af p_a)) over axes a, freqs f."""
    ang = pos[:, :, None] * omega[None, :, :]          # [N, 3, 8]
    feats = np.concatenate([np.cos(ang), np.sin(ang)], axis=2)   # [N, 3, 16]
    return feats.reshape(pos.shape[0], -1)                      # [N, 48]


def rope_tables(pos: np.ndarray, d: int) -> Tuple[np.ndarray, np.ndarray]:
    """cos/sin per (token, channel pair) of a 3D RoPE with a 44/42/42 split.

    Pairs (2k, 2k+1) inside each axis section; theta_{a,k} = base^(-2k/d_a);
    angle = p_a * theta_{a,k}.  Only defined for d = 128.
    """
    if d != sum(ROPE_SPLIT):
        raise ValueError("3D RoPE is defined for d = 128 only")
    angles = []
    for a, da in enumerate(ROPE_SPLIT):
        k = np.arange(da // 2, dtype=np.float64)
        theta = ROPE_BASE ** (-2.0 * k / da)
        angles.append(pos[:, a:a + 1] * theta[None, :])
    ang = np.concatenate(angles, axis=1)                 # [N, 64]
    return np.cos(ang), np.sin(ang)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    x0 = x[:, 0::2]
    x1 = x[:, 1::2]
    out = np.empty_like(x)
    out[:, 0::2] = x0 * cos - x1 * sin
    out[:, 1::2] = x0 * sin + x1 * cos
    return out


@dataclasses.dataclass
class Inputs:
    q: np.ndarray      # [B,H,N,d] float32 (bf16-representable for bf16 workloads)
    k: np.ndarray
    v: np.ndarray
    w: np.ndarray      # [d,d] float32
    dtype: str
    grid: Tuple[int, int, int]


def make_inputs(B: int, H: int, grid: Tuple[int, int, int], d: int, dtype: str = "bf16",
                rope: bool = False, seed: int = 0, n_tokens: Optional[int] = None) -> Inputs:
    """Build Q, K, V [B,H,N,d] and W [d,d] for a grid, with the stream above.

    n_tokens, when given, keeps only the first n_tokens tokens of the grid
    (a ragged sequence whose last block is partial).
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    ss = np.random.SeedSequence(seed)
    rng = np.random.Generator(np.random.PCG64(ss))
    pos = grid_positions(grid)
    if n_tokens is not None:
        pos = pos[:n_tokens]
    N = pos.shape[0]
    omega = rng.uniform(0.0, FREQ_MAX, size=(H, 3, N_FREQ))
    w = (rng.standard_normal((d, d)) / np.sqrt(d)).astype(np.float32)
    children = ss.spawn(B * H)
    cos = sin = None
    if rope:
        cos, sin = rope_tables(pos, d)
    q = np.empty((B, H, N, d), np.float32)
    k = np.empty((B, H, N, d), np.float32)
    v = np.empty((B, H, N, d), np.float32)
    chan = np.arange(d) % (2 * 3 * N_FREQ)

    def one_head(bh: int) -> None:
        b, h = divmod(bh, H)
        g = np.random.Generator(np.random.PCG64(children[bh]))
        feats = positional_features(pos, omega[h])[:, chan]     # [N, d]
        eq = g.standard_normal((N, d), dtype=np.float32)
        ek = g.standard_normal((N, d), dtype=np.float32)
        vv = g.standard_normal((N, d), dtype=np.float32)
        qh = NOISE * eq.astype(np.float64) + feats
        kh = NOISE * ek.astype(np.float64) + feats
        if rope:
            qh = apply_rope(qh, cos, sin)
            kh = apply_rope(kh, cos, sin)
        q[b, h] = qh
        k[b, h] = kh
        v[b, h] = vv
        if dtype == "bf16":
            q[b, h] = round_bf16(q[b, h])
            k[b, h] = round_bf16(k[b, h])
            v[b, h] = round_bf16(v[b, h])

    workers = max(1, min(16, os.cpu_count() or 1, B * H))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(one_head, range(B * H)))
    return Inputs(q, k, v, w, dtype, grid)


def make_workload(cid: int, n_tokens: Optional[int] = None) -> Inputs:
    wl = WORKLOADS[cid]
    return make_inputs(wl.B, wl.H, wl.grid, wl.d, wl.dtype, wl.rope, wl.seed, n_tokens)


def sample_query_blocks(B: int, H: int, Nb: int, per_head: int, seed: int,
                        include: Sequence[int] = ()) -> np.ndarray:
    """Seeded sample of (b*H + h, i) query-block pairs, sorted; `include` adds
    fixed block indices (e.g. the first and the ragged last) for every head."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = []
    for bh in range(B * H):
        pick = set(int(x) for x in rng.choice(Nb, size=min(per_head, Nb), replace=False))
        pick.update(int(i) % Nb for i in include)
        rows.extend((bh, i) for i in sorted(pick))
    return np.asarray(rows, dtype=np.int32).reshape(-1, 2)
