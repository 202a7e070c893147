"""LVSA frame-level attention sets and the attention they define, in fp64.

TEST INFRASTRUCTURE ONLY: imported by tests/ and by the CPU baseline of the
measurements, never by the product path.  Shares nothing with the GPU library.

Source: the LVSA page (training-free sparse attention for long-video
diffusion), sections "Core method", "Method steps in detail" and "Technical
novelty".  Notation as there: T frames, budget C frames, half window W,
global period T_per, denoising step s, attention set A(t) = G_s u W(t) of
query frame t.

Readings where the page leaves a step open (each also listed in the design doc):
  * G_s takes i = 0 .. ceil(T / T_per) - 1, the size the page states.
  * The basic window is [w_lo, w_lo + 2W] clipped to the last frame, with
    the page's adaptive lower bound w_lo = max(0, min(t - W, T - 1 - 2W)).
  * Expansion: while the window holds fewer non-global frames than
    min(2W + 1, T - |G_s|), it grows by one frame on the side with more
    frames left outside it (the earlier side on a tie).  One frame per
    iteration.
  * Frames are contiguous runs of P tokens (token n is in frame n // P);
    a query token of frame t attends every token of every frame in A(t),
    one softmax with scale 1/sqrt(d) (the page's normalised sum over
    tau in A(t) and the tokens p of frame tau).
"""
from __future__ import annotations

import math

import numpy as np


def period(T: int, C: int, W: int) -> int:
    """T_per = ceil(T / (C - (2W + 1))), the global period ("Method steps", step 1)."""
    if C - (2 * W + 1) < 1:
        raise ValueError("the budget C must exceed the window 2W + 1")
    return -(-T // (C - (2 * W + 1)))


def globals_at(T: int, T_per: int, s: int) -> list:
    """G_s = {(s mod T_per + i * T_per) mod T}, i = 0 .. ceil(T/T_per) - 1
    ("Core method", rotating periodic globals)."""
    m = -(-T // T_per)
    return sorted({(s % T_per + i * T_per) % T for i in range(m)})


def basic_window(t: int, T: int, W: int) -> tuple:
    """[w_lo, w_hi] with the adaptive lower bound of "Method steps", step 2."""
    lo = max(0, min(t - W, T - 1 - 2 * W))
    return lo, min(T - 1, lo + 2 * W)


def expanded_window(t: int, T: int, W: int, G) -> tuple:
    """Grow the basic window until it holds min(2W + 1, T - |G|) frames that
    are not global ("Method steps", step 3)."""
    gs = set(G)
    lo, hi = basic_window(t, T, W)
    target = min(2 * W + 1, T - len(gs))
    have = sum(1 for f in range(lo, hi + 1) if f not in gs)
    while have < target:
        left, right = lo, T - 1 - hi
        if left >= right and left > 0:
            lo -= 1
            have += lo not in gs
        else:
            hi += 1
            have += hi not in gs
    return lo, hi


def attention_set(t: int, T: int, C: int, W: int, s: int) -> list:
    """A(t) = G_s u W(t), ascending ("Method steps", step 5)."""
    G = globals_at(T, period(T, C, W), s)
    lo, hi = expanded_window(t, T, W, G)
    return sorted(set(G) | set(range(lo, hi + 1)))


def all_sets(T: int, C: int, W: int, s: int) -> list:
    return [attention_set(t, T, C, W, s) for t in range(T)]


def attention_lvsa(q, k, v, T: int, P: int, C: int, W: int, s: int, rows=None, blk: int = 64) -> np.ndarray:
    """q, k, v: [B, H, N, d] with N = T * P.  Every query token of frame t
    attends the tokens of the frames in A(t) ("Method steps", step 6).
    Returns out [B, H, N, d] fp64, or with rows = [(bh, i), ...] an array
    [len(rows), blk, d] holding those 64-token query blocks (pad rows zero)."""
    B, H, N, d = q.shape
    if N != T * P:
        raise ValueError("N must equal T * P")
    sets = all_sets(T, C, W, s)
    qf = np.asarray(q, np.float64).reshape(B * H, N, d)
    kf = np.asarray(k, np.float64).reshape(B * H, N, d)
    vf = np.asarray(v, np.float64).reshape(B * H, N, d)
    scale = 1.0 / math.sqrt(d)

    def rows_out(bh, r0, r1):
        res = np.zeros((r1 - r0, d))
        for t in range(r0 // P, (r1 - 1) // P + 1):
            a, b = max(r0, t * P), min(r1, (t + 1) * P)
            keys = np.concatenate([np.arange(f * P, (f + 1) * P) for f in sets[t]])
            sc = qf[bh, a:b] @ kf[bh, keys].T * scale
            sc -= sc.max(axis=1, keepdims=True)
            p = np.exp(sc)
            p /= p.sum(axis=1, keepdims=True)
            res[a - r0:b - r0] = p @ vf[bh, keys]
        return res

    if rows is not None:
        out = np.zeros((len(rows), blk, d))
        for x, (bh, i) in enumerate(rows):
            r0, r1 = blk * i, min(N, blk * (i + 1))
            out[x, :r1 - r0] = rows_out(bh, r0, r1)
        return out
    out = np.zeros((B * H, N, d))
    for bh in range(B * H):
        out[bh] = rows_out(bh, 0, N)
    return out.reshape(B, H, N, d)


def keys_per_token(T: int, P: int, C: int, W: int, s: int) -> int:
    """Total number of (query token, key token) pairs LVSA scores: sum over
    frames t of P * P * |A(t)|."""
    return sum(P * P * len(a) for a in all_sets(T, C, W, s))
