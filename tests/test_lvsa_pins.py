"""Pins of the LVSA oracle (oracle/lvsa.py): the frame sets against what the
LVSA page fixes (the size of G_s, the exact per-frame budget, the rotation,
the window bounds), a set worked by hand from the method steps, and the
attention against SDPA and a pure-Python brute force."""
import math

import numpy as np
import pytest

from oracle import lvsa

torch = pytest.importorskip("torch")

GRID = [(T, C, W) for T in (1, 2, 5, 9, 10, 17, 22, 41, 64, 121) for C in (4, 7, 21, 33) for W in (0, 1, 3)
        if C - (2 * W + 1) >= 1]


def test_global_count_is_ceil_T_over_Tper():
    """The page: taking the positions modulo T keeps |G_s| = ceil(T / T_per) at every step."""
    for T, C, W in GRID:
        Tp = lvsa.period(T, C, W)
        for s in range(2 * Tp + 1):
            G = lvsa.globals_at(T, Tp, s)
            assert len(G) == -(-T // Tp), (T, C, W, s)
            assert all(0 <= g < T for g in G)


def test_every_frame_attends_exact_budget():
    """The page: with the expanded window every frame attends exactly
    |G| + min(2W + 1, T - |G|) distinct frames."""
    for T, C, W in GRID:
        Tp = lvsa.period(T, C, W)
        m = -(-T // Tp)
        for s in range(Tp):
            for t, a in enumerate(lvsa.all_sets(T, C, W, s)):
                assert len(a) == len(set(a)) == m + min(2 * W + 1, T - m), (T, C, W, s, t)


def test_budget_within_C_plus_minus_delta_on_long_videos():
    """The page: every frame's budget lies in [C - delta, C + delta] with
    delta <= T_per - 1.  Holds on the page's long-video setting (C = 21
    latent frames, 3x to 6x the training length); near T = C it does not
    (there G_s alone takes half the frames), so the pin stays on that range."""
    C = 21
    for T in (61, 81, 101, 121):
        for W in range(1, 7):
            Tp = lvsa.period(T, C, W)
            for t, a in enumerate(lvsa.all_sets(T, C, W, 0)):
                assert abs(len(a) - C) <= Tp - 1, (T, W, t, len(a), Tp)


def test_rotation_covers_every_frame_and_shifts_by_one():
    """Within any T_per consecutive steps every frame is a global at least
    once; between steps s and s + 1 of one period the set moves by one frame
    (wrapping at T)."""
    for T, C, W in GRID:
        Tp = lvsa.period(T, C, W)
        for s0 in range(Tp):
            seen = set()
            for s in range(s0, s0 + Tp):
                seen |= set(lvsa.globals_at(T, Tp, s))
            assert seen == set(range(T)), (T, C, W, s0)
        for s in range(Tp - 1):
            a, b = lvsa.globals_at(T, Tp, s), lvsa.globals_at(T, Tp, s + 1)
            assert sorted((g + 1) % T for g in a) == b


def test_windows_hold_their_frame_and_stay_in_range():
    for T, C, W in GRID:
        Tp = lvsa.period(T, C, W)
        G = lvsa.globals_at(T, Tp, 1)
        for t in range(T):
            lo, hi = lvsa.basic_window(t, T, W)
            assert 0 <= lo <= t <= hi <= T - 1 and hi - lo + 1 == min(2 * W + 1, T)
            lo2, hi2 = lvsa.expanded_window(t, T, W, G)
            assert 0 <= lo2 <= lo and hi <= hi2 <= T - 1
            if not set(G) & set(range(lo, hi + 1)):
                assert (lo2, hi2) == (lo, hi)     # nothing to compensate: no expansion


def test_hand_worked_sets():
    """T = 10, C = 7, W = 1: T_per = ceil(10 / (7 - 3)) = 3, |G| = 4.
    Step 0: G = {0, 3, 6, 9}.  Step 1: {1, 4, 7, 10 mod 10} = {0, 1, 4, 7}.
    Frame 5 at step 0: w_lo = max(0, min(4, 7)) = 4, window [4, 6] holds the
    non-globals 4, 5 (6 is global), 2 < min(3, 10 - 4) = 3: grow.  Room
    left 4 > right 3: take 3 (global, still 2).  Room 3 and 3, a tie: take
    the earlier side, 2 (non-global, 3 reached).  A(5) = {0, 2, 3, 4, 5, 6, 9}.
    Frame 0 at step 0: window [0, 2] holds 1, 2; grow right (no room left):
    3 is global, then 4: A(0) = {0, 1, 2, 3, 4, 6, 9}.
    Frame 9 at step 1: w_lo = min(8, 7) = 7, window [7, 9] holds 8, 9; room
    left 7, right 0: take 6.  A(9) = {0, 1, 4, 6, 7, 8, 9}."""
    assert lvsa.period(10, 7, 1) == 3
    assert lvsa.globals_at(10, 3, 0) == [0, 3, 6, 9]
    assert lvsa.globals_at(10, 3, 1) == [0, 1, 4, 7]
    assert lvsa.attention_set(5, 10, 7, 1, 0) == [0, 2, 3, 4, 5, 6, 9]
    assert lvsa.attention_set(0, 10, 7, 1, 0) == [0, 1, 2, 3, 4, 6, 9]
    assert lvsa.attention_set(9, 10, 7, 1, 1) == [0, 1, 4, 6, 7, 8, 9]


def test_degenerate_sets_are_all_frames():
    """T_per = 1 makes every frame global; a window wider than the video covers it."""
    assert lvsa.period(5, 21, 1) == 1
    assert all(a == list(range(5)) for a in lvsa.all_sets(5, 21, 1, 3))
    assert lvsa.basic_window(2, 4, 3) == (0, 3)


def rand(B, H, N, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, N, d)).astype(np.float32) for _ in range(3)]


def sdpa(q, k, v, mask=None):
    t = lambda x: torch.from_numpy(np.asarray(x, np.float64))
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask).numpy()


def test_all_frames_is_dense_attention():
    T, P = 5, 37
    q, k, v = rand(1, 2, T * P, 16, 1)
    got = lvsa.attention_lvsa(q, k, v, T, P, 21, 1, 0)
    assert np.allclose(got, sdpa(q, k, v), atol=1e-12)


def test_frame_mask_attention_matches_sdpa():
    """T = 10, C = 7, W = 1, frames of 30 tokens: the token mask built from the
    frame sets, through SDPA."""
    T, P, C, W, s = 10, 30, 7, 1, 1
    q, k, v = rand(1, 1, T * P, 8, 2)
    sets = lvsa.all_sets(T, C, W, s)
    frame = np.arange(T * P) // P
    allow = np.zeros((T, T), bool)
    for t, a in enumerate(sets):
        allow[t, a] = True
    mask = torch.from_numpy(allow[frame][:, frame])
    assert np.allclose(lvsa.attention_lvsa(q, k, v, T, P, C, W, s), sdpa(q, k, v, mask), atol=1e-12)


def test_brute_force_tiny():
    T, P, C, W, s, d = 6, 3, 5, 1, 2, 4
    q, k, v = rand(1, 1, T * P, d, 3)
    got = lvsa.attention_lvsa(q, k, v, T, P, C, W, s)[0, 0]
    for n in range(T * P):
        keys = [u for u in range(T * P) if u // P in lvsa.attention_set(n // P, T, C, W, s)]
        sc = [math.fsum(float(q[0, 0, n, c]) * float(k[0, 0, u, c]) for c in range(d)) / math.sqrt(d) for u in keys]
        mx = max(sc)
        e = [math.exp(x - mx) for x in sc]
        z = math.fsum(e)
        for c in range(d):
            assert abs(got[n, c] - math.fsum(e[x] * float(v[0, 0, u, c]) for x, u in enumerate(keys)) / z) < 1e-12


def test_sampled_blocks_match_full():
    T, P = 10, 50
    q, k, v = rand(1, 2, T * P, 8, 4)
    full = lvsa.attention_lvsa(q, k, v, T, P, 7, 1, 0)
    got = lvsa.attention_lvsa(q, k, v, T, P, 7, 1, 0, rows=[(1, 7), (0, 0)])
    assert np.array_equal(got[0, :500 - 448], full[0, 1, 448:500]) and np.array_equal(got[1], full[0, 0, 0:64])
