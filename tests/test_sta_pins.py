"""Pins of the STA oracle (oracle/sta.py): the mask against hand-worked
one-axis cases, its block-dense structure and separability, the degenerate
windows (everything: dense SDPA; one tile: block-diagonal SDPA over tiles),
the tile-major order, and the attention against a pure-Python brute force."""
import math

import numpy as np
import pytest

from oracle import sta

torch = pytest.importorskip("torch")


def test_one_axis_hand_cases():
    """Tiles of 4 on one axis of 12 positions: centres 2, 6, 10.  Window 12
    (w = 6): a key tile is kept when its centre is within (-6, 6] of the
    query tile's, i.e. the tile and its two neighbours.  Window 8 (w = 4):
    (-4, 4] keeps the tile and the next one only (the interval is open on
    the left).  Window 4: the tile itself."""
    i = np.arange(12)
    tile_of = i // 4
    def keep(W):
        return sta.axis_keep(i[:, None], i[None, :], 4, W)
    k12 = keep(12)
    for a in range(12):
        assert set(tile_of[k12[a]]) == {x for x in (tile_of[a] - 1, tile_of[a], tile_of[a] + 1) if 0 <= x < 3}
    k8 = keep(8)
    for a in range(12):
        assert set(tile_of[k8[a]]) == {x for x in (tile_of[a], tile_of[a] + 1) if x < 3}
    assert np.array_equal(keep(4), tile_of[:, None] == tile_of[None, :])
    assert list(sta.centre(np.array([0, 3, 4, 11]), 4)) == [2, 2, 6, 10]
    assert list(sta.centre(np.array([0, 2, 3, 5]), 3)) == [2, 2, 5, 5]


def test_page_window_keeps_three_tiles_per_axis():
    """Window (18, 27, 24) on tiles (6, 8, 8): the query tile and its
    neighbours on every axis (27 key tiles inside the grid)."""
    for t, W in ((6, 18), (8, 27), (8, 24)):
        i = np.arange(5 * t)
        kp = sta.axis_keep(i[:, None], i[None, :], t, W)
        for a in range(5 * t):
            assert set(i[kp[a]] // t) == {x for x in (a // t - 1, a // t, a // t + 1) if 0 <= x < 5}


def test_mask_is_block_dense_and_separable():
    grid, tile, window = (4, 6, 8), (2, 3, 4), (4, 9, 8)
    m = sta.mask(grid, tile, window)
    c = sta.coords(grid)
    tid = ((c[:, 0] // 2) * 2 + c[:, 1] // 3) * 2 + c[:, 2] // 4
    for x in range(len(c)):
        for y in range(len(c)):
            if tid[x] == tid[y]:
                assert np.array_equal(m[x], m[y]) and np.array_equal(m[:, x], m[:, y])
                break
    assert m.sum() == sta.kept_pairs(grid, tile, window)


def test_tile_order_is_a_tile_major_permutation():
    grid, tile = (4, 6, 8), (2, 3, 4)
    p = sta.tile_order(grid, tile)
    assert sorted(p) == list(range(4 * 6 * 8))
    c = sta.coords(grid)[p]
    vol = 2 * 3 * 4
    for g in range(len(p) // vol):
        blk = c[g * vol:(g + 1) * vol]
        assert len({(f // 2, h // 3, w // 4) for f, h, w in blk}) == 1
        inner = [((f % 2) * 3 + h % 3) * 4 + w % 4 for f, h, w in blk]
        assert inner == list(range(vol))


def rand(B, H, N, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, N, d)).astype(np.float32) for _ in range(3)]


def sdpa(q, k, v, mask=None):
    t = lambda x: torch.from_numpy(np.asarray(x, np.float64))
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask).numpy()


def test_window_over_everything_is_dense():
    grid = (3, 4, 4)
    q, k, v = rand(1, 2, 48, 8, 1)
    got = sta.attention_sta(q, k, v, grid, (1, 2, 2), (8, 8, 8))
    assert np.allclose(got, sdpa(q, k, v), atol=1e-12)


def test_window_of_one_tile_is_block_diagonal():
    grid, tile = (4, 4, 6), (2, 2, 3)
    q, k, v = rand(1, 1, 96, 8, 2)
    c = sta.coords(grid)
    tid = (c[:, 0] // 2) * 100 + (c[:, 1] // 2) * 10 + c[:, 2] // 3
    m = torch.from_numpy(tid[:, None] == tid[None, :])
    assert np.allclose(sta.attention_sta(q, k, v, grid, tile, tile), sdpa(q, k, v, m), atol=1e-12)


def test_brute_force_tiny():
    grid, tile, window = (2, 3, 4), (1, 3, 2), (2, 3, 4)
    N, d = 24, 4
    q, k, v = rand(1, 1, N, d, 3)
    got = sta.attention_sta(q, k, v, grid, tile, window)[0, 0]
    pos = [(f, h, w) for f in range(2) for h in range(3) for w in range(4)]
    def kept(a, b):
        for ax in range(3):
            t, W = tile[ax], window[ax]
            ca = (a[ax] // t) * t + (t + 1) // 2
            cb = (b[ax] // t) * t + (t + 1) // 2
            if not (ca - W / 2 < cb <= ca + W / 2):
                return False
        return True
    for n in range(N):
        keys = [u for u in range(N) if kept(pos[n], pos[u])]
        s = [math.fsum(float(q[0, 0, n, c]) * float(k[0, 0, u, c]) for c in range(d)) / math.sqrt(d) for u in keys]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        z = math.fsum(e)
        for c in range(d):
            assert abs(got[n, c] - math.fsum(e[x] * float(v[0, 0, u, c]) for x, u in enumerate(keys)) / z) < 1e-12


def test_sampled_rows_match_full():
    grid, tile, window = (2, 4, 8), (1, 2, 4), (2, 4, 8)
    q, k, v = rand(1, 2, 64, 8, 4)
    full = sta.attention_sta(q, k, v, grid, tile, window)
    got = sta.attention_sta(q, k, v, grid, tile, window, rows=[(1, 5), (0, 63)])
    assert np.array_equal(got[0], full[0, 1, 5]) and np.array_equal(got[1], full[0, 0, 63])
