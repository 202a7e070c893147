"""Pins of the list-attention oracle (oracle/lists.py) against torch's
scaled_dot_product_attention (dense and with a block mask), closed forms and
a pure-Python brute force."""
import math

import numpy as np
import pytest

from oracle import lists as ol

torch = pytest.importorskip("torch")


def sdpa(q, k, v, mask=None):
    t = lambda x: torch.from_numpy(np.asarray(x, np.float64))
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask).numpy()


def rand(B, H, N, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, N, d)).astype(np.float32) for _ in range(3)]


def test_all_blocks_is_dense_attention():
    q, k, v = rand(1, 2, 300, 16, 1)
    Nb = 5
    lists = np.tile(np.arange(Nb, dtype=np.int32), (1, 2, Nb, 1))
    counts = np.full((1, 2, Nb), Nb, np.int32)
    got = ol.attention_lists(q, k, v, lists, counts)
    assert np.allclose(got, sdpa(q, k, v), atol=1e-12)


def test_diagonal_blocks_is_block_diagonal_attention():
    q, k, v = rand(1, 1, 200, 8, 2)
    Nb, N = 4, 200
    lists = np.arange(Nb, dtype=np.int32).reshape(1, 1, Nb, 1)
    counts = np.ones((1, 1, Nb), np.int32)
    blk = np.arange(N) // 64
    mask = torch.from_numpy(blk[:, None] == blk[None, :])
    assert np.allclose(ol.attention_lists(q, k, v, lists, counts), sdpa(q, k, v, mask), atol=1e-12)


def test_empty_row_duplicates_and_out_of_range():
    """count 0 gives zeros; a repeated block, entries past the count and
    indices outside [0, Nb) change nothing."""
    q, k, v = rand(1, 1, 256, 8, 3)
    lists = np.array([[[[1, 3, 0], [2, 2, 7], [-1, 0, 9], [3, 1, 2]]]], np.int32)
    counts = np.array([[[0, 3, 2, 2]]], np.int32)
    got = ol.attention_lists(q, k, v, lists, counts)
    assert np.all(got[0, 0, 0:64] == 0)
    ref2 = ol.attention_lists(q, k, v, np.array([[[[0], [2], [0], [1]]]], np.int32), np.array([[[0, 1, 1, 0]]], np.int32))
    assert np.allclose(got[0, 0, 64:192], ref2[0, 0, 64:192], atol=1e-14)
    ref3 = ol.attention_lists(q, k, v, np.array([[[[0, 0], [0, 0], [0, 0], [1, 3]]]], np.int32), np.array([[[0, 0, 0, 2]]], np.int32))
    assert np.allclose(got[0, 0, 192:256], ref3[0, 0, 192:256], atol=1e-14)


def test_brute_force_tiny_ragged():
    rng = np.random.default_rng(4)
    N, d, blk = 45, 4, 16
    q, k, v = [rng.standard_normal((1, 1, N, d)).astype(np.float32) for _ in range(3)]
    lists = np.array([[[[0, 2], [1, 0], [2, 1]]]], np.int32)
    counts = np.array([[[2, 1, 2]]], np.int32)
    got = ol.attention_lists(q, k, v, lists, counts, blk)[0, 0]
    for r in range(N):
        i = r // blk
        keys = [u for j in sorted(set(lists[0, 0, i, :counts[0, 0, i]])) for u in range(blk * j, min(N, blk * (j + 1)))]
        s = [math.fsum(float(q[0, 0, r, c]) * float(k[0, 0, u, c]) for c in range(d)) / math.sqrt(d) for u in keys]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        z = math.fsum(e)
        for c in range(d):
            ref = math.fsum(e[t] * float(v[0, 0, u, c]) for t, u in enumerate(keys)) / z
            assert abs(got[r, c] - ref) < 1e-12


def test_sampled_rows_match_full():
    q, k, v = rand(1, 2, 200, 8, 5)
    rng = np.random.default_rng(6)
    lists = rng.integers(0, 4, size=(1, 2, 4, 3)).astype(np.int32)
    counts = rng.integers(0, 4, size=(1, 2, 4)).astype(np.int32)
    full = ol.attention_lists(q, k, v, lists, counts)
    got = ol.attention_lists(q, k, v, lists, counts, rows=[(1, 3), (0, 0)])
    assert np.array_equal(got[0, :8], full[0, 1, 192:200]) and np.array_equal(got[1], full[0, 0, 0:64])
