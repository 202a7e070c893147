"""The seeded workload generator: shapes, determinism, dtype, RoPE, locality."""
import numpy as np
import pytest

from sparse_attention_video_sla_amd.inputs import (WORKLOADS, apply_rope, grid_positions, make_inputs,
                                                   rope_tables, round_bf16, sample_query_blocks)


def test_workload_table():
    assert [WORKLOADS[i].N for i in range(5)] == [4096, 32760, 32760, 75600, 118800]
    assert [-(-WORKLOADS[i].N // 64) for i in range(5)] == [64, 512, 512, 1182, 1857]
    assert WORKLOADS[0].dtype == "f32" and all(WORKLOADS[i].dtype == "bf16" for i in range(1, 5))


def test_deterministic_and_bf16():
    a = make_inputs(2, 3, (2, 4, 8), 16, "bf16", seed=3)
    b = make_inputs(2, 3, (2, 4, 8), 16, "bf16", seed=3)
    for x in "qkvw":
        assert np.array_equal(getattr(a, x), getattr(b, x))
    assert np.array_equal(round_bf16(a.q), a.q) and np.array_equal(round_bf16(a.v), a.v)
    c = make_inputs(2, 3, (2, 4, 8), 16, "bf16", seed=4)
    assert not np.array_equal(a.q, c.q)


def test_raster_order():
    pos = grid_positions((2, 3, 4))
    assert pos.shape == (24, 3)
    assert tuple(pos[0]) == (0, 0, 0) and tuple(pos[1]) == (0, 0, 1) and tuple(pos[4]) == (0, 1, 0)
    assert tuple(pos[12]) == (1, 0, 0)


def test_rope_preserves_norms_and_is_relative():
    pos = grid_positions((3, 4, 5))
    cos, sin = rope_tables(pos, 128)
    x = np.random.default_rng(0).standard_normal((60, 128))
    y = apply_rope(x, cos, sin)
    assert np.allclose(np.linalg.norm(x, axis=1), np.linalg.norm(y, axis=1), rtol=1e-12)
    # the same vector at two positions: the dot product depends on the offset only
    v = np.tile(x[:1], (60, 1))
    r = apply_rope(v, cos, sin)
    assert np.isclose(r[0] @ r[21], r[5] @ r[26])   # both offsets (1, 1, 1)


def test_attention_is_local():
    """Q and K share low-frequency sinusoids: q.k is largest at zero offset and
    falls off with the grid distance."""
    inp = make_inputs(1, 1, (8, 16, 16), 128, "f32", seed=9)
    q, k = inp.q[0, 0].astype(np.float64), inp.k[0, 0].astype(np.float64)
    pos = grid_positions((8, 16, 16))
    idx = np.random.default_rng(0).choice(len(pos), 400, replace=False)
    dist = np.abs(pos[idx][:, None, :] - pos[None, :, :]).sum(-1)
    s = q[idx] @ k.T
    near = s[dist == 0].mean()
    mid = s[(dist >= 4) & (dist < 8)].mean()
    far = s[dist >= 20].mean()
    assert near > mid + 5 and mid > far + 20


def test_ragged_prefix():
    full = make_inputs(1, 2, (2, 8, 8), 16, "bf16", seed=1)
    part = make_inputs(1, 2, (2, 8, 8), 16, "bf16", seed=1, n_tokens=100)
    assert part.q.shape == (1, 2, 100, 16)
    assert np.array_equal(part.w, full.w)


def test_sample_query_blocks():
    rows = sample_query_blocks(1, 3, 50, 4, seed=1, include=(0, -1))
    assert rows.shape[1] == 2
    assert list(rows[:, 0]) == sorted(rows[:, 0])
    for bh in range(3):
        got = set(rows[rows[:, 0] == bh, 1])
        assert {0, 49} <= got and len(got) >= 4
