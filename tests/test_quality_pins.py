"""Pins of the mask-quality oracle (oracle/quality.py) against what does not
depend on its own formula: closed forms, an invariant, a planted case and a
pure-Python brute force."""
import math

import numpy as np

from oracle import quality


def brute_block_mass(q, k, blk):
    """[N, d] one head; loops, math.exp and math.fsum."""
    N, d = q.shape
    Nb = -(-N // blk)
    out = []
    for i in range(Nb):
        rows = range(blk * i, min(N, blk * (i + 1)))
        acc = [[] for _ in range(Nb)]
        for r in rows:
            s = [math.fsum(float(q[r, c]) * float(k[u, c]) for c in range(d)) / math.sqrt(d) for u in range(N)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            z = math.fsum(e)
            for j in range(Nb):
                acc[j].append(math.fsum(e[blk * j:min(N, blk * (j + 1))]) / z)
        out.append([math.fsum(a) / len(rows) for a in acc])
    return np.array(out)


def test_rows_sum_to_one():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 2, 300, 16)).astype(np.float32)
    k = rng.standard_normal((1, 2, 300, 16)).astype(np.float32)
    m = quality.block_mass(q, k, 64)
    assert m.shape == (1, 2, 5, 5)
    assert np.allclose(m.sum(axis=-1), 1.0, atol=1e-12)
    assert (m >= 0).all()


def test_zero_queries_give_block_sizes_over_n():
    """q = 0: every key gets 1/N, so block j gets n_j / N (ragged last block)."""
    rng = np.random.default_rng(2)
    N = 200
    q = np.zeros((1, 1, N, 8), np.float32)
    k = rng.standard_normal((1, 1, N, 8)).astype(np.float32)
    m = quality.block_mass(q, k, 64)[0, 0]
    expect = np.array([64, 64, 64, 8]) / N
    assert np.allclose(m, expect[None, :], atol=1e-14)


def test_planted_block_takes_the_mass():
    """Every query equals u and block 2's keys equal u with |u|^2/sqrt(d) = 64,
    the other keys are small: block 2 holds all but < N e^-50 of each row."""
    rng = np.random.default_rng(3)
    N, d = 320, 16
    u = np.full(d, 4.0, np.float32)                      # |u|^2 / sqrt(d) = 256 / 4 = 64
    q = np.tile(u, (1, 1, N, 1))
    k = (0.01 * rng.standard_normal((1, 1, N, d))).astype(np.float32)
    k[0, 0, 128:192] = u
    m = quality.block_mass(q, k, 64)[0, 0]
    assert (1.0 - m[:, 2] <= N * math.exp(-50.0) + 1e-15).all()


def test_brute_force_tiny():
    rng = np.random.default_rng(4)
    for N, d, blk in ((37, 4, 8), (50, 6, 16)):
        q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
        k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
        got = quality.block_mass(q, k, blk)[0, 0]
        ref = brute_block_mass(q[0, 0], k[0, 0], blk)
        assert np.allclose(got, ref, atol=1e-12, rtol=0)


def test_sampled_rows_match_full():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 1, 150, 8)).astype(np.float32)
    k = rng.standard_normal((2, 1, 150, 8)).astype(np.float32)
    full = quality.block_mass(q, k, 64)
    rows = [(0, 2), (1, 0)]
    got = quality.block_mass(q, k, 64, blocks=rows)
    assert np.array_equal(got[0], full[0, 0, 2]) and np.array_equal(got[1], full[1, 0, 0])


def test_row_quality_hand_example():
    """Masses 0.5, 0.3, 0.15, 0.05: 95 % is reached with three blocks."""
    mass = np.array([0.15, 0.5, 0.05, 0.3])
    lab = np.array([0, 1, -1, 0])
    r = quality.row_quality(mass, lab)
    assert math.isclose(r["critical"], 0.5) and math.isclose(r["marginal"], 0.45)
    assert math.isclose(r["negligible"], 0.05) and r["density95"] == 0.75


def test_rank_of_uniform_attention_is_one():
    """q = 0 makes every row of P the uniform distribution: rank 1."""
    rng = np.random.default_rng(6)
    q = np.zeros((64, 8))
    k = rng.standard_normal((64, 8))
    assert quality.rank_split(q, k, 0.08)["rank_full"] == 1
