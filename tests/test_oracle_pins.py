"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test fixes one part of the oracle with something independent of it:
a library routine the method reduces to in a special case (dense attention
= torch's scaled_dot_product_attention at 100% critical), an algebraic
identity (state-form linear attention = its quadratic form), a token-level
brute force with a different summation and sorting, exact rational
arithmetic for the means, the tie rule, and invariants of the definition.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

from oracle import brute
from oracle import oracle as orc
from sparse_attention_video_sla_amd.inputs import make_inputs, round_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_qkv(B, H, N, d, seed, scale=1.0, bf16=True):
    rng = np.random.default_rng(seed)
    q = (scale * rng.standard_normal((B, H, N, d))).astype(np.float32)
    k = (scale * rng.standard_normal((B, H, N, d))).astype(np.float32)
    v = rng.standard_normal((B, H, N, d)).astype(np.float32)
    w = (rng.standard_normal((d, d)) / math.sqrt(d)).astype(np.float32)
    if bf16:
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return q, k, v, w


def dense_o(res, B, H, N):
    return orc.rows_to_dense(res, B, H, N, "o")


# ---------------------------------------------------------------- counts


def test_counts_golden():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "counts.txt")) if l.strip() and not l.startswith("#")]
    assert rows
    for Nb, rc, rn, kc, kn in rows:
        assert orc.counts(int(Nb), float(rc), float(rn)) == (int(kc), int(kn))
        assert brute.counts(int(Nb), float(rc), float(rn)) == (int(kc), int(kn))


def test_counts_reject():
    for rc, rn in [(-0.1, 0.1), (0.6, 0.5), (1.1, 0.0), (0.2, -0.01)]:
        with pytest.raises(ValueError):
            orc.counts(100, rc, rn)


# ---------------------------------------------------------------- P-P pooling


def test_pool_exact_mean_bf16():
    """Means of bf16 values: the fp64 sum is exact, so the float32 result must be
    the correctly rounded rational mean (Fraction), ragged last block included."""
    rng = np.random.default_rng(1)
    x = round_bf16((rng.standard_normal((1, 2, 150, 8)) * 3).astype(np.float32))
    p = orc.pool(x, 64)
    assert p.shape == (1, 2, 3, 8)
    for h in range(2):
        for i in range(3):
            seg = x[0, h, i * 64:min(150, (i + 1) * 64)]
            for c in range(8):
                exact = sum(Fraction(float(t)) for t in seg[:, c]) / seg.shape[0]
                # float(Fraction) rounds correctly to fp64; the fp64 -> fp32 step must then
                # agree with rounding the rational directly (no double-rounding hazard here
                # because the fp64 mean of <= 64 bf16 values is itself exact or correctly rounded).
                assert p[0, h, i, c] == np.float32(float(exact))


def test_pool_ragged_divides_by_valid_count():
    x = np.ones((1, 1, 70, 4), np.float32)
    x[0, 0, 64:] = 2.0
    p = orc.pool(x, 64)
    assert np.all(p[0, 0, 0] == 1.0) and np.all(p[0, 0, 1] == 2.0)


# ---------------------------------------------------------------- P-S sums


def test_softmax_rows_sum_to_one():
    q, k, v, w = rand_qkv(1, 2, 300, 16, 2)
    qp, kp = orc.pool(q, 16), orc.pool(k, 16)
    cls = orc.classify(qp, kp, 0.1, 0.2, want_scores=True, want_pc=True)
    assert np.allclose(cls["pc"].sum(-1), 1.0, atol=1e-12, rtol=0)
    # P_c is the softmax of the scores / sqrt(d) (scipy as the independent routine)
    ref = scipy.special.softmax(cls["scores"] / math.sqrt(16), axis=-1)
    assert np.allclose(cls["pc"], ref, atol=1e-14, rtol=1e-12)
    ph = orc.phi(q)
    assert np.allclose(ph.sum(-1), 1.0, atol=1e-12, rtol=0)
    assert np.allclose(ph, scipy.special.softmax(q.astype(np.float64), axis=-1), rtol=1e-13, atol=0)


def test_sparse_probabilities_sum_to_one():
    """V = 1 and W = 0: every row that has a critical block outputs exactly 1."""
    q, k, _, _ = rand_qkv(1, 1, 200, 8, 3)
    v = np.ones_like(q)
    w = np.zeros((8, 8), np.float32)
    res = orc.forward(q, k, v, w, blk=16, rho_c=0.2, rho_n=0.3)
    assert np.allclose(res["o"][:, :200 % 16 or 16], 1.0, atol=1e-13)


def test_scores_are_fp64_dots_of_means():
    q, k, _, _ = rand_qkv(1, 1, 256, 32, 4, bf16=False)
    qp, kp = orc.pool(q, 64), orc.pool(k, 64)
    cls = orc.classify(qp, kp, 0.25, 0.25, want_scores=True)
    for i in range(4):
        for j in range(4):
            exact = math.fsum(float(a) * float(b) for a, b in zip(qp[0, 0, i], kp[0, 0, j]))
            assert abs(cls["scores"][0, 0, i, j] - exact) <= 1e-12 * max(1.0, abs(exact))


# ---------------------------------------------------------------- P-D dense


@pytest.mark.parametrize("N,blk,d", [(256, 64, 64), (200, 16, 8), (37, 8, 4), (130, 64, 128)])
def test_dense_equals_sdpa(N, blk, d):
    """100% critical: the sparse branch over every block is dense softmax
    attention over exactly the N valid tokens (pad keys of a ragged block
    excluded), and the linear branch is empty."""
    q, k, v, w = rand_qkv(1, 2, N, d, 10 + N, scale=1.5)
    res = orc.forward(q, k, v, w, blk=blk, rho_c=1.0, rho_n=0.0)
    assert np.all(res["mask"] == 1)
    o = dense_o(res, 1, 2, N)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64)), torch.from_numpy(k.astype(np.float64)),
        torch.from_numpy(v.astype(np.float64))).numpy()
    assert np.abs(o - ref).max() <= 1e-12


# ---------------------------------------------------------------- P-L linear


def quadratic_linear_attention(q, k, v):
    """sum_u (phi(q).phi(k_u)) v_u / sum_u phi(q).phi(k_u), phi = scipy softmax."""
    pq = scipy.special.softmax(q.astype(np.float64), axis=-1)
    pk = scipy.special.softmax(k.astype(np.float64), axis=-1)
    a = pq @ np.swapaxes(pk, -1, -2)
    return (a @ v.astype(np.float64)) / a.sum(-1, keepdims=True)


@pytest.mark.parametrize("N,blk,d", [(256, 64, 64), (100, 16, 8), (77, 8, 16)])
def test_all_marginal_equals_linear_attention(N, blk, d):
    """0% critical, 0% negligible: the output is normalised linear attention over
    all N tokens, projected by W with torch's Linear convention (x W^T)."""
    q, k, v, w = rand_qkv(1, 2, N, d, 20 + N)
    res = orc.forward(q, k, v, w, blk=blk, rho_c=0.0, rho_n=0.0)
    assert np.all(res["mask"] == 0)
    o = dense_o(res, 1, 2, N)
    lin = quadratic_linear_attention(q, k, v)
    ref = torch.nn.functional.linear(torch.from_numpy(lin), torch.from_numpy(w.astype(np.float64))).numpy()
    assert np.abs(o - ref).max() <= 1e-12
    o_l = orc.rows_to_dense(res, 1, 2, N, "o_l")
    assert np.abs(o_l - lin).max() <= 1e-12


# ---------------------------------------------------------------- P-B brute force


@pytest.mark.parametrize("N,blk,d,rc,rn", [
    (37, 4, 4, 0.2, 0.3), (64, 8, 8, 0.25, 0.25), (100, 16, 8, 0.3, 0.1),
    (256, 64, 64, 0.5, 0.25), (100, 8, 4, 0.0, 0.5), (100, 8, 4, 1.0, 0.0),
    (100, 8, 4, 0.0, 0.0), (120, 8, 8, 0.05, 0.10),
])
def test_brute_force(N, blk, d, rc, rn):
    q, k, v, w = rand_qkv(2, 1, N, d, 30 + N + blk)
    res = orc.forward(q, k, v, w, blk=blk, rho_c=rc, rho_n=rn)
    o_ref, lab = brute.forward(q, k, v, w, blk, rc, rn)
    assert np.array_equal(res["mask"], lab)
    assert np.abs(dense_o(res, 2, 1, N) - o_ref).max() <= 1e-12


def test_brute_force_generator_inputs():
    """The workload generator's structured (local) inputs on a small ragged grid."""
    inp = make_inputs(1, 2, (2, 6, 8), 16, "bf16", rope=False, seed=5, n_tokens=90)
    res = orc.forward(inp.q, inp.k, inp.v, inp.w, blk=8, rho_c=0.2, rho_n=0.3)
    o_ref, lab = brute.forward(inp.q, inp.k, inp.v, inp.w, 8, 0.2, 0.3)
    assert np.array_equal(res["mask"], lab)
    assert np.abs(dense_o(res, 1, 2, 90) - o_ref).max() <= 1e-12


# ---------------------------------------------------------------- P-K classification


def test_classify_counts_and_order():
    q, k, _, _ = rand_qkv(1, 3, 640, 16, 40)
    qp, kp = orc.pool(q, 64), orc.pool(k, 64)
    cls = orc.classify(qp, kp, 0.2, 0.3, want_scores=True)
    kc, kn = cls["k_c"], cls["k_n"]
    assert (kc, kn) == (2, 3)
    m, s = cls["mask"], cls["scores"]
    assert np.all((m == 1).sum(-1) == kc) and np.all((m == -1).sum(-1) == kn)
    for h in range(3):
        for i in range(10):
            crit, marg, negl = s[0, h, i][m[0, h, i] == 1], s[0, h, i][m[0, h, i] == 0], s[0, h, i][m[0, h, i] == -1]
            assert crit.min() >= marg.max() >= marg.min() >= negl.max()
            assert list(cls["crit"][0, h, i]) == sorted(np.nonzero(m[0, h, i] == 1)[0])
            assert list(cls["negl"][0, h, i]) == sorted(np.nonzero(m[0, h, i] == -1)[0])


def test_ties_zero_query():
    """Q = 0: every score is exactly 0, so the total order is the block index:
    critical = the lowest k_c indices, negligible = the highest k_n."""
    _, k, _, _ = rand_qkv(1, 1, 640, 8, 41)
    qp = np.zeros((1, 1, 10, 8), np.float32)
    kp = orc.pool(k, 64)
    cls = orc.classify(qp, kp, 0.3, 0.2)
    for i in range(10):
        assert list(cls["crit"][0, 0, i]) == [0, 1, 2]
        assert list(cls["negl"][0, 0, i]) == [8, 9]


def test_ties_duplicated_blocks():
    """Duplicated key blocks score exactly alike; the lower index ranks higher
    at both ends of the order."""
    rng = np.random.default_rng(42)
    kp = np.zeros((1, 1, 8, 4), np.float32)
    base = rng.standard_normal((3, 4)).astype(np.float32)
    # blocks 1, 4, 6 share the largest direction; blocks 0, 3 share the smallest
    q = np.array([[[[1, 0, 0, 0]]]], np.float32)
    for j, val in enumerate([-5, 9, 2, -5, 9, 1, 9, 3]):
        kp[0, 0, j] = [val, *base[j % 3, 1:]]
    qp = np.repeat(q, 8, axis=2)
    cls = orc.classify(qp, kp, 2 / 8, 1 / 8)     # k_c = 2, k_n = 1
    assert list(cls["crit"][0, 0, 0]) == [1, 4]  # 6 ties with 1 and 4 but has the higher index
    assert list(cls["negl"][0, 0, 0]) == [3]     # 0 and 3 tie at the bottom; the higher index is last
    assert cls["mask"][0, 0, 0, 6] == 0 and cls["mask"][0, 0, 0, 0] == 0


# ---------------------------------------------------------------- P-I invariants


def _mixed_case():
    inp = make_inputs(1, 2, (4, 8, 8), 32, "f32", rope=False, seed=7)
    return inp.q, inp.k, inp.v, inp.w


def test_value_offset_invariant():
    """With critical and marginal blocks in every row: V -> V + v0 gives
    O -> O + v0 + W v0 (both branches are weighted averages of V)."""
    q, k, v, w = _mixed_case()
    rc, rn = 0.2, 0.3
    r0 = orc.forward(q, k, v, w, blk=16, rho_c=rc, rho_n=rn)
    assert np.all((r0["mask"] == 1).sum(-1) > 0) and np.all((r0["mask"] == 0).sum(-1) > 0)
    # bf16 V plus a dyadic offset is exact in float32, so the shift is exact too
    v = round_bf16(v)
    r0 = orc.forward(q, k, v, w, blk=16, rho_c=rc, rho_n=rn)
    v0 = (np.arange(32, dtype=np.float32) - 16) / 8
    assert np.array_equal((v + v0) - v0, v)
    r1 = orc.forward(q, k, v + v0, w, blk=16, rho_c=rc, rho_n=rn)
    shift = v0.astype(np.float64) + w.astype(np.float64) @ v0.astype(np.float64)
    assert np.abs(r1["o"] - r0["o"] - shift).max() <= 1e-11


def test_linear_in_v_and_mask_independent_of_v():
    q, k, _, w = _mixed_case()
    # values on a 1/8 grid, so 2 v + 3 v2 is exact in float32
    rng = np.random.default_rng(8)
    v = (rng.integers(-64, 64, size=q.shape) / 8).astype(np.float32)
    v2 = (rng.integers(-64, 64, size=q.shape) / 8).astype(np.float32)
    a = orc.forward(q, k, v, w, blk=16, rho_c=0.2, rho_n=0.3)
    b = orc.forward(q, k, v2, w, blk=16, rho_c=0.2, rho_n=0.3)
    c = orc.forward(q, k, (2 * v + 3 * v2).astype(np.float32), w, blk=16, rho_c=0.2, rho_n=0.3)
    assert np.array_equal(a["mask"], b["mask"])
    assert np.abs(c["o"] - (2 * a["o"] + 3 * b["o"])).max() <= 1e-11


def test_projection_scales_only_linear_part():
    q, k, v, w = _mixed_case()
    a = orc.forward(q, k, v, w, blk=16, rho_c=0.2, rho_n=0.3)
    b = orc.forward(q, k, v, (4 * w).astype(np.float32), blk=16, rho_c=0.2, rho_n=0.3)  # exact scaling
    assert np.abs(b["o_s"] - a["o_s"]).max() == 0
    assert np.abs(b["o"] - a["o_s"] - 4 * (a["o"] - a["o_s"])).max() <= 1e-12


def test_permute_within_block():
    """bf16 inputs: permuting tokens inside each block leaves the means (exact
    fp64 sums) and so the mask unchanged, and permutes the output rows."""
    q, k, v, w = rand_qkv(1, 1, 128, 16, 9)
    perm = np.concatenate([np.random.default_rng(1).permutation(32) + 32 * b for b in range(4)])
    a = orc.forward(q, k, v, w, blk=32, rho_c=0.25, rho_n=0.25)
    b = orc.forward(q[:, :, perm], k[:, :, perm], v[:, :, perm], w, blk=32, rho_c=0.25, rho_n=0.25)
    assert np.array_equal(a["mask"], b["mask"])
    oa, ob = dense_o(a, 1, 1, 128), dense_o(b, 1, 1, 128)
    assert np.abs(ob - oa[:, :, perm]).max() <= 1e-12


def test_negligible_blocks_do_not_matter():
    """Changing the K and V tokens of a block that is negligible for a row
    changes nothing in that row unless it changes the labels."""
    q, k, v, w = _mixed_case()
    a = orc.forward(q, k, v, w, blk=16, rho_c=0.2, rho_n=0.3)
    m = a["mask"][0, 0, 0]
    j = int(np.nonzero(m == -1)[0][0])
    v2 = v.copy()
    v2[0, 0, 16 * j:16 * (j + 1)] += 100.0
    b = orc.forward(q, k, v2, w, blk=16, rho_c=0.2, rho_n=0.3)
    assert np.array_equal(a["mask"], b["mask"])
    assert np.abs(a["o"][0] - b["o"][0]).max() == 0


def test_sampled_rows_match_full():
    q, k, v, w = _mixed_case()
    full = orc.forward(q, k, v, w, blk=16, rho_c=0.2, rho_n=0.3)
    rows = np.array([[0, 3], [1, 0], [1, 15]], np.int32)
    part = orc.forward(q, k, v, w, blk=16, rho_c=0.2, rho_n=0.3, rows=rows)
    for r, (bh, i) in enumerate(rows):
        idx = list(map(tuple, full["rows"])).index((bh, i))
        assert np.array_equal(part["o"][r], full["o"][idx])


@pytest.mark.parametrize("B,H,N,d", [(1, 2, 1000, 128), (2, 1, 777, 64), (1, 1, 64, 16)])
def test_dense_rows_equal_c_oracle_at_full_critical(B, H, N, d):
    """oracle/dense.py (matrix products over all keys) against the C oracle's
    sparse branch with every block critical, on ragged shapes and sampled
    blocks: the same dense softmax attention from two independent codes."""
    from oracle import dense
    q, k, v, w = rand_qkv(B, H, N, d, seed=N + d)
    Nb = -(-N // 64)
    rows = np.array([(bh, i) for bh in range(B * H) for i in range(Nb) if (i * 7 + bh) % 3 != 1 or i == Nb - 1],
                    np.int32)
    ref = orc.forward(q, k, v, w, 64, 1.0, 0.0, rows=rows)["o"]
    got = dense.attention_rows(q, k, v, rows)
    assert np.abs(got - ref).max() <= 1e-12
