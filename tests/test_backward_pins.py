"""Pins of the backward oracle (oracle/backward.py): its token-level forward
against the C oracle's forward, its gradients against central finite
differences of that forward, and against torch's scaled_dot_product_attention
backward when every block is critical."""
import numpy as np
import pytest

from oracle import backward as ob
from oracle import oracle as orc

torch = pytest.importorskip("torch")


def rand(B, H, N, d, seed):
    rng = np.random.default_rng(seed)
    q, k, v = [rng.standard_normal((B, H, N, d)).astype(np.float32) for _ in range(3)]
    w = (rng.standard_normal((d, d)) / np.sqrt(d)).astype(np.float32)
    return q, k, v, w


@pytest.mark.parametrize("B,H,N,d,rc,rn", [(1, 2, 300, 16, 0.25, 0.25), (2, 1, 256, 8, 0.5, 0.0),
                                           (1, 1, 200, 16, 0.0, 0.5), (1, 1, 130, 8, 1.0, 0.0)])
def test_token_forward_matches_c_oracle(B, H, N, d, rc, rn):
    q, k, v, w = rand(B, H, N, d, N + d)
    res = orc.forward(q, k, v, w, 64, rc, rn)
    ref = orc.rows_to_dense(res, B, H, N, "o")
    crit, marg = ob.token_masks(res["mask"], N)
    t = lambda x: torch.from_numpy(np.asarray(x, np.float64).reshape(B * H, N, d))
    got = ob.forward_tokens(t(q), t(k), t(v), torch.from_numpy(w.astype(np.float64)), crit, marg)
    assert np.allclose(got.numpy().reshape(B, H, N, d), ref, atol=1e-10)


def test_gradients_match_central_differences():
    B, H, N, d = 1, 1, 150, 4
    q, k, v, w = rand(B, H, N, d, 5)
    res = orc.forward(q, k, v, w, 64, 0.34, 0.34)
    mask = res["mask"]
    rng = np.random.default_rng(6)
    dout = rng.standard_normal((B, H, N, d))
    _, dq, dk, dv, dw = ob.gradients(q, k, v, w, mask, dout)
    crit, marg = ob.token_masks(mask, N)

    def loss(q_, k_, v_, w_):
        t = lambda x: torch.from_numpy(np.asarray(x, np.float64).reshape(B * H, N, d))
        o = ob.forward_tokens(t(q_), t(k_), t(v_), torch.from_numpy(np.asarray(w_, np.float64)), crit, marg)
        return float((o.numpy().reshape(B, H, N, d) * dout).sum())

    base = [np.asarray(x, np.float64) for x in (q, k, v, w)]
    grads = [dq, dk, dv, dw]
    eps = 1e-6
    for which in range(4):
        g = grads[which]
        for idx in [tuple(rng.integers(0, s) for s in g.shape) for _ in range(6)]:
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (which, idx, fd, g[idx])


def test_all_critical_is_sdpa_backward():
    B, H, N, d = 1, 2, 200, 8
    q, k, v, w = rand(B, H, N, d, 7)
    Nb = 4
    mask = np.ones((B, H, Nb, Nb), np.int8)
    rng = np.random.default_rng(8)
    dout = rng.standard_normal((B, H, N, d))
    _, dq, dk, dv, dw = ob.gradients(q, k, v, w, mask, dout)
    t = lambda x: torch.tensor(np.asarray(x, np.float64), requires_grad=True)
    tq, tk, tv = t(q), t(k), t(v)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    gq, gk, gv = torch.autograd.grad(o, (tq, tk, tv), torch.from_numpy(dout))
    assert np.allclose(dq, gq.numpy(), atol=1e-10) and np.allclose(dk, gk.numpy(), atol=1e-10)
    assert np.allclose(dv, gv.numpy(), atol=1e-10) and np.abs(dw).max() == 0.0


@pytest.mark.parametrize("N,d,rc,rn,seed", [(300, 16, 0.25, 0.25, 1), (200, 8, 0.0, 0.5, 2), (450, 8, 0.3, 0.0, 3),
                                            (260, 16, 0.4, 0.2, 4)])
def test_block_gradients_match_full(N, d, rc, rn, seed):
    """gradients_blocks (sparse rows restricted to the blocks that matter,
    linear sums grouped by key block) gives the full autograd gradients of
    those rows, and the head's whole dW."""
    q, k, v, w = rand(1, 1, N, d, seed)
    mask = orc.forward(q, k, v, w, 64, rc, rn)["mask"]
    dout = np.random.default_rng(seed + 50).standard_normal((1, 1, N, d))
    _, dq, dk, dv, dw = ob.gradients(q, k, v, w, mask, dout)
    Nb = -(-N // 64)
    qb, kb = [0, Nb - 1], [1, Nb - 1]
    gq, gk, gv, gw = ob.gradients_blocks(q[0, 0], k[0, 0], v[0, 0], w, mask[0, 0], dout[0, 0], qb, kb)
    rows = lambda blocks: np.concatenate([np.arange(b * 64, min(N, (b + 1) * 64)) for b in sorted(blocks)])
    assert np.allclose(gq, dq[0, 0, rows(qb)], atol=1e-10, rtol=0)
    assert np.allclose(gk, dk[0, 0, rows(kb)], atol=1e-10, rtol=0)
    assert np.allclose(gv, dv[0, 0, rows(kb)], atol=1e-10, rtol=0)
    assert np.allclose(gw, dw, atol=1e-10, rtol=0)
