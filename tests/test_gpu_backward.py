"""GPU parity of the SLA backward pass (sla_backward) against the fp64
autograd oracle (oracle/backward.py), with the block labels from the C
oracle's classification (bit-identical to the GPU's).  Bar: relative L2
error <= 1e-2 for each of dq, dk, dv, dw (bf16 inputs; P and dS go to the
matrix cores in bf16, 2^-9 relative rounding, accumulated in fp32)."""
import sys

import numpy as np
import pytest

from oracle import backward as ob
from oracle import oracle as orc
from sparse_attention_video_sla_amd.inputs import make_inputs, round_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def sla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_video_sla_amd as sla
    sla._lib.load()
    return sla


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(torch.bfloat16)


@pytest.mark.parametrize("B,H,N,d,rc,rn", [
    (1, 2, 1000, 128, 0.25, 0.25),
    (1, 1, 777, 64, 0.1, 0.2),      # ragged last block
    (2, 1, 640, 128, 1.0, 0.0),     # dense: no linear branch
    (1, 1, 600, 64, 0.0, 0.5),      # no critical block: linear branch only
    (1, 1, 2048, 128, 0.05, 0.10),  # the default fractions
    (2, 2, 700, 64, 0.2, 0.3),      # dW summed over batch and heads, ragged
])
def test_backward_matches_oracle(sla, B, H, N, d, rc, rn):
    say("backward", B, H, N, d, rc, rn)
    inp = make_inputs(B, H, (1, 1, N), d, "bf16", seed=N + d)
    rng = np.random.default_rng(N)
    dout = round_bf16(rng.standard_normal((B, H, N, d)).astype(np.float32))
    qp, kp = orc.pool(inp.q), orc.pool(inp.k)
    mask = orc.classify(qp, kp, rc, rn)["mask"]
    _, rq, rk, rv, rw = ob.gradients(inp.q, inp.k, inp.v, inp.w, mask, dout)
    w = torch.from_numpy(inp.w).cuda()
    dq, dk, dv, dw = sla.backward(dev(inp.q), dev(inp.k), dev(inp.v), w, dev(dout), rc, rn)
    torch.cuda.synchronize()
    worst = 0.0
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv), ("dw", dw, rw)):
        g = got.double().cpu().numpy()
        nr = np.linalg.norm(ref)
        rel = np.linalg.norm(g - ref) / nr if nr > 0 else np.linalg.norm(g)
        say("  %s rel %.3g max|d| %.3g max|ref| %.3g" % (name, rel, np.abs(g - ref).max(), np.abs(ref).max()))
        assert np.isfinite(g).all()
        worst = max(worst, rel)
    assert worst <= 1e-2


@pytest.mark.parametrize("gscale", [2.0 ** -40, 2.0 ** 20])
def test_backward_gradient_scale(sla, gscale):
    """The same bar for an output gradient scaled far from 1: the linear
    part's f16 operands take a power-of-two scale per block, so the relative
    error does not depend on the gradient's magnitude."""
    B, H, N, d, rc, rn = 1, 1, 1100, 128, 0.1, 0.2
    say("backward scale", gscale)
    inp = make_inputs(B, H, (1, 1, N), d, "bf16", seed=31)
    rng = np.random.default_rng(32)
    dout = round_bf16((rng.standard_normal((B, H, N, d)) * gscale).astype(np.float32))
    mask = orc.classify(orc.pool(inp.q), orc.pool(inp.k), rc, rn)["mask"]
    _, rq, rk, rv, rw = ob.gradients(inp.q, inp.k, inp.v, inp.w, mask, dout)
    w = torch.from_numpy(inp.w).cuda()
    dq, dk, dv, dw = sla.backward(dev(inp.q), dev(inp.k), dev(inp.v), w, dev(dout), rc, rn)
    torch.cuda.synchronize()
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv), ("dw", dw, rw)):
        g = got.double().cpu().numpy()
        rel = np.linalg.norm(g - ref) / np.linalg.norm(ref)
        say("  %s rel %.3g" % (name, rel))
        assert np.isfinite(g).all() and rel <= 1e-2


def test_backward_full_size_sampled_blocks(sla):
    """The Wan2.1 480p workload (B=1, H=12, N=32760, d=128, 5 % / 10 %) in one
    call, as the backward bench runs it; the oracle computes one head's
    gradients on sampled blocks exactly (gradients_blocks): dq of the first,
    an interior and the ragged last query block, dk and dv of three key
    blocks.  Same bar per gradient over the sampled rows."""
    from sparse_attention_video_sla_amd.inputs import make_workload
    inp = make_workload(1)
    B, H, N, d = inp.q.shape
    rc, rn = 0.05, 0.10
    rng = np.random.default_rng(77)
    dout = round_bf16(rng.standard_normal((B, H, N, d)).astype(np.float32))
    say("backward full size", B, H, N, d)
    w = torch.from_numpy(inp.w).cuda()
    dq, dk, dv, dw = sla.backward(dev(inp.q), dev(inp.k), dev(inp.v), w, dev(dout), rc, rn)
    torch.cuda.synchronize()
    mask = orc.classify(orc.pool(inp.q), orc.pool(inp.k), rc, rn)["mask"]
    Nb = -(-N // 64)
    h, qb, kb = 5, [0, 137, Nb - 1], [0, 300, Nb - 1]
    gq, gk, gv, _ = ob.gradients_blocks(inp.q[0, h], inp.k[0, h], inp.v[0, h], inp.w, mask[0, h], dout[0, h], qb, kb)
    rows = lambda blocks: np.concatenate([np.arange(b * 64, min(N, (b + 1) * 64)) for b in blocks])
    for name, got, ref, blocks in (("dq", dq, gq, qb), ("dk", dk, gk, kb), ("dv", dv, gv, kb)):
        g = got[0, h].double().cpu().numpy()[rows(blocks)]
        rel = np.linalg.norm(g - ref) / np.linalg.norm(ref)
        say("  %s rel %.3g max|d| %.3g max|ref| %.3g" % (name, rel, np.abs(g - ref).max(), np.abs(ref).max()))
        assert np.isfinite(g).all() and rel <= 1e-2
