"""GPU parity of the SLA backward pass (sla_backward) against the fp64
autograd oracle (oracle/backward.py), with the block labels from the C
oracle's classification (bit-identical to the GPU's).  Bar, for each of dq,
dk, dv and dw: relative L2 error <= 1e-2 and every element within 2e-2 of
the largest magnitude of that gradient's reference (bf16 inputs; P and dS
go to the matrix cores in bf16, 2^-9 relative rounding, accumulated in
fp32; the linear branch in fp16 with a power-of-two scale per block)."""
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


REL_L2, REL_ELEM = 1e-2, 2e-2


def check(name, g, ref):
    """Relative L2 and a per-element bound scaled by the reference's largest
    magnitude (an all-zero reference must give all zeros)."""
    assert np.isfinite(g).all(), name
    d = np.abs(g - ref)
    mref = np.abs(ref).max()
    nr = np.linalg.norm(ref)
    rel = np.linalg.norm(g - ref) / nr if nr > 0 else np.linalg.norm(g)
    say("  %s rel %.3g max|d| %.3g max|ref| %.3g (max|d| / max|ref| %.3g)"
        % (name, rel, d.max(), mref, d.max() / mref if mref > 0 else d.max()))
    assert rel <= REL_L2, (name, rel)
    if mref > 0:
        assert d.max() <= REL_ELEM * mref, (name, np.unravel_index(d.argmax(), d.shape), d.max(), mref)
    else:
        assert d.max() == 0.0, name


@pytest.mark.parametrize("B,H,N,d,rc,rn", [
    (1, 2, 1000, 128, 0.25, 0.25),
    (1, 1, 777, 64, 0.1, 0.2),      # ragged last block
    (2, 1, 640, 128, 1.0, 0.0),     # dense: no linear branch
    (1, 1, 600, 64, 0.0, 0.5),      # no critical block: linear branch only
    (1, 1, 2048, 128, 0.05, 0.10),  # the default fractions
    (2, 2, 700, 64, 0.2, 0.3),      # dW summed over batch and heads, ragged
    # degenerate sizes (a single token is left out: its dq and dk are exactly
    # zero, which products rounded to bf16 cannot cancel to the bit)
    (1, 1, 65, 64, 0.5, 0.5),       # two blocks, the last of one token, no marginal block
    (2, 1, 129, 128, 0.0, 0.0),     # linear only over three blocks, one-token tail
    (1, 1, 37, 64, 1.0, 0.0),       # one ragged block, dense
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
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv), ("dw", dw, rw)):
        check(name, got.double().cpu().numpy(), ref)


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
        check(name, got.double().cpu().numpy(), ref)


@pytest.mark.timeout(900)
def test_backward_full_size(sla):
    """The Wan2.1 480p workload (B=1, H=12, N=32760, d=128, 5 % / 10 %) in one
    call, as the backward bench runs it.  The oracle computes, exactly on
    selected blocks (gradients_blocks): dq of the first, two interior and the
    ragged last query block and dk, dv of four key blocks, on three heads; and
    every head's dW, summed over the twelve heads as the GPU's dw is."""
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
    dq, dk, dv, dw = (x.double().cpu().numpy() for x in (dq, dk, dv, dw))
    mask = orc.classify(orc.pool(inp.q), orc.pool(inp.k), rc, rn)["mask"]
    Nb = -(-N // 64)
    qb, kb = [0, 137, 301, Nb - 1], [0, 55, 300, Nb - 1]
    rows = lambda blocks: np.concatenate([np.arange(b * 64, min(N, (b + 1) * 64)) for b in blocks])
    dw_ref = np.zeros((d, d))
    for h in range(H):
        sampled = h in (0, 5, 11)
        gq, gk, gv, gw = ob.gradients_blocks(inp.q[0, h], inp.k[0, h], inp.v[0, h], inp.w, mask[0, h], dout[0, h],
                                             qb if sampled else [0], kb if sampled else [0])
        dw_ref += gw
        if sampled:
            say(" head", h)
            for name, got, ref, blocks in (("dq", dq, gq, qb), ("dk", dk, gk, kb), ("dv", dv, gv, kb)):
                check(name, got[0, h][rows(blocks)], ref)
    check("dw (12 heads)", dw, dw_ref)


def test_backward_deterministic(sla):
    """Two calls on the same inputs give the same bits in every gradient,
    dW (a sum over workgroups) included."""
    B, H, N, d, rc, rn = 2, 3, 3000, 128, 0.05, 0.10
    inp = make_inputs(B, H, (1, 1, N), d, "bf16", seed=5)
    rng = np.random.default_rng(6)
    dout = dev(round_bf16(rng.standard_normal((B, H, N, d)).astype(np.float32)))
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    w = torch.from_numpy(inp.w).cuda()
    a = sla.backward(q, k, v, w, dout, rc, rn)
    b = sla.backward(q, k, v, w, dout, rc, rn)
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv", "dw"), a, b):
        assert torch.equal(x, y), name


@pytest.mark.parametrize("B,H,N,d,rc,rn,out_bf16", [
    (1, 2, 1000, 128, 0.25, 0.25, False),
    (1, 1, 777, 64, 0.1, 0.2, True),      # ragged last block, bf16 output
    (2, 1, 640, 128, 1.0, 0.0, False),    # dense: no linear branch
    (1, 1, 600, 64, 0.0, 0.5, False),     # no critical block: linear branch only
    (2, 2, 2100, 128, 0.05, 0.10, True),  # the default fractions, ragged
])
def test_backward_saved_equals_recompute(sla, B, H, N, d, rc, rn, out_bf16):
    """sla_forward_save gives sla_forward's output and labels bit for bit,
    and sla_backward_saved on what it saved gives sla_backward's gradients
    bit for bit, also when run a second time on the same saved state with
    another output gradient."""
    say("saved", B, H, N, d, rc, rn, out_bf16)
    inp = make_inputs(B, H, (1, 1, N), d, "bf16", seed=N + 3)
    rng = np.random.default_rng(N + 4)
    douts = [dev(round_bf16(rng.standard_normal((B, H, N, d)).astype(np.float32))) for _ in range(2)]
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    w = torch.from_numpy(inp.w).cuda()
    odt = torch.bfloat16 if out_bf16 else torch.float32
    ref_out, ref_mask = sla.forward(q, k, v, w, rc, rn, out_dtype=odt, return_mask=True)
    out, mask, saved = sla.forward_save(q, k, v, w, rc, rn, out_dtype=odt, return_mask=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    assert torch.equal(mask, ref_mask)
    for t, dout in enumerate(douts):
        a = sla.backward(q, k, v, w, dout, rc, rn)
        b = sla.backward_saved(saved, q, k, v, w, dout)
        torch.cuda.synchronize()
        for name, x, y in zip(("dq", "dk", "dv", "dw"), a, b):
            assert torch.equal(x, y), (name, t)


@pytest.mark.timeout(300)
def test_backward_saved_full_size(sla):
    """The same identities at the Wan2.1 480p workload (B=1, H=12, N=32760,
    d=128, 5 % / 10 %), as the backward bench runs it."""
    from sparse_attention_video_sla_amd.inputs import make_workload
    inp = make_workload(1)
    B, H, N, d = inp.q.shape
    rc, rn = 0.05, 0.10
    rng = np.random.default_rng(78)
    dout = dev(round_bf16(rng.standard_normal((B, H, N, d)).astype(np.float32)))
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    w = torch.from_numpy(inp.w).cuda()
    say("saved full size", B, H, N, d)
    ref_out = sla.forward(q, k, v, w, rc, rn)
    out, saved = sla.forward_save(q, k, v, w, rc, rn)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    del ref_out, out
    a = sla.backward(q, k, v, w, dout, rc, rn)
    b = sla.backward_saved(saved, q, k, v, w, dout)
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv", "dw"), a, b):
        assert torch.equal(x, y), name
