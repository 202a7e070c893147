"""GPU parity of the LVSA path: the frame sets built on the device
(sla_lvsa_sets) bit-exact against the oracle's, and the attention
(sla_forward_lvsa) against the fp64 oracle (oracle/lvsa.py) with the bf16
bar of the forward pass: max|d| <= 1e-2 and relative L2 <= 5e-3."""
import sys

import numpy as np
import pytest

from oracle import lvsa
from sparse_attention_video_sla_amd.inputs import LVSA_WORKLOADS, make_inputs, make_lvsa_workload, sample_query_blocks

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


def check(got, ref):
    got = np.asarray(got, np.float64)
    d = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    say("  max|d| %.3g rel %.3g" % (d.max(), rel))
    assert d.max() <= 1e-2 and rel <= 5e-3


SET_GRID = [(T, C, W) for T in (1, 2, 5, 10, 22, 41, 121, 300) for C in (4, 7, 21) for W in (0, 1, 3)
            if C - (2 * W + 1) >= 1]


def test_lvsa_sets_bit_exact(sla):
    say("lvsa sets", len(SET_GRID), "configurations")
    for T, C, W in SET_GRID:
        Tp = lvsa.period(T, C, W)
        for s in sorted({0, 1, Tp - 1, Tp, 2 * Tp + 1}):
            sets, cnt = sla.lvsa_sets(T, C, W, s)
            sets, cnt = sets.cpu().numpy(), cnt.cpu().numpy()
            for t, ref in enumerate(lvsa.all_sets(T, C, W, s)):
                assert cnt[t] == len(ref) and list(sets[t, :cnt[t]]) == ref, (T, C, W, s, t)


@pytest.mark.parametrize("B,H,T,P,d,C,W,s", [
    (1, 2, 9, 100, 128, 5, 1, 0),       # frames of 100 tokens: most blocks straddle a boundary
    (1, 2, 9, 100, 128, 5, 1, 2),
    (2, 1, 6, 64, 64, 5, 1, 1),         # frames aligned with blocks
    (1, 1, 10, 130, 128, 7, 1, 3),
    (1, 1, 12, 97, 64, 6, 0, 5),        # W = 0, ragged last block
    (1, 1, 1, 300, 128, 3, 0, 0),       # one frame: dense attention
    (1, 1, 4, 70, 128, 21, 3, 0),       # T_per = 1: every frame global
    (1, 1, 30, 640, 64, 21, 3, 0),      # 300 slots per row: the chunked schedule
    (1, 1, 31, 620, 128, 21, 3, 1),     # chunked, frames straddling blocks, ragged last block
])
@pytest.mark.timeout(600)
def test_forward_lvsa_all_rows(sla, B, H, T, P, d, C, W, s):
    say("lvsa", B, H, T, P, d, C, W, s)
    inp = make_inputs(B, H, (T, 1, P), d, "bf16", seed=T * P + s)
    out = sla.forward_lvsa(dev(inp.q), dev(inp.k), dev(inp.v), T, C, W, s)
    torch.cuda.synchronize()
    check(out.double().cpu().numpy(), lvsa.attention_lvsa(inp.q, inp.k, inp.v, T, P, C, W, s))


def test_forward_lvsa_bf16_output_and_reuse(sla):
    T, P, C, W, s = 9, 100, 5, 1, 1
    inp = make_inputs(1, 1, (T, 1, P), 128, "bf16", seed=77)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    a = sla.forward_lvsa(q, k, v, T, C, W, s, out_dtype=torch.bfloat16)
    b = sla.forward_lvsa(q, k, v, T, C, W, s)
    torch.cuda.synchronize()
    assert (a.float() - b).abs().max().item() <= 2.0 ** -8 * b.abs().max().item() + 1e-6
    ref = lvsa.attention_lvsa(inp.q, inp.k, inp.v, T, P, C, W, s)
    check(b.double().cpu().numpy(), ref)


def test_forward_lvsa_rejects_bad_shapes(sla):
    q = torch.zeros((1, 1, 1000, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sla.SlaError):
        sla.forward_lvsa(q, q, q, 3, 5, 1, 0)          # N not a multiple of T
    with pytest.raises(sla.SlaError):
        sla.forward_lvsa(q, q, q, 20, 5, 1, 0)         # frames of 50 tokens
    with pytest.raises(sla.SlaError):
        sla.forward_lvsa(q, q, q, 10, 3, 1, 0)         # C <= 2W + 1


@pytest.mark.timeout(600)
def test_lvsa_workload_sampled(sla):
    """Wan2.1 1.3B at 6x length (121 x 30 x 52 tokens, C = 21, W = 3), two of
    its heads: sampled query blocks (the first, the last, and blocks that
    straddle a frame boundary) against the oracle."""
    wl = LVSA_WORKLOADS["wan6x"]
    say("lvsa workload", wl.name)
    inp = make_lvsa_workload("wan6x", heads=2)
    out = sla.forward_lvsa(dev(inp.q), dev(inp.k), dev(inp.v), wl.T, wl.C, wl.W, wl.step)
    torch.cuda.synchronize()
    Nb = -(-wl.N // 64)
    straddle = [i for i in range(Nb) if (64 * i) // wl.P != min(64 * i + 63, wl.N - 1) // wl.P]
    rows = sample_query_blocks(1, 2, Nb, 4, 11, include=(0, Nb - 1, straddle[0], straddle[len(straddle) // 2]))
    ref = lvsa.attention_lvsa(inp.q, inp.k, inp.v, wl.T, wl.P, wl.C, wl.W, wl.step, rows=[tuple(r) for r in rows])
    o = out.reshape(2, wl.N, wl.d)
    got = np.zeros_like(ref)
    for x, (bh, i) in enumerate(rows):
        r1 = min(wl.N, 64 * (i + 1))
        got[x, :r1 - 64 * i] = o[bh, 64 * i:r1].double().cpu().numpy()
    check(got, ref)
    assert torch.isfinite(out).all()
