"""GPU parity of the mask-quality diagnostics (sla_block_mass, sla_mask_stats)
against the fp64 oracle (oracle/quality.py).

Bars: block masses within 5e-5 absolute of the oracle (fp32 accumulation of
exp2 over up to N keys; masses are <= 1) and rows summing to 1 within 1e-4;
from the statistics kernel, given the GPU's float32 masses, the class
masses within float32 rounding (relative 2^-23) of the oracle's fp64 sums
and the 95 % density equal to the oracle's (both count by fp64 sums).
"""
import sys

import numpy as np
import pytest

from oracle import oracle as orc
from oracle import quality
from sparse_attention_video_sla_amd.inputs import WORKLOADS, make_inputs, make_workload, sample_query_blocks

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


@pytest.mark.parametrize("B,H,N,d", [(1, 2, 1000, 128), (2, 1, 777, 64), (1, 1, 4096, 128)])
def test_block_mass_matches_oracle(sla, B, H, N, d):
    say("block mass", B, H, N, d)
    inp = make_inputs(B, H, (1, 1, N), d, "bf16", seed=N + d)
    mass = sla.block_mass(dev(inp.q), dev(inp.k))
    torch.cuda.synchronize()
    got = mass.cpu().numpy().astype(np.float64)
    ref = quality.block_mass(inp.q, inp.k, 64)
    err = np.abs(got - ref).max()
    say("  max|d| %.3g" % err)
    assert err <= 5e-5
    assert np.abs(got.sum(axis=-1) - 1.0).max() <= 1e-4


def test_block_mass_deterministic(sla):
    inp = make_inputs(1, 2, (1, 1, 2000), 128, "bf16", seed=9)
    q, k = dev(inp.q), dev(inp.k)
    a = sla.block_mass(q, k)
    b = sla.block_mass(q, k)
    assert torch.equal(a, b)


@pytest.mark.parametrize("N,rc,rn", [(3000, 0.05, 0.10), (32760, 0.05, 0.10), (4096, 0.3, 0.2)])
def test_mask_stats_match_oracle(sla, N, rc, rn):
    """Every row: the oracle's row_quality on the GPU's own float32 masses."""
    say("mask stats", N, rc, rn)
    d = 128
    inp = make_inputs(1, 2, (1, 1, N), d, "bf16", seed=12 + N)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    w = torch.from_numpy(inp.w).to("cuda")
    _, mask = sla.forward(q, k, v, w, rc, rn, return_mask=True)
    mass = sla.block_mass(q, k)
    stats = sla.mask_stats(mass, mask)
    torch.cuda.synchronize()
    m, lab, st = mass.cpu().numpy().astype(np.float64), mask.cpu().numpy(), stats.cpu().numpy()
    Nb = m.shape[-1]
    worst, differ = 0.0, 0
    for bh in range(2):
        for i in range(Nb):
            r = quality.row_quality(m[0, bh, i], lab[0, bh, i])
            got = st[0, bh, i].astype(np.float64)
            for x, key in enumerate(("critical", "marginal", "negligible")):
                err = abs(got[x] - r[key])
                worst = max(worst, err)
                assert err <= 2.0 ** -23 * abs(r[key]) + 1e-30, (bh, i, key, got[x], r[key])
            differ += int(round(got[3] * Nb)) != int(round(r["density95"] * Nb))
    say("  class masses max|d| %.3g, density rows differing: %d of %d" % (worst, differ, 2 * Nb))
    assert differ == 0


def test_mask_stats_hand_rows(sla):
    """Rows with known answers, including ties at the 95 % threshold."""
    Nb = 8
    mass = np.zeros((1, 1, 3, Nb), np.float32)
    mass[0, 0, 0] = [0.5, 0.3, 0.16, 0.04, 0, 0, 0, 0]          # 0.95 reached with 3 blocks
    mass[0, 0, 1] = [0.125] * 8                                   # uniform: 0.95 needs 8 blocks
    mass[0, 0, 2] = [0.4, 0.2, 0.2, 0.2, 0, 0, 0, 0]              # ties at the threshold: 4 blocks
    lab = np.zeros((1, 1, 3, Nb), np.int8)
    lab[0, 0, :, 0] = 1
    lab[0, 0, :, 3] = -1
    st = sla.mask_stats(torch.from_numpy(mass).cuda(), torch.from_numpy(lab).cuda()).cpu().numpy()[0, 0]
    assert np.allclose(st[:, 3] * Nb, [3, 8, 4])
    assert np.allclose(st[0, :3], [0.5, 0.46, 0.04], atol=1e-7)
    assert np.allclose(st[:, :3].sum(axis=1), 1.0, atol=1e-6)


@pytest.mark.timeout(600)
def test_block_mass_workload1_sampled(sla):
    """Wan2.1 480p shape: sampled rows of blocks against the oracle, every row sums to 1."""
    wl = WORKLOADS[1]
    say("block mass workload", wl.name)
    inp = make_workload(1)
    mass = sla.block_mass(dev(inp.q), dev(inp.k))
    torch.cuda.synchronize()
    Nb = -(-wl.N // 64)
    rows = sample_query_blocks(wl.B, wl.H, Nb, 2, 5, include=(0, Nb - 1))
    ref = quality.block_mass(inp.q, inp.k, 64, blocks=rows)
    got = mass.reshape(wl.B * wl.H, Nb, Nb).cpu().numpy().astype(np.float64)
    err = max(np.abs(got[bh, i] - ref[x]).max() for x, (bh, i) in enumerate(rows))
    say("  max|d| %.3g over %d rows" % (err, len(rows)))
    assert err <= 5e-5
    assert np.abs(got.sum(axis=-1) - 1.0).max() <= 1e-4
