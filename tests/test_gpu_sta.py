"""GPU parity of sliding tile attention (sla_forward_sta) against the fp64
oracle (oracle/sta.py): the GPU takes tile-major tokens, the oracle raster
ones, and the test permutes between the two.  Bar of the forward pass in
bf16: max|d| <= 1e-2 and relative L2 <= 5e-3."""
import sys

import numpy as np
import pytest

from oracle import sta
from sparse_attention_video_sla_amd.inputs import make_inputs

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


def dev_tm(x, perm):
    return torch.from_numpy(np.ascontiguousarray(x[:, :, perm])).to("cuda").to(torch.bfloat16)


def check(got, ref):
    d = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    say("  max|d| %.3g rel %.3g" % (d.max(), rel))
    assert d.max() <= 1e-2 and rel <= 5e-3


CASES = [
    ((4, 8, 16), (2, 4, 8), (4, 8, 16), 128),      # one block per tile, neighbours on every axis
    ((4, 8, 16), (2, 4, 8), (2, 4, 8), 64),        # one tile: block-diagonal
    ((4, 8, 16), (2, 4, 8), (64, 64, 64), 128),    # every tile: dense
    ((6, 16, 16), (6, 8, 8), (18, 27, 24), 128),   # the page's window, 6 blocks per tile
    ((6, 16, 24), (2, 4, 8), (4, 8, 8), 64),       # even ratios: the tile and the next one
]


@pytest.mark.parametrize("grid,tile,window,d", CASES)
def test_forward_sta_all_rows(sla, grid, tile, window, d):
    say("sta", grid, tile, window, d)
    N = grid[0] * grid[1] * grid[2]
    inp = make_inputs(1, 2, grid, d, "bf16", seed=N + d)
    perm = sta.tile_order(grid, tile)
    out = sla.forward_sta(dev_tm(inp.q, perm), dev_tm(inp.k, perm), dev_tm(inp.v, perm), grid, tile, window)
    torch.cuda.synchronize()
    got = np.empty((1, 2, N, d))
    got[:, :, perm] = out.double().cpu().numpy()
    check(got, sta.attention_sta(inp.q, inp.k, inp.v, grid, tile, window))


def test_forward_sta_bf16_output(sla):
    grid, tile, window, d = (4, 8, 16), (2, 4, 8), (4, 8, 16), 128
    inp = make_inputs(1, 1, grid, d, "bf16", seed=5)
    perm = sta.tile_order(grid, tile)
    q, k, v = dev_tm(inp.q, perm), dev_tm(inp.k, perm), dev_tm(inp.v, perm)
    a = sla.forward_sta(q, k, v, grid, tile, window, out_dtype=torch.bfloat16)
    b = sla.forward_sta(q, k, v, grid, tile, window)
    torch.cuda.synchronize()
    assert (a.float() - b).abs().max().item() <= 2.0 ** -8 * b.abs().max().item() + 1e-6


@pytest.mark.timeout(600)
def test_sta_workload_sampled(sla):
    """HunyuanVideo-sized latent 30 x 48 x 80, tiles (6, 8, 8), window
    (18, 27, 24), two heads: sampled tokens (corners, tile edges, random)
    against the oracle."""
    grid, tile, window, d = (30, 48, 80), (6, 8, 8), (18, 27, 24), 128
    N = grid[0] * grid[1] * grid[2]
    say("sta workload", grid)
    inp = make_inputs(1, 2, grid, d, "bf16", seed=3001)
    perm = sla.sta_tile_order(grid, tile)
    out = sla.forward_sta(dev_tm(inp.q, perm), dev_tm(inp.k, perm), dev_tm(inp.v, perm), grid, tile, window)
    torch.cuda.synchronize()
    inv = np.empty(N, np.int64)
    inv[perm] = np.arange(N)
    rng = np.random.default_rng(7)
    toks = [0, N - 1, 5 * 48 * 80 + 7 * 80 + 8, 6 * 48 * 80 + 8 * 80 + 7] + list(rng.choice(N, 20, replace=False))
    rows = [(bh, int(n)) for bh in range(2) for n in toks]
    ref = sta.attention_sta(inp.q, inp.k, inp.v, grid, tile, window, rows=rows)
    o = out.reshape(2, N, d)
    got = np.stack([o[bh, int(inv[n])].double().cpu().numpy() for bh, n in rows])
    check(got, ref)
    assert torch.isfinite(out).all()
