"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: masks, critical lists and pooled means bit-exact; outputs for bf16
inputs within max|d| <= 1e-2 and relative L2 <= 5e-3 of the fp64 oracle, for
float32 inputs within 1e-5 (both).  Small cases and the Wan2.1 480p
workloads (with and without RoPE, every critical share) compare every
output row; the 720p and HunyuanVideo workloads (sparse and dense) compare
every mask row and a seeded sample of 64 query blocks per head (plus the
first and the ragged last block of each head).
"""
import math
import sys

import numpy as np
import pytest

from oracle import dense as odense
from oracle import oracle as orc
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


def dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def gpu_forward(sla, inp, rc, rn, out_dtype=None):
    q, k, v = dev(inp.q, inp.dtype), dev(inp.k, inp.dtype), dev(inp.v, inp.dtype)
    w = torch.from_numpy(inp.w).to("cuda")
    out, mask = sla.forward(q, k, v, w, rc, rn, out_dtype=out_dtype, return_mask=True)
    torch.cuda.synchronize()
    return out, mask


TOL = {"bf16": (1e-2, 5e-3), "f32": (1e-5, 1e-5)}


def gather_blocks(out_gpu, rows, N):
    """The query blocks `rows` ([n, 2] of (b*H + h, i)) of a [B,H,N,d] GPU
    output as fp64 numpy [n, 64, d], rows past N zero (as the oracle's)."""
    B, H, _, d = out_gpu.shape
    Nb = -(-N // 64)
    padded = torch.zeros((B * H, Nb * 64, d), dtype=torch.float32, device=out_gpu.device)
    padded[:, :N] = out_gpu.reshape(B * H, N, d).float()
    idx = torch.from_numpy(np.asarray(rows, np.int64)).to(out_gpu.device)
    g = padded.view(B * H, Nb, 64, d)[idx[:, 0], idx[:, 1]]
    del padded
    return g.cpu().numpy().astype(np.float64)


def check_blocks(got, ref, rows, dtype, extra_abs=None):
    """Element bound and relative L2 of got against ref ([n, 64, d] fp64)."""
    d = got - ref
    tol = TOL[dtype][0] if extra_abs is None else TOL[dtype][0] + extra_abs * np.abs(ref)
    bad = np.abs(d) > tol
    if bad.any():
        x, t, c = np.argwhere(bad)[0]
        raise AssertionError("block (bh=%d, i=%d) row %d channel %d: |d| %.3g (max over all %.3g)"
                             % (rows[x][0], rows[x][1], t, c, abs(d[x, t, c]), np.abs(d).max()))
    rel = np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= TOL[dtype][1], "relative L2 %.3g" % rel
    return float(np.abs(d).max()), float(rel)


def compare_rows(out_gpu, res, N, dtype, extra_abs=None):
    """out_gpu: [B,H,N,d] torch; res: oracle result with 'rows' and 'o'."""
    rows = res["rows"]
    return check_blocks(gather_blocks(out_gpu, rows, N), res["o"], rows, dtype, extra_abs)


# ------------------------------------------------------------------ stage checks


@pytest.mark.parametrize("dtype,d,N", [("bf16", 128, 1000), ("bf16", 64, 4096), ("f32", 64, 777), ("f32", 128, 200)])
def test_pool_bit_exact(sla, dtype, d, N):
    say("pool", dtype, d, N)
    inp = make_inputs(2, 3, (1, 1, N), d, dtype, seed=11)
    qp, kp = sla.pool(dev(inp.q, dtype), dev(inp.k, dtype))
    torch.cuda.synchronize()
    assert np.array_equal(qp.cpu().numpy(), orc.pool(inp.q))
    assert np.array_equal(kp.cpu().numpy(), orc.pool(inp.k))


@pytest.mark.parametrize("Nb,d,rc,rn", [(64, 64, 0.05, 0.10), (512, 128, 0.05, 0.10), (100, 128, 0.3, 0.3),
                                        (70, 64, 0.0, 0.5), (33, 128, 1.0, 0.0), (1857, 128, 0.05, 0.10),
                                        (2432, 64, 0.02, 0.01)])
def test_classify_bit_exact(sla, Nb, d, rc, rn):
    say("classify", Nb, d, rc, rn)
    rng = np.random.default_rng(Nb)
    qp = rng.standard_normal((1, 2, Nb, d)).astype(np.float32)
    kp = rng.standard_normal((1, 2, Nb, d)).astype(np.float32)
    ref = orc.classify(qp, kp, rc, rn, want_pc=True)
    got = sla.classify(dev(qp, "f32"), dev(kp, "f32"), rc, rn, want_excl=True, want_pc=True)
    torch.cuda.synchronize()
    assert (got["k_c"], got["k_n"]) == (ref["k_c"], ref["k_n"])
    assert np.array_equal(got["mask"].cpu().numpy(), ref["mask"])
    assert np.array_equal(got["crit"].cpu().numpy(), ref["crit"])
    excl = np.sort(np.concatenate([ref["crit"], ref["negl"]], axis=-1), axis=-1)
    assert np.array_equal(got["excl"].cpu().numpy(), excl)
    assert np.allclose(got["pc"].cpu().numpy(), ref["pc"], rtol=1e-5, atol=1e-9)


def test_classify_ties(sla):
    """Equal scores: the lower block index ranks higher at both ends."""
    say("classify ties")
    rng = np.random.default_rng(5)
    kp = rng.standard_normal((1, 1, 200, 64)).astype(np.float32)
    kp[0, 0, 100:150] = kp[0, 0, 10]          # 51 identical blocks
    qp = rng.standard_normal((1, 1, 200, 64)).astype(np.float32)
    qp[0, 0, :50] = 0.0                        # all-zero rows: every score ties at 0
    for rc, rn in [(0.05, 0.10), (0.2, 0.3), (0.5, 0.5)]:
        ref = orc.classify(qp, kp, rc, rn)
        got = sla.classify(dev(qp, "f32"), dev(kp, "f32"), rc, rn)
        torch.cuda.synchronize()
        assert np.array_equal(got["mask"].cpu().numpy(), ref["mask"])
        assert np.array_equal(got["crit"].cpu().numpy(), ref["crit"])


@pytest.mark.parametrize("Nb,d,dtype", [(150, 64, "f32"), (600, 128, "f32"), (1857, 128, "bf16"),
                                        (2432, 64, "bf16")])
def test_forward_labels_ties_and_near_ties(sla, Nb, d, dtype):
    """The forward pass ranks on float32 scores and settles the keys near
    each cut in fp64.  Its labels must equal the oracle's also on rows built
    against float32: exact ties of many blocks (200 copies of one key block,
    more than one wave's band), all-zero query blocks (every score 0), and
    near ties below float32 resolution (float inputs: copies of a key block
    with one element moved by one ulp), at several shares so that the groups
    straddle the cuts."""
    from sparse_attention_video_sla_amd.inputs import round_bf16
    say("forward labels with ties", Nb, d, dtype)
    N = 64 * Nb - 17
    rng = np.random.default_rng(Nb + d)
    H = 2
    q = rng.standard_normal((1, H, N, d)).astype(np.float32)
    k = rng.standard_normal((1, H, N, d)).astype(np.float32)
    v = rng.standard_normal((1, H, N, d)).astype(np.float32)
    # head 0: key blocks 100..299 (or as many as there are) copy block 10;
    # query blocks 0..20 are zero
    hi = min(300, Nb - 1)
    for j in range(100, hi):
        k[0, 0, 64 * j:64 * j + 64] = k[0, 0, 640:704]
    q[0, 0, :64 * 21] = 0.0
    # head 1: key blocks 40..79 copy block 7 with one element moved by j ulps
    for t, j in enumerate(range(40, 80)):
        blk = k[0, 1, 448:512].copy()
        blk[t % 64, t % d] = np.nextafter(blk[t % 64, t % d], np.float32(np.inf), dtype=np.float32)
        for _ in range(t % 3):
            blk[(t + 1) % 64, (t + 5) % d] = np.nextafter(blk[(t + 1) % 64, (t + 5) % d], np.float32(-np.inf),
                                                          dtype=np.float32)
        k[0, 1, 64 * j:64 * j + 64] = blk
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    w = (rng.standard_normal((d, d)) / np.sqrt(d)).astype(np.float32)
    qp, kp = orc.pool(q), orc.pool(k)
    qd, kd, vd = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    wd = torch.from_numpy(w).to("cuda")
    for rc, rn in [(0.02, 0.05), (0.05, 0.10), (0.13, 0.2), (0.3, 0.3), (0.5, 0.45)]:
        ref = orc.classify(qp, kp, rc, rn)
        _, mask = sla.forward(qd, kd, vd, wd, rc, rn, return_mask=True)
        torch.cuda.synchronize()
        got = mask.cpu().numpy()
        bad = np.argwhere((got != ref["mask"]).any(axis=-1))
        assert bad.size == 0, "rows with other labels (b, h, i): %s" % bad[:5].tolist()


# ------------------------------------------------------------------ forward, small


SMALL = [
    # B, H, N, d, dtype, rc, rn
    (1, 2, 1000, 128, "bf16", 0.05, 0.10),
    (1, 2, 4096, 128, "bf16", 0.25, 0.25),
    (2, 1, 2000, 64, "bf16", 0.10, 0.20),
    (1, 2, 777, 64, "f32", 0.2, 0.3),
    (1, 1, 4096, 128, "f32", 0.05, 0.10),
    (1, 3, 70, 128, "bf16", 0.5, 0.0),
    (1, 1, 5000, 128, "bf16", 0.0, 0.5),
    # odd Nb: the last pair of query blocks has no second block
    (1, 2, 3000, 128, "bf16", 0.1, 0.1),
    # last block of exactly 32 tokens: keys 32..63 of that tile are all past N
    (1, 1, 2080, 128, "bf16", 0.05, 0.1),
    (2, 2, 1100, 64, "bf16", 0.3, 0.2),
    (1, 1, 1050, 128, "bf16", 1.0, 0.0),
    # degenerate sizes: one token (Nb = 1, its only block critical), one
    # ragged block, a last block of one token, and linear attention over
    # three blocks, the last of one token
    (1, 2, 1, 128, "bf16", 0.05, 0.10),
    (1, 1, 37, 64, "f32", 0.05, 0.10),
    (1, 2, 65, 128, "bf16", 0.5, 0.5),
    (1, 1, 65, 64, "f32", 1.0, 0.0),
    (2, 1, 129, 64, "bf16", 0.0, 0.0),
]


@pytest.mark.parametrize("B,H,N,d,dtype,rc,rn", SMALL)
def test_forward_small(sla, B, H, N, d, dtype, rc, rn):
    say("forward", B, H, N, d, dtype, rc, rn)
    inp = make_inputs(B, H, (1, 1, N), d, dtype, seed=N + d)
    out, mask = gpu_forward(sla, inp, rc, rn)
    res = orc.forward(inp.q, inp.k, inp.v, inp.w, 64, rc, rn)
    assert np.array_equal(mask.cpu().numpy(), res["mask"])
    worst, rel = compare_rows(out, res, N, dtype)
    say("  max|d| %.3g rel %.3g" % (worst, rel))


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_forward_dense_mode(sla, dtype, d):
    """100% critical: dense softmax attention over the N valid tokens."""
    say("dense", dtype, d)
    N = 1000
    inp = make_inputs(1, 2, (1, 1, N), d, dtype, seed=7)
    out, mask = gpu_forward(sla, inp, 1.0, 0.0)
    res = orc.forward(inp.q, inp.k, inp.v, inp.w, 64, 1.0, 0.0)
    assert np.all(mask.cpu().numpy() == 1)
    compare_rows(out, res, N, dtype)


@pytest.mark.parametrize("dtype,d,N", [("bf16", 128, 1000), ("f32", 64, 4096), ("bf16", 64, 333)])
def test_forward_linear_mode(sla, dtype, d, N):
    """0% critical, 0% negligible: linear attention over all tokens, projected."""
    say("linear", dtype, d, N)
    inp = make_inputs(1, 2, (1, 1, N), d, dtype, seed=8)
    out, mask = gpu_forward(sla, inp, 0.0, 0.0)
    res = orc.forward(inp.q, inp.k, inp.v, inp.w, 64, 0.0, 0.0)
    assert np.all(mask.cpu().numpy() == 0)
    compare_rows(out, res, N, dtype)


def test_value_offset_reaches_linear_branch(sla):
    """V + v0 must move O by v0 + W v0 (the linear branch carries W v0)."""
    say("value offset")
    inp = make_inputs(1, 2, (4, 16, 16), 128, "bf16", seed=21)
    inp.v = (np.clip(np.round(inp.v * 8), -32, 32) / 8).astype(np.float32)   # V and V + v0 exact in bf16
    v0 = ((np.arange(128) % 16) - 8).astype(np.float32) / 4
    out0, _ = gpu_forward(sla, inp, 0.05, 0.10)
    inp.v = inp.v + v0
    out1, _ = gpu_forward(sla, inp, 0.05, 0.10)
    shift = v0.astype(np.float64) + inp.w.astype(np.float64) @ v0.astype(np.float64)
    d = (out1.double() - out0.double()).cpu().numpy() - shift
    assert np.abs(d).max() < 2e-2


def test_bf16_output(sla):
    say("bf16 out")
    N = 1500
    inp = make_inputs(1, 2, (1, 1, N), 128, "bf16", seed=3)
    out, _ = gpu_forward(sla, inp, 0.1, 0.1, out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16
    res = orc.forward(inp.q, inp.k, inp.v, inp.w, 64, 0.1, 0.1)
    compare_rows(out, res, N, "bf16", extra_abs=2.0 ** -8)


def test_deterministic(sla):
    say("determinism")
    inp = make_inputs(1, 4, (4, 20, 20), 128, "bf16", seed=4)
    a, ma = gpu_forward(sla, inp, 0.05, 0.10)
    b, mb = gpu_forward(sla, inp, 0.05, 0.10)
    assert torch.equal(a, b) and torch.equal(ma, mb)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_tail_reads_nothing_past_the_tensors(sla, dtype):
    """K and V end right before a region of NaNs.  The last head's ragged
    last block must read zeros (or nothing) past N: a NaN value of V would
    reach the output through 0 * NaN."""
    say("ragged tail", dtype)
    B, H, N, d, rc, rn = 1, 2, 1000, 128, 0.3, 0.1
    inp = make_inputs(B, H, (1, 1, N), d, dtype, seed=41)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    n = B * H * N * d
    guarded = []
    for x in (inp.k, inp.v):
        buf = torch.full((n + 64 * d * 4,), float("nan"), dtype=tdt, device="cuda")
        buf[:n].copy_(torch.from_numpy(np.ascontiguousarray(x)).reshape(-1).to(tdt))
        guarded.append(buf[:n].view(B, H, N, d))
    q = dev(inp.q, dtype)
    w = torch.from_numpy(inp.w).to("cuda")
    out = sla.forward(q, guarded[0], guarded[1], w, rc, rn)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    res = orc.forward(inp.q, inp.k, inp.v, inp.w, 64, rc, rn)
    compare_rows(out, res, N, dtype)


def test_stream_ordering(sla):
    """Every kernel of a call runs on the caller's stream: a call must see K
    and V written on that stream just before it (behind other queued work),
    and a second call that reuses the workspace must not overwrite the first
    call's states before they are used.  Nothing is synchronised between the
    steps below."""
    say("stream ordering")
    N, d, rc, rn = 3000, 128, 0.05, 0.10
    a = make_inputs(1, 2, (1, 1, N), d, "bf16", seed=31)
    b = make_inputs(1, 2, (1, 1, N), d, "bf16", seed=32)
    qa, ka, va = dev(a.q, "bf16"), dev(a.k, "bf16"), dev(a.v, "bf16")
    qb, kb, vb = dev(b.q, "bf16"), dev(b.k, "bf16"), dev(b.v, "bf16")
    wa, wb = torch.from_numpy(a.w).to("cuda"), torch.from_numpy(b.w).to("cuda")
    ws = torch.empty(sla.workspace_size(1, 2, N, d, "bf16", rc, rn), dtype=torch.uint8, device="cuda")
    busy = torch.randn(2048, 2048, device="cuda")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q, k, v = qa.clone(), ka.clone(), va.clone()
        out_a = sla.forward(q, k, v, wa, rc, rn, workspace=ws)
        for _ in range(8):                               # queue work ahead of the writes
            busy = torch.mm(busy, busy) * 1e-3
        q.copy_(qb)
        k.copy_(kb)
        v.copy_(vb)
        out_b = sla.forward(q, k, v, wb, rc, rn, workspace=ws)
    torch.cuda.synchronize()
    for inp, out in ((a, out_a), (b, out_b)):
        res = orc.forward(inp.q, inp.k, inp.v, inp.w, 64, rc, rn)
        worst, rel = compare_rows(out, res, N, "bf16")
        say("  max|d| %.3g rel %.3g" % (worst, rel))


def test_stage_timing(sla):
    """Stage timing records every stage of each call (pool, classify, block
    states, marginal-state GEMM, fused kernel)."""
    import ctypes
    say("stage timing")
    inp = make_inputs(1, 2, (1, 1, 3000), 128, "bf16", seed=5)
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    w = torch.from_numpy(inp.w).to("cuda")
    L = sla._lib.load()
    ms = (ctypes.c_float * 5)()
    calls = ctypes.c_int()
    L.sla_set_stage_timing(1)
    try:
        L.sla_stage_times(ms, ctypes.byref(calls))
        for _ in range(3):
            sla.forward(q, k, v, w, 0.05, 0.10)
        sla._lib.check(L.sla_stage_times(ms, ctypes.byref(calls)))
    finally:
        L.sla_set_stage_timing(0)
    assert calls.value == 3
    assert all(ms[i] > 0 for i in range(5)), list(ms)


# ------------------------------------------------------------------ named workloads, full size


def run_workload(sla, cid, per_head=None, fracs=None, sample_seed=77):
    """Every mask row against the oracle's classification; every output row
    (per_head None) or a seeded sample of per_head query blocks per head
    plus the first and the ragged last block."""
    wl = WORKLOADS[cid]
    say("workload", cid, wl.name)
    inp = make_workload(cid)
    N, Nb = wl.N, -(-wl.N // 64)
    qp, kp = orc.pool(inp.q), orc.pool(inp.k)
    for rc, rn in (fracs or wl.fracs):
        say("  fractions", rc, rn)
        cls = orc.classify(qp, kp, rc, rn)
        out, mask = gpu_forward(sla, inp, rc, rn)
        assert np.array_equal(mask.cpu().numpy(), cls["mask"]), "mask mismatch"
        del mask
        rows = None if per_head is None else sample_query_blocks(wl.B, wl.H, Nb, per_head, sample_seed,
                                                                 include=(0, Nb - 1))
        if rc >= 1.0 and rn == 0.0:
            # every block critical: dense attention, from the matrix-product oracle
            rows = rows if rows is not None else np.array([(bh, i) for bh in range(wl.B * wl.H)
                                                           for i in range(Nb)], np.int32)
            ref = odense.attention_rows(inp.q, inp.k, inp.v, rows)
        else:
            res = orc.forward(inp.q, inp.k, inp.v, inp.w, 64, rc, rn, rows=rows, cls=cls)
            rows, ref = res["rows"], res["o"]
            del res
        got = gather_blocks(out, rows, N)
        del out
        torch.cuda.empty_cache()
        worst, rel = check_blocks(got, ref, rows, wl.dtype)
        say("  max|d| %.3g rel %.3g over %d query blocks of %d" % (worst, rel, len(rows), wl.B * wl.H * Nb))
        del got, ref


@pytest.mark.timeout(600)
def test_workload0_tiny_all_rows(sla):
    run_workload(sla, 0)


@pytest.mark.timeout(600)
def test_workload1_wan480p_all_rows(sla):
    run_workload(sla, 1)


@pytest.mark.timeout(600)
def test_workload1_all_marginal_all_rows(sla):
    """The linear branch alone at the metric workload's size."""
    run_workload(sla, 1, fracs=[(0.0, 0.0)])


@pytest.mark.timeout(900)
def test_workload2_rope_cfg_pair_all_rows(sla):
    run_workload(sla, 2)


@pytest.mark.timeout(900)
def test_workload3_720p(sla):
    run_workload(sla, 3, per_head=64)


@pytest.mark.timeout(900)
def test_workload4_hunyuan(sla):
    run_workload(sla, 4, per_head=64, fracs=[(0.05, 0.10)])


@pytest.mark.timeout(900)
def test_workload4_dense(sla):
    run_workload(sla, 4, per_head=64, fracs=[(1.0, 0.0)])
