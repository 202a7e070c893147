#!/usr/bin/env python3
"""Benchmark of the SLA sparse-linear attention forward on one MI355X.

A step is one sla_forward call (pool -> classify -> linear states ->
marginal-state GEMM -> fused sparse+linear kernel) over one of the named
synthetic workloads, inputs resident in HBM.  The default is the Wan2.1-1.3B
480p shape: B=1, H=12, N=32760 (21x30x52 latent grid), d=128, bf16, 5%
critical / 10% negligible.  --workload picks another (0 tiny fp32, 2 the
same grid with RoPE and a batch of two, 3 720p, 4 HunyuanVideo), --crit /
--negl override the shares, --all prints one line for every workload and
setting: 0, 1, 2 at 2.5/5/10 % critical, 3, 4 and 4 at 100 % critical (dense
attention in the same kernels).

Printed: one JSON line per setting.  `value` is effective TFLOP/s over the
whole call, counting the method's work F = 4*64*64*d per critical block pair
+ 4*64*d*d per query block with marginal blocks, and `ms_per_step` the mean
of the K timed steps.  Before the W warm-up steps, untimed calls run for
about 0.2 s, so that the GPU clock has ramped up from idle.  `timing` gives the median, p10 and p90 of 100 calls
timed one by one with HIP events on the call's stream, with the 256 MB
last-level cache (MALL) warm and flushed before each call (a 512 MB fill),
and the GPU clock sampled through amdsmi while calls run back to back.  `roofline`
is for the fused kernel, timed with HIP events recorded on its stream; its
algorithmic flops are the critical pairs plus 2*64*d*d per query block
(phi(Q) times the marginal state; the projection is folded into the state
kernel).  `roofline.traffic` is the kernel's HBM bytes per launch from a
committed rocprofv3 counter summary for the same workload, reported only
while the kernel source and the package headers it includes match the ones
the counters were taken with.  `cpu_baseline` times the CPU oracle on a
bounded sample of the same inputs.

With --lvsa it prints instead one JSON line for LVSA frame-level sparse
attention (the LVSA page's sets A(t) = G_s U W(t)) on a long-video workload:
Wan2.1-1.3B at 6x its training length, 121 latent frames of 30x52 tokens
(N = 188760), H=12, d=128, budget C = 21 frames, W = 3, step 0.  A step is
one sla_forward_lvsa call (frame sets, block schedule, attention); `value`
counts 4*d flops per (query token, key token) pair the sets allow.

With --sta it prints instead one JSON line for sliding tile attention (the
VORTA page's STA: a 3D window kept by whole tiles) on a HunyuanVideo-sized
latent: 30x48x80 tokens (N = 115200, tile-major), tiles (6, 8, 8), window
(18, 27, 24), H=24, d=128; `value` counts 4*d flops per kept (query, key)
pair.

With --backward it prints instead one JSON line for the SLA backward pass
on the same Wan2.1 480p workload: `value` and `ms_per_step` are those of
sla_backward_saved (dQ, dK, dV, dW from the state sla_forward_save left, as
a training step runs it), counting 10*64*64*d per critical pair (five
products), 6*64*d*d per query block and 10*64*d*d per key block of the
linear branch, and (d*d + d) per marginal pair (the transposed sums);
`recompute` gives sla_backward (the forward run again inside, its F counted
too) and `training_step_ms` sla_forward_save + sla_backward_saved.  Its
`roofline` is for the slowest stage; `traffic` is filled from the
backward's counter summary when that stage is one kernel (dQ, dK/dV or the
linear keys).

With --quality it prints instead one JSON line for the mask-quality
diagnostics (sla_block_mass + sla_mask_stats) on the same workload: the
exact block attention mass kept by the critical, marginal and negligible
blocks, the 95 % block density, the relative error against dense attention
(the same fused kernel at 100 % critical) of sparse-only attention as the
skipped share grows and of sparse + linear attention (projection = identity:
W is learned in the article), and the block-mass kernel's rate against the
bf16 MFMA roofline, with the fp64 oracle timed on a sample of rows.
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s + ms/call of sparse-linear attn fwd at N=32760, %MFMA peak"
CSRC = os.path.join(ROOT, "sparse_attention_video_sla_amd", "csrc")
# backward stages that are one kernel each (the others span several)
BWD_STAGE_KERNEL = {"dq": "bwd_dq_kernel", "dkv": "bwd_dkv_kernel", "linear_keys": "bwd_lin_key_kernel"}
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0


def work(B, H, N, d, kc, kn):
    Nb = -(-N // 64)
    pairs = B * H * Nb * kc
    marg_rows = B * H * Nb if kc + kn < Nb else 0
    f_comp = 4 * 64 * 64 * d * pairs + 4 * 64 * d * d * marg_rows
    f_fused = 4 * 64 * 64 * d * pairs + 2 * 64 * d * d * marg_rows
    return f_comp, f_fused, pairs, marg_rows


def profile_traffic(kernel, workload, source):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 summaries (a line `traffic: kernel=K workload=W
    bytes_per_launch=B source=F sha256=H`: FETCH_SIZE + WRITE_SIZE scaled by
    the copy-kernel calibration), or None when no summary covers them or the
    kernel source has changed since the counters were taken."""
    import glob
    import re
    try:
        sha = source_sha(source)
    except OSError:
        return None
    pat = re.compile(r"traffic: kernel=(\S+) workload=(\S+) bytes_per_launch=(\d+) source=(\S+) sha256=([0-9a-f]{16})")
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for m in pat.finditer(open(path).read()):
            if m.group(1) == kernel and m.group(2) == workload and m.group(4) == source and m.group(5) == sha:
                return int(m.group(3))
    return None


def source_sha(source):
    """First 16 hex digits of the sha256 over a kernel source and, depth
    first, every header of the package it includes with quotes (each once),
    so that a change to a shared header also voids stored counters."""
    import hashlib
    import re
    h, seen = hashlib.sha256(), set()

    def add(name):
        if name in seen:
            return
        seen.add(name)
        path = os.path.join(CSRC, name)
        if not os.path.exists(path):
            path = os.path.join(ROOT, "include", name)
        src = open(path, "rb").read()
        h.update(src)
        for inc in re.findall(rb'^#include "([^"]+)"', src, re.M):
            add(inc.decode())
    add(source)
    return h.hexdigest()[:16]


def block_flops(d, kc, linear):
    """The method's F for one query block of one head (as work() counts it)."""
    return 4 * 64 * 64 * d * kc + (4 * 64 * d * d if linear else 0)


def cpu_baseline(inp, wl, rc, rn, per_head=None, seed=5):
    """The C oracle (as it stands) on the same inputs: every query block of
    every head (per_head None), or a seeded sample of per_head query blocks
    per head; F counted for the blocks evaluated."""
    import numpy as np
    from oracle import oracle as orc
    from sparse_attention_video_sla_amd.inputs import sample_query_blocks
    B, H, N, d = inp.q.shape
    Nb = -(-N // 64)
    t0 = time.perf_counter()
    qp, kp = orc.pool(inp.q), orc.pool(inp.k)
    cls = orc.classify(qp, kp, rc, rn)
    rows = None if per_head is None else sample_query_blocks(B, H, Nb, per_head, seed)
    res = orc.forward(inp.q, inp.k, inp.v, inp.w, 64, rc, rn, rows=rows, cls=cls)
    t = time.perf_counter() - t0
    n_rows = len(res["rows"])
    kc, kn = res["k_c"], res["k_n"]
    f = n_rows * block_flops(d, kc, kc + kn < Nb)
    total_rows = B * H * Nb
    if per_head is None:
        sample = "every query block of all %d heads: pool, classify, sparse and linear branches in fp64" % (B * H)
    else:
        sample = ("%d query blocks (%d per head, seeded) of %d, after pool and classify of every row; "
                  "sparse and linear branches in fp64" % (n_rows, per_head, total_rows))
    return {"value": round(f / t / 1e12, 6), "unit": "TFLOP/s", "cores": orc.threads(), "kind": "oracle",
            "seconds": round(t, 3), "sample": sample,
            "ms_per_call_extrapolated": round(t * 1e3 * total_rows / n_rows, 1)}


def run_quality(args, wl):
    import torch
    import sparse_attention_video_sla_amd as sla
    from sparse_attention_video_sla_amd.inputs import make_workload

    rc = args.crit if args.crit is not None else wl.fracs[0][0]
    rn = args.negl if args.negl is not None else wl.fracs[0][1]
    inp = make_workload(args.workload)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (inp.q, inp.k, inp.v))
    B, H, N, d = q.shape
    Nb = -(-N // 64)
    eye = torch.eye(d, dtype=torch.float32, device=dev)

    for _ in range(args.warmup):
        sla.block_mass(q, k)
    st = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(args.steps):
        mass = sla.block_mass(q, k)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    flops = 2 * 2.0 * B * H * N * N * d          # two passes of Q K^T
    tflops = flops / (ms * 1e-3) / 1e12

    _, mask = sla.forward(q, k, v, eye, rc, rn, return_mask=True)
    stats = sla.mask_stats(mass, mask)
    mean = stats.reshape(-1, 4).double().mean(dim=0).tolist()

    def rel(a, b):
        return float(torch.linalg.vector_norm((a - b).double()) / torch.linalg.vector_norm(b.double()))

    dense = sla.forward(q, k, v, eye, 1.0, 0.0)
    sweep = []
    for skip in (0.45, 0.70, 0.85, 0.92, 0.95):
        so = sla.forward(q, k, v, eye, 1.0 - skip, skip)         # critical = the rest, nothing linear
        sweep.append({"skipped_share": skip, "rel_err_sparse_only": round(rel(so, dense), 5)})
    sl = sla.forward(q, k, v, eye, rc, rn)
    so = sla.forward(q, k, v, eye, rc, 1.0 - rc)
    torch.cuda.synchronize()

    line = {
        "metric": "exact block attention mass (mask-quality diagnostics): TFLOP/s of the block-mass kernel",
        "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "dtype": "bf16", "data": "synthetic (seeded)",
        "config": {"workload": wl.name, "B": B, "H": H, "N": N, "d": d, "block": 64, "crit_frac": rc, "negl_frac": rn},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "kernel": "block_mass16_kernel<128>",
                     "flops_per_launch": flops},
        "quality": {"critical_mass": round(mean[0], 5), "marginal_mass": round(mean[1], 5),
                    "negligible_mass": round(mean[2], 5), "density95": round(mean[3], 5),
                    "rel_err_sparse_linear_identity_w": round(rel(sl, dense), 5),
                    "rel_err_sparse_only_same_critical": round(rel(so, dense), 5),
                    "skip_sweep": sweep},
    }
    if not args.no_cpu:
        from oracle import quality as oq
        from sparse_attention_video_sla_amd.inputs import sample_query_blocks
        rows = sample_query_blocks(B, H, Nb, max(1, args.cpu_heads or 4), 11)
        t0 = time.perf_counter()
        ref = oq.block_mass(inp.q, inp.k, 64, blocks=rows)
        t = time.perf_counter() - t0
        got = mass.reshape(B * H, Nb, Nb).cpu().numpy()
        err = max(float(abs(got[bh, i] - ref[x]).max()) for x, (bh, i) in enumerate(rows))
        f_rows = len(rows) * 64 * 2.0 * N * d
        line["cpu_baseline"] = {"value": round(f_rows / t / 1e12, 6), "unit": "TFLOP/s", "cores": os.cpu_count(),
                                "kind": "oracle", "seconds": round(t, 3),
                                "sample": "%d query blocks (fp64, one pass of Q K^T each)" % len(rows),
                                "max_abs_diff_vs_gpu": err}
    print(json.dumps(line), flush=True)


def run_lvsa(args):
    import numpy as np
    import torch
    import sparse_attention_video_sla_amd as sla
    from sparse_attention_video_sla_amd import _lib
    from sparse_attention_video_sla_amd.inputs import LVSA_WORKLOADS, make_lvsa_workload

    wl = LVSA_WORKLOADS["wan6x"]
    inp = make_lvsa_workload("wan6x")
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (inp.q, inp.k, inp.v))
    B, H, N, d = q.shape
    T, P = wl.T, wl.P
    out = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    ws = torch.empty(sla.lvsa_workspace_size(B, H, N, T, wl.C, wl.W), dtype=torch.uint8, device=dev)
    t_per, n_glob, per_set = sla.lvsa_plan(T, wl.C, wl.W)

    def step():
        sla.forward_lvsa(q, k, v, T, wl.C, wl.W, wl.step, out=out, workspace=ws)

    prewarm(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    L = _lib.load()
    L.sla_set_stage_timing(1)
    ms_buf = (ctypes.c_float * 5)()
    calls = ctypes.c_int()
    L.sla_stage_times(ms_buf, ctypes.byref(calls))
    for _ in range(args.steps):
        step()
    _lib.check(L.sla_stage_times(ms_buf, ctypes.byref(calls)))
    L.sla_set_stage_timing(0)
    stage_ms = {name: ms_buf[i] / max(calls.value, 1) for i, name in enumerate(_lib.STAGES)}

    sets, cnt = sla.lvsa_sets(T, wl.C, wl.W, wl.step)
    frames_seen = int(cnt.sum().item())                  # sum over query frames of |A(t)|
    pairs = frames_seen * P * P                          # (query token, key token) pairs per head
    flops = 4.0 * d * pairs * B * H
    ms = (t1 - t0) * 1e3 / args.steps
    value = flops / (ms * 1e-3) / 1e12
    t_fused = stage_ms["fused"] * 1e-3
    achieved = flops / t_fused / 1e12 if t_fused > 0 else 0.0
    dense = 4.0 * d * N * N * B * H
    line = {
        "metric": "effective TFLOP/s + ms/call of LVSA frame-level sparse attention fwd, Wan2.1-1.3B 6x length, %MFMA peak",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded; local sinusoid Q/K + noise, V ~ N(0,1))",
        "config": {"workload": wl.name, "B": B, "H": H, "N": N, "d": d, "block": 64, "T": T, "P": P, "C": wl.C,
                   "W": wl.W, "step": wl.step, "T_per": t_per, "globals": n_glob, "frames_per_set": per_set,
                   "density_vs_dense": round(flops / dense, 5), "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": profile_traffic("fused16s_kernel", wl.name, "fused16s.hip"),
                     "kernel": "fused16s_kernel<bf16,f16,128,f16,slots,frame marks>, 4 shares per row pair, fp16 partial outputs (merged apart)",
                     "flops_per_launch": flops,
                     "avg_launch_ms": round(stage_ms["fused"], 4)},
        "stages": {"schedule": {"ms": round(stage_ms["classify"], 4)}, "fused": {"ms": round(stage_ms["fused"], 4)},
                   "merge": {"ms": round(stage_ms["assemble"], 4)}},
    }
    if not args.no_cpu:
        from oracle import lvsa as olv
        from sparse_attention_video_sla_amd.inputs import sample_query_blocks
        Nb = -(-N // 64)
        rows = sample_query_blocks(B, H, Nb, max(1, args.cpu_heads or 24), 13)
        t0 = time.perf_counter()
        ref = olv.attention_lvsa(inp.q, inp.k, inp.v, T, P, wl.C, wl.W, wl.step,
                                 rows=[tuple(int(x) for x in r) for r in rows])
        t = time.perf_counter() - t0
        o = out.reshape(B * H, N, d)
        err = 0.0
        for x, (bh, i) in enumerate(rows):
            r1 = min(N, 64 * (i + 1))
            err = max(err, float(np.abs(o[bh, 64 * i:r1].double().cpu().numpy() - ref[x, :r1 - 64 * i]).max()))
        f_rows = 4.0 * d * 64 * per_set * P * len(rows)
        line["cpu_baseline"] = {"value": round(f_rows / t / 1e12, 6), "unit": "TFLOP/s", "cores": os.cpu_count(),
                                "kind": "oracle", "seconds": round(t, 3),
                                "sample": "%d query blocks of 64 tokens (fp64), each against the %d frames of its set"
                                          % (len(rows), per_set),
                                "max_abs_diff_vs_gpu": err}
    print(json.dumps(line), flush=True)


STA_WORKLOAD = {"name": "hunyuanvideo-30x48x80-sta", "B": 1, "H": 24, "grid": (30, 48, 80), "d": 128,
                "tile": (6, 8, 8), "window": (18, 27, 24), "seed": 3001}


def sta_pairs(grid, tile, window):
    """(query, key) pairs the tile window keeps, per head: a product over the
    axes of the pairs (i, j) whose tile centres differ by 2*delta*t in (-W, W]."""
    total = 1
    for n, t, w in zip(grid, tile, window):
        c = 0
        for a in range(n // t):
            for b in range(n // t):
                if -w < 2 * (b - a) * t <= w:
                    c += t * t
        total *= c
    return total


def run_sta(args):
    import numpy as np
    import torch
    import sparse_attention_video_sla_amd as sla
    from sparse_attention_video_sla_amd import _lib
    from sparse_attention_video_sla_amd.inputs import make_inputs

    wl = STA_WORKLOAD
    grid, tile, window, d = wl["grid"], wl["tile"], wl["window"], wl["d"]
    B, H = wl["B"], wl["H"]
    N = grid[0] * grid[1] * grid[2]
    inp = make_inputs(B, H, grid, d, "bf16", seed=wl["seed"])
    perm = sla.sta_tile_order(grid, tile)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x[:, :, perm])).to(dev).to(torch.bfloat16)
               for x in (inp.q, inp.k, inp.v))
    out = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    ws = torch.empty(sla.sta_workspace_size(B, H, grid, tile, window), dtype=torch.uint8, device=dev)

    def step():
        sla.forward_sta(q, k, v, grid, tile, window, out=out, workspace=ws)

    prewarm(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    L = _lib.load()
    L.sla_set_stage_timing(1)
    ms_buf = (ctypes.c_float * 5)()
    calls = ctypes.c_int()
    L.sla_stage_times(ms_buf, ctypes.byref(calls))
    for _ in range(args.steps):
        step()
    _lib.check(L.sla_stage_times(ms_buf, ctypes.byref(calls)))
    L.sla_set_stage_timing(0)
    stage_ms = {name: ms_buf[i] / max(calls.value, 1) for i, name in enumerate(_lib.STAGES)}

    pairs = sta_pairs(grid, tile, window)
    flops = 4.0 * d * pairs * B * H
    ms = (t1 - t0) * 1e3 / args.steps
    value = flops / (ms * 1e-3) / 1e12
    t_fused = stage_ms["fused"] * 1e-3
    achieved = flops / t_fused / 1e12 if t_fused > 0 else 0.0
    line = {
        "metric": "effective TFLOP/s + ms/call of sliding tile attention fwd, HunyuanVideo-sized latent, %MFMA peak",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded; local sinusoid Q/K + noise, V ~ N(0,1)), tile-major tokens",
        "config": {"workload": wl["name"], "B": B, "H": H, "N": N, "d": d, "block": 64, "grid": list(grid),
                   "tile": list(tile), "window": list(window), "density_vs_dense": round(pairs / N / N, 5),
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": profile_traffic("fused16s_kernel", wl["name"], "fused16s.hip"),
                     "kernel": "fused16s_kernel<bf16,f16,128,float,slots> (tile schedule)", "flops_per_launch": flops,
                     "avg_launch_ms": round(stage_ms["fused"], 4)},
        "stages": {"schedule": {"ms": round(stage_ms["classify"], 4)}, "fused": {"ms": round(stage_ms["fused"], 4)},
                   "merge": {"ms": round(stage_ms["assemble"], 4)}},
    }
    if not args.no_cpu:
        from oracle import sta as osta
        inv = np.empty(N, np.int64)
        inv[perm] = np.arange(N)
        rng = np.random.default_rng(17)
        per_head = max(1, args.cpu_heads or 200)
        rows = [(bh, int(n)) for bh in range(B * H) for n in rng.choice(N, per_head, replace=False)]
        t0 = time.perf_counter()
        ref = osta.attention_sta(inp.q, inp.k, inp.v, grid, tile, window, rows=rows)
        t = time.perf_counter() - t0
        o = out.reshape(B * H, N, d)
        got = np.stack([o[bh, int(inv[n])].double().cpu().numpy() for bh, n in rows])
        keys = pairs / N
        f_rows = 4.0 * d * keys * len(rows)
        line["cpu_baseline"] = {"value": round(f_rows / t / 1e12, 6), "unit": "TFLOP/s", "cores": os.cpu_count(),
                                "kind": "oracle", "seconds": round(t, 3),
                                "sample": "%d query tokens (fp64), each against its kept keys" % len(rows),
                                "max_abs_diff_vs_gpu": float(np.abs(got - ref).max())}
    print(json.dumps(line), flush=True)


BWD_STAGES = ("forward", "dq", "dkv", "linear_rows", "linear_keys")


def run_backward(args, wl):
    import numpy as np
    import torch
    import sparse_attention_video_sla_amd as sla
    from sparse_attention_video_sla_amd import _lib
    from sparse_attention_video_sla_amd.inputs import make_workload, round_bf16

    rc = args.crit if args.crit is not None else wl.fracs[0][0]
    rn = args.negl if args.negl is not None else wl.fracs[0][1]
    inp = make_workload(args.workload)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (inp.q, inp.k, inp.v))
    w = torch.from_numpy(inp.w).to(dev)
    rng = np.random.default_rng(wl.seed + 7)
    dout_h = round_bf16(rng.standard_normal(inp.q.shape).astype(np.float32))
    dout = torch.from_numpy(dout_h).to(dev).to(torch.bfloat16)
    B, H, N, d = q.shape
    Nb = -(-N // 64)
    kc, kn = sla.counts(Nb, rc, rn)
    ws = torch.empty(sla.backward_workspace_size(B, H, N, d, rc, rn), dtype=torch.uint8, device=dev)
    _, saved = sla.forward_save(q, k, v, w, rc, rn)
    saved_ws = torch.empty_like(ws)

    def recompute():
        sla.backward(q, k, v, w, dout, rc, rn, workspace=ws)

    def step():
        sla.backward_saved(saved, q, k, v, w, dout)

    def train_step():
        sla.forward_save(q, k, v, w, rc, rn, saved=saved_train)
        sla.backward_saved(saved_train, q, k, v, w, dout)

    saved_train = sla.SavedForward(saved_ws, q.shape, rc, rn, 64)

    def timed(fn):
        prewarm(fn)
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    ms = timed(step)
    ms_recompute = timed(recompute)
    ms_train = timed(train_step)
    L = _lib.load()
    L.sla_set_stage_timing(1)
    ms_buf = (ctypes.c_float * 5)()
    calls = ctypes.c_int()
    L.sla_stage_times(ms_buf, ctypes.byref(calls))
    for _ in range(args.steps):
        recompute()
    _lib.check(L.sla_stage_times(ms_buf, ctypes.byref(calls)))
    L.sla_set_stage_timing(0)
    st_ms = {name: ms_buf[i] / max(calls.value, 1) for i, name in enumerate(BWD_STAGES)}

    f_fwd, _, pairs, marg_rows = work(B, H, N, d, kc, kn)
    lin = kc + kn < Nb
    marg_pairs = B * H * Nb * (Nb - kc - kn) if lin else 0
    f_sparse = 10.0 * 64 * 64 * d * pairs
    f_rows = 6.0 * 64 * d * d * marg_rows
    f_keys = 10.0 * 64 * d * d * B * H * Nb if lin else 0.0
    f_sums = float(marg_pairs) * (d * d + d)
    grads = f_sparse + f_rows + f_keys + f_sums
    value = grads / (ms * 1e-3) / 1e12
    per_stage = {
        "forward": (f_fwd, "mfma"), "dq": (6.0 * 64 * 64 * d * pairs, "mfma"), "dkv": (8.0 * 64 * 64 * d * pairs, "mfma"),
        "linear_rows": (f_rows + f_sums, "mfma"), "linear_keys": (f_keys, "mfma")}
    stages = {}
    for name in BWD_STAGES:
        fl, bound = per_stage[name]
        stages[name] = {"ms": round(st_ms[name], 4),
                        "TFLOP/s": round(fl / max(st_ms[name], 1e-9) / 1e9, 1), "bound": bound}
    dom = max((n for n in BWD_STAGES if n != "forward"), key=lambda n: st_ms[n])   # the saved path's stages
    fl, bound = per_stage[dom]
    peak = PEAK_BF16_TFLOPS
    achieved = fl / max(st_ms[dom], 1e-9) / 1e9
    line = {
        "metric": "effective TFLOP/s + ms/call of the SLA backward (dQ, dK, dV, dW from the saved forward state) "
                  "at N=32760",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded; local sinusoid Q/K + noise, V ~ N(0,1); dO ~ N(0,1))",
        "config": {"workload": wl.name, "B": B, "H": H, "N": N, "d": d, "block": 64, "crit_frac": rc,
                   "negl_frac": rn, "k_c": kc, "k_n": kn, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": (profile_traffic(BWD_STAGE_KERNEL[dom], wl.name, "backward.hip")
                                 if dom in BWD_STAGE_KERNEL else None),
                     "kernel": "backward stage " + dom,
                     "flops_per_launch": fl, "avg_launch_ms": round(st_ms[dom], 4)},
        "stages": stages,
        "stages_of": "sla_backward (stage forward: the forward run again inside)",
        "recompute": {"ms": round(ms_recompute, 4),
                      "TFLOP/s": round((f_fwd + grads) / (ms_recompute * 1e-3) / 1e12, 3),
                      "what": "sla_backward: the forward run again inside, then the same gradient kernels"},
        "training_step_ms": round(ms_train, 4),
    }
    if not args.no_cpu:
        from oracle import backward as ob
        from oracle import oracle as orc
        n_tok, heads = 8192, 2
        sub = make_workload(args.workload, n_tokens=n_tok)
        sq, sk, sv = (x[:, :heads] for x in (sub.q, sub.k, sub.v))
        sd = dout_h[:, :heads, :n_tok]
        t0 = time.perf_counter()
        mask = orc.classify(orc.pool(sq), orc.pool(sk), rc, rn)["mask"]
        ob.gradients(sq, sk, sv, sub.w, mask, sd)
        t = time.perf_counter() - t0
        nb = -(-n_tok // 64)
        kcs, kns = sla.counts(nb, rc, rn)
        ff, _, pp, mr = work(1, heads, n_tok, d, kcs, kns)
        fs = ff + 10.0 * 64 * 64 * d * pp + 6.0 * 64 * d * d * mr + 10.0 * 64 * d * d * heads * nb + \
            float(heads * nb * (nb - kcs - kns)) * (d * d + d)
        line["cpu_baseline"] = {"value": round(fs / t / 1e12, 6), "unit": "TFLOP/s", "cores": os.cpu_count(),
                                "kind": "oracle", "seconds": round(t, 3),
                                "sample": "the first %d tokens of heads 0-%d (the token-level oracle is quadratic in N): "
                                          "labels, then autograd of the fp64 forward; F counts the forward's and the gradients' "
                                          "flops, both of which the oracle computes"
                                          % (n_tok, heads - 1)}
    print(json.dumps(line), flush=True)


# fused kernel per input dtype: name, source, peak of its matrix-core type
FUSED_KERNEL = {"bf16": ("fused16s_kernel", "fused16s.hip", PEAK_BF16_TFLOPS, "bf16"),
                "f32": ("fused_kernel", "fused.hip", PEAK_FP32_TFLOPS, "fp32")}


def clock_sampler():
    """A background sampler of the GPU's current graphics clock (MHz)
    through amdsmi, or None where amdsmi is missing."""
    import threading
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception:
        return None
    samples, stop = [], threading.Event()

    def read():
        # the mean over the eight XCDs where the metrics table has them
        try:
            clks = amdsmi.amdsmi_get_gpu_metrics_info(handle)["current_gfxclks"]
            clks = [float(c) for c in clks if isinstance(c, (int, float)) and 0 < c < 65535]
            if clks:
                return sum(clks) / len(clks)
        except Exception:
            pass
        try:
            return float(amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX)["clk"])
        except Exception:
            return None

    def run():
        while not stop.is_set():
            c = read()
            if c is not None:
                samples.append(c)
            stop.wait(0.02)
    th = threading.Thread(target=run, daemon=True)
    th.start()

    def finish():
        stop.set()
        th.join()
        return samples
    return finish


def busy_clock(step, call_ms, seconds=0.8):
    """The graphics clock (MHz) sampled while the GPU runs `step` back to
    back for about `seconds`; calls are enqueued in batches of about 50 ms
    of GPU work between synchronisations, so that short calls do not leave
    the GPU idle (and clocked down) while the host waits; the first fifth
    of the samples (the clock ramping up) is dropped."""
    import torch
    finish = clock_sampler()
    if finish is None:
        return []
    batch = max(4, int(math.ceil(50.0 / max(call_ms, 1e-3))))
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(batch):
            step()
        torch.cuda.synchronize()
    samples = finish()
    return samples[len(samples) // 5:]


def prewarm(step, seconds=0.2, cap=2000):
    """Untimed calls for about `seconds` before the warm-up steps: the GPU's
    clock takes several milliseconds of load to ramp up from idle, which a
    few warm-up steps of a sub-millisecond call do not cover."""
    import torch
    t0, n = time.perf_counter(), 0
    while n < cap and time.perf_counter() - t0 < seconds:
        for _ in range(8):
            step()
        n += 8
        torch.cuda.synchronize()


def per_call_ms(step, n, flush=None):
    """n calls timed one by one with HIP events on torch's current stream
    (the stream the library enqueues on); with `flush` a fill kernel runs
    before each call, outside its events."""
    import torch
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        if flush is not None:
            flush.zero_()
        a.record(st)
        step()
        b.record(st)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def spread(ms):
    import numpy as np
    x = np.asarray(ms)
    return {"median": round(float(np.median(x)), 4), "p10": round(float(np.percentile(x, 10)), 4),
            "p90": round(float(np.percentile(x, 90)), 4)}


def run_forward(args, cid, rc, rn, flush, cpu=True):
    """One JSON line for workload cid at shares (rc, rn)."""
    import torch
    import sparse_attention_video_sla_amd as sla
    from sparse_attention_video_sla_amd import _lib
    from sparse_attention_video_sla_amd.inputs import WORKLOADS, make_workload

    wl = WORKLOADS[cid]
    inp = make_workload(cid)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x).to(dev).to(tdt) for x in (inp.q, inp.k, inp.v))
    w = torch.from_numpy(inp.w).to(dev)
    B, H, N, d = q.shape
    Nb = -(-N // 64)
    kc, kn = sla.counts(Nb, rc, rn)
    out = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    ws = torch.empty(sla.workspace_size(B, H, N, d, wl.dtype, rc, rn), dtype=torch.uint8, device=dev)

    def step():
        sla.forward(q, k, v, w, rc, rn, out=out, workspace=ws)

    prewarm(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    warm = per_call_ms(step, args.calls)
    flushed = per_call_ms(step, args.calls, flush)
    clocks = busy_clock(step, sorted(warm)[len(warm) // 2])
    # per-stage times (HIP events around each kernel, on the stream it runs
    # on) in a separate pass, so that the event records stay out of the
    # timed steps
    L = _lib.load()
    L.sla_set_stage_timing(1)
    ms_buf = (ctypes.c_float * 5)()
    calls = ctypes.c_int()
    L.sla_stage_times(ms_buf, ctypes.byref(calls))          # drop anything recorded before
    for _ in range(args.steps):
        step()
    _lib.check(L.sla_stage_times(ms_buf, ctypes.byref(calls)))
    L.sla_set_stage_timing(0)
    stage_ms = {name: ms_buf[i] / max(calls.value, 1) for i, name in enumerate(_lib.STAGES)}

    ms = (t1 - t0) * 1e3 / args.steps
    f_comp, f_fused, pairs, marg_rows = work(B, H, N, d, kc, kn)
    value = f_comp / (ms * 1e-3) / 1e12
    kname, ksrc, peak, mfma_type = FUSED_KERNEL[wl.dtype]
    t_fused = stage_ms["fused"] * 1e-3
    achieved = f_fused / t_fused / 1e12 if t_fused > 0 else 0.0
    Lp = -(-(d * d + d) // 256) * 256
    Nbc = -(-Nb // 64) * 64
    es = 2 if wl.dtype == "bf16" else 4
    nbytes = {   # algorithmic bytes per launch
        "pool": 2 * B * H * N * d * es + 2 * B * H * Nb * d * 4,
        "state": 2 * B * H * N * d * es + B * H * Nbc * Lp * es,
        "assemble": B * H * Nb * Nbc // 8 + B * H * Nbc * Lp * es + B * H * Nb * Lp * es,
    }
    stages = {}
    for name in _lib.STAGES:
        st_ = {"ms": round(stage_ms[name], 4)}
        if name in nbytes and stage_ms[name] > 0:
            st_["GB/s"] = round(nbytes[name] / (stage_ms[name] * 1e-3) / 1e9, 1)
        stages[name] = st_
    if marg_rows:
        stages["assemble"]["TFLOP/s"] = round(2 * B * H * Nb * Nbc * Lp / max(stage_ms["assemble"], 1e-9) / 1e9, 1)
    # the fraction at the sampled clock takes the 90th percentile of the
    # samples (the clock while the calls run; a dip in the samples, which
    # the kernel times do not show, would otherwise inflate it)
    clk = None
    if clocks:
        cs = sorted(clocks)
        clk = {"median_mhz": round(float(cs[len(cs) // 2]), 1), "p90_mhz": round(float(cs[(9 * len(cs)) // 10]), 1),
               "samples": len(cs)}
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; local sinusoid Q/K + noise, V ~ N(0,1))",
        "config": {"workload": wl.name, "B": B, "H": H, "N": N, "d": d, "block": 64,
                   "crit_frac": rc, "negl_frac": rn, "k_c": kc, "k_n": kn, "parallelism": "none (1 GPU)"},
        "mfma_frac_fused": round(achieved / peak, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": profile_traffic(kname, "%s:%g/%g" % (wl.name, rc, rn), ksrc),
                     "kernel": kname, "mfma_type": mfma_type,
                     "flops_per_launch": f_fused, "avg_launch_ms": round(stage_ms["fused"], 4)},
        "timing": {"calls": args.calls, "warm_ms": spread(warm), "mall_flushed_ms": spread(flushed),
                   "flush": "512 MB fill before each call (MALL 256 MB)", "clock": clk},
        "dense_equivalent_tflops": round(4.0 * B * H * N * N * d / (ms * 1e-3) / 1e12, 3),
        "stages": stages,
    }
    if clk and clk["p90_mhz"] >= 1000.0:
        # the nominal peak is quoted at 2.4 GHz; the same peak at the sampled
        # clock (not given when the sampled clock shows a mostly idle GPU, as
        # for calls too short to keep it busy from the host)
        line["roofline"]["frac_at_measured_clock"] = round(achieved / (peak * clk["p90_mhz"] / 2400.0), 4)
    if cpu and not args.no_cpu:
        # bounded samples: whole heads for the small workloads, 64 query
        # blocks per head at 720p and HunyuanVideo, one per head when dense
        per_head = None if cid in (0, 1) else (1 if kc == Nb else 64)
        line["cpu_baseline"] = cpu_baseline(inp, wl, rc, rn, per_head)
    del q, k, v, out, ws
    torch.cuda.empty_cache()
    return line, ms


ALL_SETTINGS = [(0, 0.05, 0.10), (1, 0.05, 0.10), (2, 0.025, 0.10), (2, 0.05, 0.10), (2, 0.10, 0.10),
                (3, 0.05, 0.10), (4, 0.05, 0.10), (4, 1.0, 0.0)]


def copy_calibration(calls=5):
    """A plain elementwise kernel of known traffic (torch.neg on 2^28 float32:
    1 GiB read, 1 GiB written per launch): its FETCH_SIZE and WRITE_SIZE
    readings give the factors that turn those counters into HBM bytes."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(calls):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"kernel": "torch.neg float32 elementwise", "elements": n,
                                           "bytes_read_per_launch": 4 * n, "bytes_written_per_launch": 4 * n,
                                           "launches": calls}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--calls", type=int, default=100, help="calls timed one by one for the median / p10 / p90")
    ap.add_argument("--workload", type=int, default=1, help="named workload id (1 = Wan2.1 480p)")
    ap.add_argument("--crit", type=float, default=None)
    ap.add_argument("--negl", type=float, default=None)
    ap.add_argument("--all", action="store_true", help="one line per workload and setting (0-4, 4 dense)")
    ap.add_argument("--cpu-heads", type=int, default=0, help="heads in the CPU sample (0: all)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--quality", action="store_true", help="mask-quality diagnostics line instead of the forward line")
    ap.add_argument("--lvsa", action="store_true", help="LVSA frame-level sparse attention line (long-video workload)")
    ap.add_argument("--sta", action="store_true", help="sliding tile attention line (HunyuanVideo-sized latent)")
    ap.add_argument("--backward", action="store_true", help="SLA backward line (same workload as the forward)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain elementwise copy of known size (for scaling the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the SLA forward here is a single-GPU kernel "
              "pipeline (heads would shard across GPUs with no exchange); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_attention_video_sla_amd.inputs import WORKLOADS

    if args.copy_calibration:
        copy_calibration()
        return
    if args.lvsa:
        run_lvsa(args)
        return
    if args.sta:
        run_sta(args)
        return
    wl = WORKLOADS[args.workload]
    if args.backward:
        run_backward(args, wl)
        return
    if args.quality:
        run_quality(args, wl)
        return
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    if args.all:
        sparse_ms = None
        for cid, rc, rn in ALL_SETTINGS:
            line, ms = run_forward(args, cid, rc, rn, flush)
            if cid == 4 and rc < 1.0:
                sparse_ms = ms
            if cid == 4 and rc == 1.0 and sparse_ms:
                # the analogue of the SLA article's kernel-against-dense comparison (context only)
                line["dense_over_sparse_time"] = round(ms / sparse_ms, 2)
            print(json.dumps(line), flush=True)
        return
    rc = args.crit if args.crit is not None else wl.fracs[0][0]
    rn = args.negl if args.negl is not None else wl.fracs[0][1]
    line, _ = run_forward(args, args.workload, rc, rn, flush)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
