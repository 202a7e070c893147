"""The C-ABI library: it loads, exports every symbol include/sla.h declares,
and rejects bad arguments on the host before launching anything (no GPU
needed for these calls)."""
import ctypes
import os
import re

import pytest

from sparse_attention_video_sla_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sla.h")


@pytest.fixture(scope="module")
def lib():
    # SLA_TEST_LIB: another build of the same sources (the sanitizer test
    # runs this file against a host-sanitized copy)
    path = os.environ.get("SLA_TEST_LIB") or _lib.LIB_PATH
    if not os.path.exists(path):
        from sparse_attention_video_sla_amd import build
        build.build()
    return _lib.load(path)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sla_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert getattr(lib, n) is not None


def test_version(lib):
    assert lib.sla_version() >= 100


def test_counts(lib):
    kc, kn = ctypes.c_int(), ctypes.c_int()
    assert lib.sla_counts(512, 0.05, 0.10, ctypes.byref(kc), ctypes.byref(kn)) == _lib.SLA_OK
    assert (kc.value, kn.value) == (26, 51)
    assert lib.sla_counts(1857, 1.0, 0.0, ctypes.byref(kc), ctypes.byref(kn)) == _lib.SLA_OK
    assert (kc.value, kn.value) == (1857, 0)
    assert lib.sla_counts(512, 0.6, 0.5, ctypes.byref(kc), ctypes.byref(kn)) == _lib.SLA_ERR_INVALID_ARG
    assert b"fractions" in lib.sla_last_error()


def test_counts_match_golden(lib):
    path = os.path.join(ROOT, "tests", "golden", "counts.txt")
    for line in open(path):
        if not line.strip() or line.startswith("#"):
            continue
        Nb, rc, rn, ekc, ekn = line.split()
        kc, kn = ctypes.c_int(), ctypes.c_int()
        assert lib.sla_counts(int(Nb), float(rc), float(rn), ctypes.byref(kc), ctypes.byref(kn)) == 0
        assert (kc.value, kn.value) == (int(ekc), int(ekn))


def test_workspace_size(lib):
    n = ctypes.c_size_t()
    assert lib.sla_workspace_size(1, 12, 32760, 128, 64, _lib.SLA_BF16, 0.05, 0.10, ctypes.byref(n)) == 0
    assert n.value > 0
    big = n.value
    assert lib.sla_workspace_size(1, 12, 32760, 128, 64, _lib.SLA_BF16, 1.0, 0.0, ctypes.byref(n)) == 0
    assert n.value < big        # no marginal blocks: no linear states
    assert lib.sla_workspace_size(1, 12, 32760, 96, 64, _lib.SLA_BF16, 0.05, 0.10, ctypes.byref(n)) == _lib.SLA_ERR_UNSUPPORTED
    assert lib.sla_workspace_size(1, 12, 32760, 128, 32, _lib.SLA_BF16, 0.05, 0.10, ctypes.byref(n)) == _lib.SLA_ERR_UNSUPPORTED
    assert lib.sla_workspace_size(1, 12, 64 * 2433, 128, 64, _lib.SLA_BF16, 0.05, 0.10, ctypes.byref(n)) == _lib.SLA_ERR_UNSUPPORTED
    assert lib.sla_workspace_size(0, 12, 100, 128, 64, _lib.SLA_BF16, 0.05, 0.10, ctypes.byref(n)) == _lib.SLA_ERR_INVALID_ARG
    assert lib.sla_workspace_size(1, 1, 100, 128, 64, 7, 0.05, 0.10, ctypes.byref(n)) == _lib.SLA_ERR_UNSUPPORTED


FAKE = 0x10000   # never dereferenced: every call below fails validation first


def fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w=FAKE, ind=_lib.SLA_BF16, outd=_lib.SLA_F32, B=1, H=1, N=128, d=128,
             block=64, rc=0.05, rn=0.10, phi=0, out=FAKE, mask=None, ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    return lib.sla_forward(a["q"], a["k"], a["v"], a["w"], a["ind"], a["outd"], a["B"], a["H"], a["N"], a["d"],
                           a["block"], a["rc"], a["rn"], a["phi"], a["out"], a["mask"], a["ws"], a["wsb"],
                           a["stream"])


def test_forward_rejects_before_launch(lib):
    assert fwd(lib, q=None) == _lib.SLA_ERR_INVALID_ARG
    assert fwd(lib, out=None) == _lib.SLA_ERR_INVALID_ARG
    assert fwd(lib, d=32) == _lib.SLA_ERR_UNSUPPORTED
    assert fwd(lib, block=128) == _lib.SLA_ERR_UNSUPPORTED
    assert fwd(lib, N=0) == _lib.SLA_ERR_INVALID_ARG
    assert fwd(lib, rc=0.7, rn=0.4) == _lib.SLA_ERR_INVALID_ARG
    assert fwd(lib, rc=-0.1) == _lib.SLA_ERR_INVALID_ARG
    assert fwd(lib, phi=1) == _lib.SLA_ERR_UNSUPPORTED
    assert fwd(lib, ind=_lib.SLA_F32, outd=_lib.SLA_BF16) == _lib.SLA_ERR_UNSUPPORTED
    assert fwd(lib, wsb=16) == _lib.SLA_ERR_WORKSPACE
    assert b"workspace" in lib.sla_last_error()
    n = ctypes.c_size_t()
    lib.sla_workspace_size(1, 1, 128, 128, 64, _lib.SLA_BF16, 0.05, 0.10, ctypes.byref(n))
    assert fwd(lib, ws=FAKE + 8, wsb=n.value) == _lib.SLA_ERR_INVALID_ARG   # misaligned workspace


def test_pool_classify_reject(lib):
    assert lib.sla_pool(None, FAKE, _lib.SLA_BF16, 1, 1, 64, 128, 64, FAKE, FAKE, None) == _lib.SLA_ERR_INVALID_ARG
    assert lib.sla_pool(FAKE, FAKE, _lib.SLA_BF16, 1, 1, 64, 100, 64, FAKE, FAKE, None) == _lib.SLA_ERR_UNSUPPORTED
    assert lib.sla_classify(FAKE, FAKE, 1, 1, 8, 128, 0.5, 0.1, None, FAKE, None, None, None) == _lib.SLA_ERR_INVALID_ARG
    assert lib.sla_classify(FAKE, FAKE, 1, 1, 8, 128, 0.5, 0.1, FAKE, None, None, None, None) == _lib.SLA_ERR_INVALID_ARG
    assert lib.sla_classify(FAKE, FAKE, 1, 1, 2433, 128, 0.05, 0.1, FAKE, FAKE, None, None, None) == _lib.SLA_ERR_UNSUPPORTED


def test_lvsa_plan_matches_oracle_and_rejects(lib):
    """sla_lvsa_plan is host arithmetic: T_per, |G_s| and the set size of the
    LVSA page's frame sets, checked against the oracle's sets."""
    from oracle import lvsa
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    for T in (1, 3, 10, 21, 41, 121, 481):
        for C in (4, 7, 21, 33):
            for W in (0, 1, 3):
                if C - (2 * W + 1) < 1:
                    assert lib.sla_lvsa_plan(T, C, W, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)) != 0
                    continue
                assert lib.sla_lvsa_plan(T, C, W, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)) == 0
                sets = lvsa.all_sets(T, C, W, 0)
                assert a.value == lvsa.period(T, C, W)
                assert b.value == len(lvsa.globals_at(T, a.value, 0))
                assert {c.value} == {len(x) for x in sets}


def test_lvsa_entry_points_reject_bad_shapes(lib):
    n = ctypes.c_size_t()
    assert lib.sla_lvsa_workspace_size(1, 1, 1000, 3, 5, 1, ctypes.byref(n)) != 0    # N % T
    assert lib.sla_lvsa_workspace_size(1, 1, 1000, 20, 5, 1, ctypes.byref(n)) != 0   # 50-token frames
    assert lib.sla_lvsa_workspace_size(1, 1, 1000, 10, 3, 1, ctypes.byref(n)) != 0   # C <= 2W + 1
    assert lib.sla_lvsa_workspace_size(1, 1, 64 * 4096, 64, 21, 3, ctypes.byref(n)) != 0   # 4096 blocks
    assert lib.sla_lvsa_workspace_size(1, 12, 188760, 121, 21, 3, ctypes.byref(n)) == 0 and n.value > 0


def test_sta_tile_order_matches_oracle_and_shapes_are_checked(lib):
    """sla_sta_tile_order is host arithmetic: the tile-major permutation,
    against the oracle's; the STA entry points reject bad shapes on the host."""
    import numpy as np
    from oracle import sta
    for grid, tile in (((4, 6, 8), (2, 3, 4)), ((30, 48, 80), (6, 8, 8)), ((3, 4, 16), (1, 4, 16))):
        perm = np.empty(grid[0] * grid[1] * grid[2], np.int32)
        assert lib.sla_sta_tile_order(*grid, *tile, perm.ctypes.data) == 0
        assert np.array_equal(perm, sta.tile_order(grid, tile))
    n = ctypes.c_size_t()
    assert lib.sla_sta_workspace_size(1, 1, 30, 48, 80, 6, 8, 8, 18, 27, 24, ctypes.byref(n)) == 0 and n.value > 0
    assert lib.sla_sta_workspace_size(1, 1, 30, 48, 80, 4, 8, 8, 18, 27, 24, ctypes.byref(n)) != 0   # 4 does not divide 30
    assert lib.sla_sta_workspace_size(1, 1, 30, 48, 80, 6, 8, 5, 18, 27, 24, ctypes.byref(n)) != 0   # 5 does not divide 80
    assert lib.sla_sta_workspace_size(1, 1, 6, 6, 6, 3, 3, 3, 18, 27, 24, ctypes.byref(n)) != 0      # 27-token tiles
    assert lib.sla_sta_workspace_size(1, 1, 30, 48, 80, 6, 8, 8, 0, 27, 24, ctypes.byref(n)) != 0    # empty window


def bwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w=FAKE, do=FAKE, ind=_lib.SLA_BF16, B=1, H=1, N=128, d=128, block=64,
             rc=0.05, rn=0.10, phi=0, dq=FAKE, dk=FAKE, dv=FAKE, dw=FAKE, ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    return lib.sla_backward(a["q"], a["k"], a["v"], a["w"], a["do"], a["ind"], a["B"], a["H"], a["N"], a["d"],
                            a["block"], a["rc"], a["rn"], a["phi"], a["dq"], a["dk"], a["dv"], a["dw"], a["ws"],
                            a["wsb"], a["stream"])


def test_backward_rejects_before_launch(lib):
    """sla_backward validates everything on the host before any launch."""
    assert bwd(lib, do=None) == _lib.SLA_ERR_INVALID_ARG
    assert bwd(lib, dw=None) == _lib.SLA_ERR_INVALID_ARG
    assert bwd(lib, ind=_lib.SLA_F32) == _lib.SLA_ERR_UNSUPPORTED
    assert bwd(lib, phi=1) == _lib.SLA_ERR_UNSUPPORTED
    assert bwd(lib, d=96) == _lib.SLA_ERR_UNSUPPORTED
    assert bwd(lib, N=0) == _lib.SLA_ERR_INVALID_ARG
    assert bwd(lib, rc=0.7, rn=0.4) == _lib.SLA_ERR_INVALID_ARG
    assert bwd(lib, ws=None) == _lib.SLA_ERR_INVALID_ARG
    assert bwd(lib, wsb=16) == _lib.SLA_ERR_WORKSPACE
    n = ctypes.c_size_t()
    assert lib.sla_backward_workspace_size(1, 1, 128, 128, 64, 0.05, 0.10, ctypes.byref(n)) == 0
    assert bwd(lib, ws=FAKE + 8, wsb=n.value) == _lib.SLA_ERR_INVALID_ARG   # misaligned workspace


def bwd_saved(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w=FAKE, do=FAKE, ind=_lib.SLA_BF16, B=1, H=1, N=128, d=128, block=64,
             rc=0.05, rn=0.10, phi=0, dq=FAKE, dk=FAKE, dv=FAKE, dw=FAKE, ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    return lib.sla_backward_saved(a["q"], a["k"], a["v"], a["w"], a["do"], a["ind"], a["B"], a["H"], a["N"], a["d"],
                                  a["block"], a["rc"], a["rn"], a["phi"], a["dq"], a["dk"], a["dv"], a["dw"], a["ws"],
                                  a["wsb"], a["stream"])


def fwd_save(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w=FAKE, ind=_lib.SLA_BF16, outd=_lib.SLA_F32, B=1, H=1, N=128, d=128, block=64,
             rc=0.05, rn=0.10, phi=0, out=FAKE, mask=None, ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    return lib.sla_forward_save(a["q"], a["k"], a["v"], a["w"], a["ind"], a["outd"], a["B"], a["H"], a["N"], a["d"],
                                a["block"], a["rc"], a["rn"], a["phi"], a["out"], a["mask"], a["ws"], a["wsb"],
                                a["stream"])


def test_saved_backward_rejects_before_launch(lib):
    """sla_forward_save and sla_backward_saved validate everything on the
    host before any launch; the saved state is sla_backward's workspace."""
    n = ctypes.c_size_t()
    assert lib.sla_backward_workspace_size(1, 1, 128, 128, 64, 0.05, 0.10, ctypes.byref(n)) == 0
    for call in (bwd_saved, fwd_save):
        assert call(lib, q=None) == _lib.SLA_ERR_INVALID_ARG
        assert call(lib, ind=_lib.SLA_F32) == _lib.SLA_ERR_UNSUPPORTED
        assert call(lib, phi=1) == _lib.SLA_ERR_UNSUPPORTED
        assert call(lib, d=96) == _lib.SLA_ERR_UNSUPPORTED
        assert call(lib, N=0) == _lib.SLA_ERR_INVALID_ARG
        assert call(lib, rc=0.7, rn=0.4) == _lib.SLA_ERR_INVALID_ARG
        assert call(lib, ws=None, wsb=n.value) == _lib.SLA_ERR_INVALID_ARG
        assert call(lib, wsb=16) == _lib.SLA_ERR_WORKSPACE
        assert call(lib, wsb=n.value - 1) == _lib.SLA_ERR_WORKSPACE
        assert call(lib, ws=FAKE + 8, wsb=n.value) == _lib.SLA_ERR_INVALID_ARG   # misaligned
    assert bwd_saved(lib, do=None) == _lib.SLA_ERR_INVALID_ARG
    assert bwd_saved(lib, dw=None) == _lib.SLA_ERR_INVALID_ARG
    assert fwd_save(lib, out=None) == _lib.SLA_ERR_INVALID_ARG
    assert fwd_save(lib, outd=2) == _lib.SLA_ERR_UNSUPPORTED


def test_backward_workspace_size(lib):
    """The backward workspace holds the forward's and grows with the sequence."""
    nf, nb, nb2 = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.sla_workspace_size(1, 12, 32760, 128, 64, _lib.SLA_BF16, 0.05, 0.10, ctypes.byref(nf)) == 0
    assert lib.sla_backward_workspace_size(1, 12, 32760, 128, 64, 0.05, 0.10, ctypes.byref(nb)) == 0
    assert nb.value > nf.value
    assert lib.sla_backward_workspace_size(1, 12, 2 * 32760, 128, 64, 0.05, 0.10, ctypes.byref(nb2)) == 0
    assert nb2.value > nb.value
    assert lib.sla_backward_workspace_size(1, 12, 32760, 128, 64, 0.05, 0.10, None) == _lib.SLA_ERR_INVALID_ARG
    assert lib.sla_backward_workspace_size(1, 12, 32760, 64, 32, 0.05, 0.10, ctypes.byref(nb)) == _lib.SLA_ERR_UNSUPPORTED


def test_lists_entry_points_reject(lib):
    n = ctypes.c_size_t()
    assert lib.sla_lists_workspace_size(1, 2, 1000, 0, ctypes.byref(n)) == _lib.SLA_ERR_INVALID_ARG    # kmax < 1
    assert lib.sla_lists_workspace_size(1, 2, 1000, 17, ctypes.byref(n)) == _lib.SLA_ERR_INVALID_ARG   # kmax > Nb = 16
    assert lib.sla_lists_workspace_size(1, 2, 64 * 4096, 8, ctypes.byref(n)) == _lib.SLA_ERR_UNSUPPORTED   # 4096 blocks
    assert lib.sla_lists_workspace_size(1, 2, 1000, 16, ctypes.byref(n)) == 0 and n.value > 0
    args = [FAKE, FAKE, FAKE, _lib.SLA_BF16, _lib.SLA_F32, 1, 2, 1000, 128, 64, FAKE, FAKE, 8, FAKE, FAKE, 0, None]
    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.sla_forward_lists(*a)
    assert call(a10=None) == _lib.SLA_ERR_INVALID_ARG            # no lists
    assert call(a3=_lib.SLA_F32) == _lib.SLA_ERR_UNSUPPORTED      # float inputs
    assert call(a12=40) == _lib.SLA_ERR_INVALID_ARG              # kmax > Nb
    assert call() == _lib.SLA_ERR_WORKSPACE                      # no room for the schedule


def test_noalloc_rejects_on_the_host(lib):
    """sla_forward_noalloc checks its arguments like sla_forward, and rejects
    sizes whose workspace exceeds its static scratch before any device call."""
    def call(B=1, H=2, N=3000, d=128, ind=_lib.SLA_BF16, rc=0.05, rn=0.10, q=FAKE):
        return lib.sla_forward_noalloc(q, FAKE, FAKE, FAKE, ind, _lib.SLA_F32, B, H, N, d, 64, rc, rn,
                                       _lib.SLA_PHI_SOFTMAX, FAKE, None, None)
    assert call(B=1, H=24, N=118800) == _lib.SLA_ERR_WORKSPACE          # 3048 MiB of workspace
    assert b"static scratch" in lib.sla_last_error()
    n = ctypes.c_size_t()
    assert lib.sla_workspace_size(1, 12, 32760, 128, 64, _lib.SLA_BF16, 0.05, 0.10, ctypes.byref(n)) == 0
    assert n.value <= _lib.NOALLOC_SCRATCH_BYTES                          # the Wan2.1 480p shape fits
    assert call(N=0) == _lib.SLA_ERR_INVALID_ARG
    assert call(d=96) == _lib.SLA_ERR_UNSUPPORTED
    assert call(ind=7) == _lib.SLA_ERR_UNSUPPORTED
    assert call(rc=0.7, rn=0.4) == _lib.SLA_ERR_INVALID_ARG
    assert call(q=None) == _lib.SLA_ERR_INVALID_ARG


def test_noalloc_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define SLA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES
