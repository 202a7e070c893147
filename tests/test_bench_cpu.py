"""Host-side pieces of bench.py: the stored-counter lookup is voided by any
change to the kernel source or to a package header it includes."""
import hashlib
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_source_sha_covers_included_headers(tmp_path, monkeypatch):
    (tmp_path / "a.h").write_bytes(b"// a\n")
    (tmp_path / "b.h").write_bytes(b'#include "a.h"\n// b\n')
    (tmp_path / "k.hip").write_bytes(b'#include "b.h"\n#include "a.h"\n#include <stdint.h>\n')
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    alone = hashlib.sha256((tmp_path / "k.hip").read_bytes()).hexdigest()[:16]
    first = bench.source_sha("k.hip")
    assert first != alone
    (tmp_path / "a.h").write_bytes(b"// a, changed\n")
    assert bench.source_sha("k.hip") != first


def test_fused_traffic_needs_matching_sha(tmp_path, monkeypatch):
    (tmp_path / "k.hip").write_bytes(b"// kernel\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    sha = bench.source_sha("k.hip")
    prof = tmp_path / "p.md"
    prof.write_text("k_kernel HBM bytes per launch: 1234 (source sha256 %s)\n" % sha)
    assert bench.fused_traffic(str(prof), "k_kernel", "k.hip") == 1234
    prof.write_text("k_kernel HBM bytes per launch: 1234 (source sha256 %s)\n" % ("0" * 16))
    assert bench.fused_traffic(str(prof), "k_kernel", "k.hip") is None
    assert bench.fused_traffic(str(tmp_path / "missing.md"), "k_kernel", "k.hip") is None
