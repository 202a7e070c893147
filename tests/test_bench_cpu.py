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


def test_profile_traffic_keyed_on_kernel_workload_and_sha(tmp_path, monkeypatch):
    (tmp_path / "csrc").mkdir()
    (tmp_path / "profiles").mkdir()
    (tmp_path / "csrc" / "k.hip").write_bytes(b"// kernel\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path / "csrc"))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench.source_sha("k.hip")
    prof = tmp_path / "profiles" / "k_w1_stats.md"
    line = "traffic: kernel=k_kernel workload=%s bytes_per_launch=%d source=k.hip sha256=%s\n"
    prof.write_text(line % ("w1", 1234, sha) + line % ("w2", 99, sha))
    assert bench.profile_traffic("k_kernel", "w1", "k.hip") == 1234
    assert bench.profile_traffic("k_kernel", "w2", "k.hip") == 99
    assert bench.profile_traffic("k_kernel", "w3", "k.hip") is None          # no summary for that workload
    assert bench.profile_traffic("other_kernel", "w1", "k.hip") is None
    prof.write_text(line % ("w1", 1234, "0" * 16))
    assert bench.profile_traffic("k_kernel", "w1", "k.hip") is None          # counters of another source
    assert bench.profile_traffic("k_kernel", "w1", "missing.hip") is None
