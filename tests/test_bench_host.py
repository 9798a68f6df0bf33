"""CPU checks of bench.py's host logic (no GPU): the one-GPU guard and the
rule that PMC traffic is taken from a committed summary only while the
summary's recorded source hash matches the kernel source."""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert out.returncode == 2
    assert "one GPU" in out.stderr


def test_traffic_needs_a_matching_source_hash(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel source\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    doc = prof / "pmc_kern_wl.md"
    doc.write_text(f"# x\n\ntraffic_bytes_per_launch: 12345 source_sha256: {sha} source: k.hip\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profiles("kern", "wl") == 12345.0
    src.write_text("kernel source, changed\n")             # the kernel changed since the counters were taken
    assert bench.traffic_from_profiles("kern", "wl") is None
    assert bench.traffic_from_profiles("other", "wl") is None


def test_committed_profiles_match_the_sources():
    """The committed PMC summaries carry a traffic figure; when a kernel source
    has changed since they were taken the bench reports null, and this test
    says so (skip) rather than failing the suite."""
    stale = []
    for kern, wl in (("gemm_smfmac_wide", "prefill"), ("gemv_tok1_24", "decode"), ("gemv_stream_68", "decode"),
                     ("gemv_stream_d2", "decode"), ("gemv_stream_j6", "decode")):
        assert os.path.exists(os.path.join(ROOT, "profiles", f"pmc_{kern}_{wl}.md")), (kern, wl)
        if bench.traffic_from_profiles(kern, wl) is None:
            stale.append(f"{kern}/{wl}")
    if stale:
        pytest.skip("PMC summaries older than the kernel source (retake them): " + ", ".join(stale))


@pytest.mark.parametrize("name,T,R,K", [("prefill", 4096, 6912, 2560), ("train", 8192, 11008, 4096),
                                        ("decode", 16, 4096, 4096), ("tiny", 16, 256, 256),
                                        ("sweep", 2048, 8192, 8192)])
def test_workload_shapes(name, T, R, K):
    from workloads import WORKLOADS
    wl = WORKLOADS[name]
    assert (wl.T, wl.R, wl.K) == (T, R, K)
