"""Host-side checks of bench.py (no GPU): argument handling that must not
touch the device, the algorithmic byte counts, and the traffic lookup that
ties the reported HBM bytes to the kernel sources they were measured on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    p = _run("--gpus", "2")
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_unknown_workload_is_refused_before_the_device():
    p = _run("--only", "no_such_workload")
    assert p.returncode == 2
    assert "unknown workload" in p.stderr and "step_48_layers" in p.stderr


def test_algorithmic_bytes_per_token():
    # one pass reads the E fp32 scores and alpha once; the step has two passes
    for E in (16, 256):
        bpt = bench.bytes_per_token(E)
        assert bpt["pass1"] == 4 * E + 4 and bpt["pass2"] == 4 * E + 4
        assert bpt["step"] == bpt["pass1"] + bpt["pass2"]
    assert 1048576 * bench.bytes_per_token(256)["pass1"] == 1077936128


def test_traffic_summary_matches_the_kernel_sources():
    """When the committed counter summary was taken on the current pass
    kernels (its source hash matches), the benchmark reports its bytes, and
    they are within a few percent of the algorithmic bytes (no wasted
    re-reads).  After a kernel change the benchmark reports null until the
    counters are taken again; this test then says so."""
    t1 = bench.measured_traffic("pass1_topk_hist_hi")
    if t1 is None:
        pytest.skip("traffic summary taken on other kernel sources: take the FETCH_SIZE / WRITE_SIZE "
                    "counters again")
    for k in ("pass1_topk_hist_hi", "pass2_hist_lo"):
        t = bench.measured_traffic(k)
        assert t is not None and 1.0 <= t / 1077936128 < 1.05, (k, t)
    assert bench.measured_traffic("no_such_kernel") is None


def test_suites_are_named():
    assert set(bench.SUITES) >= {"single", "step_48_layers", "router", "controller", "k3_skew"}
