"""Host-side pieces of bench.py that its reported figures rest on (CPU only):
the algorithmic Newton-Schulz FLOP count (Notes on Muon blog, "Analysis":
2 (2 n m^2 + m^3) per iteration of an n x m matrix, m <= n) against the
per-configuration totals the measurement plan states, and the rule that a
committed traffic file is used only while it was taken from the current
kernel source."""
import os
import shutil

import pytest

import bench
import workloads as wl


def test_ns_flops_is_the_iteration_count():
    # orientation does not matter: the Gram matrix is always the smaller side
    assert bench.ns_flops(2048, 7168, 5) == bench.ns_flops(7168, 2048, 5)
    m, n = 2048, 7168
    assert bench.ns_flops(m, n, 1) == 2.0 * (2.0 * n * m * m + m ** 3)
    assert bench.ns_flops(m, n, 5) == 5 * bench.ns_flops(m, n, 1)


@pytest.mark.parametrize("cfg_id,total", [(2, 1.031e12), (3, 1.323e13), (4, 7.937e14), (5, 8.748e14)])
def test_config_totals(cfg_id, total):
    cfg = wl.config(cfg_id)
    got = sum(bench.ns_flops(s.rows, s.cols, 5) for s in cfg.matrices)
    assert abs(got - total) <= 5e-4 * total


def test_traffic_file_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    src = bench.traffic_file("full_layer")
    if not os.path.exists(src):
        pytest.skip("no committed traffic file")
    profiles = tmp_path / "profiles"
    profiles.mkdir()
    shutil.copy(src, profiles / "ns_gemm_traffic_full_layer.txt")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    value = bench.measured_traffic("full_layer")
    if value is None:
        pytest.skip("the committed traffic file predates the current kernel source")
    assert value > 0
    # another kernel source: the file no longer applies
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: "0" * 16)
    assert bench.measured_traffic("full_layer") is None
    assert bench.measured_traffic("no_such_workload") is None
