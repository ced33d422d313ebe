"""Host-side checks of bench.py: the one-GPU contract and the traffic figures
it reads from profiles/ (no GPU needed)."""

import os
import subprocess
import sys

import bench
from moe_grouped_gemm_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_every_workload_maps_to_a_kernel_with_hashed_sources():
    for i in range(synth.NUM_WORKLOADS):
        kernel = bench.kernel_of(synth.workload_spec(i))
        assert kernel in bench.KERNEL_SOURCES
        for name in bench.KERNEL_SOURCES[kernel]:
            assert os.path.exists(os.path.join(bench.CSRC, name)), name
        assert len(bench.kernel_source_sha(kernel)) == 16


def test_committed_traffic_figures_are_well_formed():
    # A traffic file is only used while its kernel's sources hash to the
    # value it records (otherwise the bench line reports traffic as null);
    # every committed one names a hash and a positive byte count.
    found = 0
    for i in range(synth.NUM_WORKLOADS):
        spec = synth.workload_spec(i)
        path = os.path.join(bench.PROFILES, f"traffic_{spec.name}.txt")
        if not os.path.exists(path):
            continue
        found += 1
        fields = dict(line.split(":", 1) for line in open(path) if ":" in line and not line.startswith("#"))
        assert len(fields["kernel_source_sha256_16"].strip()) == 16
        assert float(fields["hbm_bytes_per_launch"]) > 0
        traffic = bench.read_traffic(spec)
        assert traffic is None or traffic == float(fields["hbm_bytes_per_launch"])
    assert found >= 1


def test_stale_traffic_figure_is_ignored(tmp_path, monkeypatch):
    spec = synth.workload_spec(1)
    (tmp_path / f"traffic_{spec.name}.txt").write_text(
        "kernel_source_sha256_16: 0000000000000000\nhbm_bytes_per_launch: 123\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.read_traffic(spec) is None
    sha = bench.kernel_source_sha(bench.kernel_of(spec))
    (tmp_path / f"traffic_{spec.name}.txt").write_text(
        f"kernel_source_sha256_16: {sha}\nhbm_bytes_per_launch: 123\n")
    assert bench.read_traffic(spec) == 123.0
