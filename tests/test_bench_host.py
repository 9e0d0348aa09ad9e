"""Host-side checks of bench.py (no GPU): the one-GPU contract and the reading
of the committed HBM-traffic summaries."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_rows_are_used_only_for_the_profiled_sources(tmp_path, monkeypatch):
    kernel = "flash_kernel<bf16,4,partial>"
    good = bench.kernel_sources_hash(kernel)
    assert good == bench.kernel_sources_hash(kernel) and len(good) == 16
    prof = tmp_path / "profiles"
    prof.mkdir()

    def write(sources):
        (prof / "hbm_traffic_demo.md").write_text(
            "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched GB | written GB | sources |\n"
            "|---|---|---|---|---|---|---|\n"
            f"| {kernel} | 4 | 1 | 1 | 10.72 | 0.18 | {sources} |\n")

    # the profiles are read from the temporary folder; the source hash stays
    # the one of the real kernel sources
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sources_hash", lambda k: good)
    write(good)
    assert bench.measured_traffic((kernel,), "demo workload") == round((10.72 + 0.18) * 1e9)
    write("0" * 16)
    assert bench.measured_traffic((kernel,), "demo workload") is None
    # a stage needs every one of its kernels' rows
    write(good)
    assert bench.measured_traffic((kernel, "select_kernel<bf16,1>"), "demo workload") is None
    assert bench.measured_traffic((kernel,), "absent workload") is None


def test_trace_rows_are_used_only_for_the_profiled_sources(tmp_path, monkeypatch):
    kernel = "flash_kernel<bf16,4,bound>"
    good = bench.kernel_sources_hash(kernel)
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sources_hash", lambda k: good)

    def write(sources):
        (prof / "gsa_forward_demo_kernel_trace.md").write_text(
            "| kernel | calls | average ms | min ms | max ms | share | sources |\n"
            "|---|---|---|---|---|---|---|\n"
            f"| {kernel} | 8 | 28.117 | 27.9 | 28.4 | 31.4% | {sources} |\n")

    write(good)
    assert bench.traced_ms("demo workload") == {kernel: 28.117}
    write("f" * 16)
    assert bench.traced_ms("demo workload") == {}


def test_clock_sampler_reads_the_marked_level(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1500Mhz *\n2: 2400Mhz\n")
    assert bench.ClockSampler._read(str(f)) == 1500.0
