"""The profile summaries bench.py writes and reads back (no GPU).

bench.py reports the dominant kernel's HBM traffic and kernel-trace
duration from the committed summaries in profiles/ only while the kernel
sources are those the summaries were taken from.  These tests feed the
summarisers small counter and trace tables of known content (written to a
temporary directory; the committed profiles are not touched) and check the
arithmetic (the copy calibration's scale factors, per-launch averages, the
dominant kernel) and the staleness gate.
"""
import csv
import importlib.util
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PAIR = "gemm_pair_kernel<128, 128, 32, 3, false, false, true, false, true>"
COPY = "at::native::vectorized_elementwise_kernel<4, MulFunctor<float>, std::array<char*, 2ul> >"


@pytest.fixture
def bench(monkeypatch, tmp_path):
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    monkeypatch.setattr(b, "KTRACE_FILE", str(tmp_path / "ktrace.json"))
    return b


def write_pmc(path, counter, rows):
    """rows: (kernel, value KiB, start ns, end ns) dispatches."""
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        for i, (k, v, t0, t1) in enumerate(rows):
            w.writerow([i, f"void (anonymous namespace)::{k}(float*)" if "gemm" in k or "adamw" in k else k, counter, v,
                        t0, t1])


def test_traffic_summary_scales_by_the_copy_and_gates_on_sources(bench, tmp_path, capsys):
    # a 1024 MiB copy read as 524288 KiB by FETCH_SIZE (64-byte units) and 1048576 KiB by WRITE_SIZE
    fetch = [(COPY, 524288.0, 0, 10**6)]
    write = [(COPY, 1048576.0, 0, 10**6)]
    for i in range(3):  # the pair: 3 dispatches of 10 ms, 1000 KiB fetched and 500 KiB written each
        fetch.append((PAIR, 1000.0, 10**7 * i, 10**7 * (i + 1)))
        write.append((PAIR, 500.0, 10**7 * i, 10**7 * (i + 1)))
    fetch.append(("adamw_kernel", 9000.0, 0, 10**6))  # larger traffic, shorter in total: not dominant
    write.append(("adamw_kernel", 9000.0, 0, 10**6))
    fetch.append(("mfma_probe_kernel", 0.0, 0, 10**8))  # the peak probe, longest of all, is not a step kernel
    write.append(("mfma_probe_kernel", 0.0, 0, 10**8))
    write_pmc(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    write_pmc(tmp_path / "w.csv", "WRITE_SIZE", write)
    bench.pmc_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 3, 1024, "cmd", "124m")
    text = capsys.readouterr().out
    assert "scale 2.000" in text and "scale 1.000" in text
    t = json.load(open(tmp_path / "traffic.json"))
    assert t["kernel"] == PAIR and t["dispatches"] == 3
    assert t["hbm_read_bytes_per_launch"] == pytest.approx(1000 * 1024 * 2.0)
    assert t["hbm_write_bytes_per_launch"] == pytest.approx(500 * 1024 * 1.0)
    assert bench.measured_traffic(PAIR, "124m") == pytest.approx(1000 * 1024 * 2.0 + 500 * 1024)
    assert bench.measured_traffic(PAIR, "xl") is None  # another workload
    assert bench.measured_traffic("adamw_kernel", "124m") is None  # not the summarised kernel
    bench.sources_sha256 = lambda: "0" * 64  # the kernel sources changed since
    assert bench.measured_traffic(PAIR, "124m") is None


def test_trace_summary_averages_and_gates_on_sources(bench, tmp_path, capsys):
    with open(tmp_path / "stats.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        w.writerow([f"void (anonymous namespace)::{PAIR}(GemmArgs, GemmArgs, int, int)", 13, 8.8e6, 676923.0,
                    3.3e5, 5.2e6, 60.0])
        w.writerow(["void (anonymous namespace)::adamw_kernel(float*)", 1, 6.0e5, 6.0e5, 6.0e5, 6.0e5, 4.0])
    bench.kt_summary(str(tmp_path / "stats.csv"), "cmd", "124m")
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("| `")]
    assert lines[0].startswith(f"| `{PAIR}` | 13 | 8.800 | 0.6769")  # sorted by total time
    assert bench.traced_duration(PAIR, "124m") == pytest.approx(0.676923)
    assert bench.traced_duration(PAIR, "xl") is None
    bench.sources_sha256 = lambda: "f" * 64
    assert bench.traced_duration(PAIR, "124m") is None


def test_trace_summary_of_another_workload_leaves_the_headline_figures(bench, tmp_path, monkeypatch, capsys):
    with open(tmp_path / "stats.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        w.writerow(["void (anonymous namespace)::adamw_kernel(float*)", 2, 1.6e7, 8.0e6, 7.9e6, 8.1e6, 100.0])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "sources_sha256", lambda: "a" * 64)
    os.makedirs(tmp_path / "profiles")
    bench.kt_summary(str(tmp_path / "stats.csv"), "cmd", "xl")
    capsys.readouterr()
    with open(tmp_path / "profiles" / "kernel_trace_gpt2_xl_b4_t1024.json") as fh:
        t = json.load(fh)
    assert t["config"] == "xl" and t["kernels"]["adamw_kernel"]["avg_ms"] == pytest.approx(8.0)
    assert not os.path.exists(tmp_path / "ktrace.json")  # the headline's summary is not written
    assert bench.traced_duration("adamw_kernel", "xl") is None  # nor read for another workload


def test_step_roofline_takes_each_site_at_its_slower_bound(bench):
    ms_flops, ms_bytes = 157.3e9, 8e9  # one ms at the fp32 matrix peak, one ms at the HBM peak
    sites = [dict(flops=2 * ms_flops, bytes=0.1 * ms_bytes),
             dict(flops=0.0, bytes=3 * ms_bytes),
             dict(flops=ms_flops, bytes=ms_bytes)]
    assert bench.step_roofline_ms(sites, 1) == pytest.approx(2.0 + 3.0 + 1.0)
    assert bench.step_roofline_ms(sites, 2) == pytest.approx(3.0)
