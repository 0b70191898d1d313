"""Host-side checks of bench.py's measurement plumbing (no GPU): the
rocprofv3 counter and traffic summaries are computed from synthetic CSVs with
known medians and calibration, and a request for more than one GPU is refused
before anything touches a device."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
SAMPLE = "void rts::sample_kernel<32, true, false>(rts::SampleArgs)"
COPY = "void at::native::elementwise_kernel_manual_unroll<copy>"
READ = "void rts::read_rows_kernel<32, true>(float const*, int, int, long, int, int, float*, int)"


def write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow(dict(Dispatch_Id=i + 1, Kernel_Name=kernel, Counter_Name=counter,
                            Counter_Value=value))


def read_summary(path):
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    return vals


def test_counter_summary_medians_and_ratios(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    a, b = tmp_path / "a.csv", tmp_path / "b.csv"
    rows_a = []
    for waves, cycles, wait, valu in ((100, 1000, 200, 50), (100, 2000, 400, 70), (100, 3000, 900, 60)):
        rows_a += [(SAMPLE, "SQ_WAVES", waves), (SAMPLE, "SQ_WAVE_CYCLES", cycles),
                   (SAMPLE, "SQ_WAIT_INST_ANY", wait), (SAMPLE, "SQ_INSTS_VALU", valu)]
    rows_a.append((COPY, "SQ_WAVES", 999999))   # other kernels are ignored
    write_csv(a, rows_a)
    write_csv(b, [(SAMPLE, "SQ_WAIT_ANY", v) for v in (500, 1200, 1300)])
    bench.summarize_counters([str(a), str(b)], "batch", "cmd")
    v = read_summary(tmp_path / "counters_sample_kernel_batch.txt")
    assert float(v["SQ_WAVES"]) == 100.0
    assert float(v["SQ_WAVE_CYCLES"]) == 2000.0
    assert float(v["SQ_WAIT_INST_ANY"]) == 400.0
    assert float(v["SQ_INSTS_VALU_dispatches"]) == 3
    assert float(v["wait_any_per_wave_cycle"]) == pytest.approx(0.2)
    assert float(v["wait_any_per_wave_cycle_all"]) == pytest.approx(0.6)
    assert float(v["SQ_INSTS_VALU_per_wave"]) == pytest.approx(0.6)
    assert v["source_sha256"] == bench.kernel_source_hash()


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    copy_kib = bench.COPY_BYTES / 1024.0
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    # FETCH_SIZE reads half the bytes for the copy; the sampler's median is 1,000 KiB raw;
    # the read kernel reads the batch's known bytes at the same factor
    known = bench.WORKLOAD_LOGIT_BYTES["batch"]
    write_csv(f, [(COPY, "FETCH_SIZE", copy_kib / 2)] * 3 +
              [(SAMPLE, "FETCH_SIZE", x) for x in (900.0, 1000.0, 1100.0)] +
              [(READ, "FETCH_SIZE", known / 1024.0 / 2)] * 2)
    write_csv(w, [(COPY, "WRITE_SIZE", copy_kib)] * 3 + [(SAMPLE, "WRITE_SIZE", 10.0)] * 3)
    bench.summarize_pmc(str(f), str(w), "batch", "cmd")
    v = read_summary(tmp_path / "traffic_sample_kernel_batch.txt")
    assert float(v["fetch_scale"]) == pytest.approx(2.0)
    assert float(v["write_scale"]) == pytest.approx(1.0)
    assert float(v["fetch_bytes_per_launch"]) == pytest.approx(2.0 * 1000.0 * 1024, rel=1e-6)
    assert float(v["hbm_bytes_per_launch"]) == pytest.approx(2.0 * 1000.0 * 1024 + 10.0 * 1024,
                                                            rel=1e-6)
    assert float(v["read_rows_fetch_scale"]) == pytest.approx(2.0, rel=1e-3)
    # the traffic figure the bench line reports comes back from the summary
    assert bench.read_traffic("batch") == pytest.approx(float(v["hbm_bytes_per_launch"]))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
