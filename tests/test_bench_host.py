"""Host-side logic of bench.py (no GPU): the one-GPU contract and the HBM
traffic figure built from two rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE)
scaled by what the same counters read for a copy kernel of known size."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture()
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _counter_csv(path, counter, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="", encoding="utf-8") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_from_counters_and_copy_calibration(bench, tmp_path, monkeypatch):
    layer = "void (anonymous namespace)::moe_barrier_kernel<1, false>((anonymous namespace)::MoeArgs)"
    copy = "void at::native::elementwise_kernel_copy(int)"
    # the calibration copies move 1 GiB each way; FETCH reads half of it in KiB
    # (factor 2), WRITE all of it (factor 1).  They are the pass's last three
    # copies: the workload's own copies before them (a small one, a 2 GiB one)
    # must not enter the mean
    cal = [(copy, 524288.0)] * 3
    fetch = [(copy, 4.0), (copy, 1048576.0 * 1.3), (layer, 1000.0), (layer, 1100.0), (layer, 900.0)] + cal
    write = [(copy, 2.0), (copy, 2097152.0), (layer, 10.0), (layer, 10.0), (layer, 10.0)] + [(copy, 1048576.0)] * 3
    fcsv, wcsv = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(fcsv, "FETCH_SIZE", fetch)
    _counter_csv(wcsv, "WRITE_SIZE", write)
    summary = tmp_path / "summary.txt"
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(summary))
    bench.ingest_pmc(str(fcsv), str(wcsv))
    assert summary.exists()
    t = bench.read_traffic(0)
    assert t == pytest.approx(1000.0 * 1024 * 2.0 + 10.0 * 1024 * 1.0)


def test_traffic_is_withheld_once_the_kernel_source_changed(bench, tmp_path, monkeypatch):
    layer = "moe_barrier_kernel<1, false>"
    fcsv, wcsv = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(fcsv, "FETCH_SIZE", [(layer, 100.0), ("copy", 524288.0)])
    _counter_csv(wcsv, "WRITE_SIZE", [(layer, 1.0), ("copy", 1048576.0)])
    summary = tmp_path / "summary.txt"
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(summary))
    bench.ingest_pmc(str(fcsv), str(wcsv))
    assert bench.read_traffic(0) is not None
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "0" * 16)
    assert bench.read_traffic(0) is None


def test_summary_hash_covers_the_kernels_own_sources(bench, tmp_path):
    # a summary records the hash of the sources its kernel is built from, so an
    # edit to another kernel's file leaves it valid and an edit to its own does not
    q4 = "void (anonymous namespace)::gemv_q4_kernel<2, 1, true>(Q4Group)"
    fcsv, wcsv = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(fcsv, "FETCH_SIZE", [(q4, 100.0), ("copy", 524288.0)])
    _counter_csv(wcsv, "WRITE_SIZE", [(q4, 1.0), ("copy", 1048576.0)])
    summary = tmp_path / "q4.pmc.txt"
    bench.ingest_pmc(str(fcsv), str(wcsv), kernel="gemv_q4_kernel", summary=str(summary))
    d = json.loads(summary.read_text().split("\n---\n")[0])
    assert d["source_sha"] == bench.kernel_source_sha("gemv_q4")
    assert d["source_sha"] != bench.kernel_source_sha("moe_barrier_kernel")
    assert len({bench.kernel_source_sha(k) for k in ("moe_", "gemv_q4", "gemv_fp8", "gemm_fp8")}) == 4
    with pytest.raises(KeyError):
        bench.kernel_source_sha("some_other_kernel")


def test_missing_counter_summary_gives_no_traffic(bench, tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(tmp_path / "absent.txt"))
    assert bench.read_traffic(123) is None
