"""Host-side logic of bench.py that needs no GPU: the one-GPU guard, the rocprofv3 CSV
summary (kernel-trace percentiles, counter means per dispatch) and the traffic lookup that
turns null when the kernel sources no longer match the stored counters."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(str(v) for v in r) + "\n")


def test_rocprof_summary_percentiles_and_counters(tmp_path, capsys):
    d = tmp_path / "prof" / "host" / "1234"
    # eleven dispatches of one kernel with durations 100, 200, ..., 1100 ns, and one other kernel
    rows = [[i, "rhtq_a", 1000 * i, 1000 * i + 100 * (i + 1)] for i in range(11)]
    rows.append([11, "other", 0, 5])
    _write(str(d / "trace_kernel_trace.csv"), ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           rows)
    # a counter reported in two dimension rows per dispatch (summed per dispatch, then averaged)
    crow = [[1, "rhtq_a", "FETCH_SIZE", 10.0], [1, "rhtq_a", "FETCH_SIZE", 5.0],
            [2, "rhtq_a", "FETCH_SIZE", 20.0], [2, "rhtq_a", "FETCH_SIZE", 1.0], [3, "other", "FETCH_SIZE", 99.0]]
    _write(str(d / "pmc_counter_collection.csv"), ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
           crow)
    bench.rocprof_summary(str(tmp_path / "prof"), "rhtq")
    out = capsys.readouterr().out.splitlines()
    assert "TRACE calls 11 p10_ns 200 median_ns 600 p90_ns 1000 kernel rhtq_a" in out
    assert "PMC FETCH_SIZE mean_per_dispatch 18 dispatches 2 kernel rhtq_a" in out
    assert not any("other" in l for l in out)


def test_kernel_hash_covers_every_source():
    """Every file the library is built from enters the hash that ties stored counters to the
    kernels they were taken on."""
    csrc = os.path.join(ROOT, "randomized_hadamard_rotation_amd", "csrc")
    built = {os.path.join("randomized_hadamard_rotation_amd", "csrc", f) for f in os.listdir(csrc)}
    built.add(os.path.join("include", "rhtq.h"))
    built.add(os.path.join("randomized_hadamard_rotation_amd", "build.py"))   # the flags
    assert built <= set(bench.KERNEL_SOURCES)


def test_traffic_is_null_when_sources_changed(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    good = {"kernel_source_hash": bench.kernel_source_hash(), "hbm_bytes_per_launch": 1234}
    stale = {"kernel_source_hash": "0" * 16, "hbm_bytes_per_launch": 1234}
    (prof / "w_good_traffic.json").write_text(json.dumps(good))
    (prof / "w_stale_traffic.json").write_text(json.dumps(stale))
    src = tmp_path / "randomized_hadamard_rotation_amd" / "csrc"
    src.mkdir(parents=True)
    (tmp_path / "include").mkdir()
    for p in bench.KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            (tmp_path / p).write_bytes(f.read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_for("w_good") == 1234
    assert bench.traffic_for("w_stale") is None
    assert bench.traffic_for("w_missing") is None


@pytest.mark.parametrize("name", [bench.HEADLINE] + bench.OTHERS + [g + "_given" for g in bench.GIVEN])
def test_committed_profiles_cover_every_bench_workload(name):
    with open(os.path.join(ROOT, "profiles", f"{name}_traffic.json")) as f:
        d = json.load(f)
    assert 0.99 < d["ratio_to_algorithmic"] < 1.1
    assert os.path.exists(os.path.join(ROOT, "profiles", f"{name}_trace.md"))
