"""Host-side logic of bench.py (no GPU): the multi-GPU refusal and the
rocprofv3 counter summary that turns FETCH_SIZE / WRITE_SIZE into HBM bytes."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
    assert "{" not in r.stdout          # no JSON line


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def _stats_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                    "MaxNs", "StdDev"])
        for name, calls, avg_ns in rows:
            w.writerow([name, calls, calls * avg_ns, avg_ns, 0, avg_ns, avg_ns, 0])


def test_profile_summary_scales_by_the_calibration_and_keeps_the_shard_kernel_apart(
        tmp_path, monkeypatch, capsys):
    import bench
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    cal = "void at::native::vectorized_elementwise_kernel<4, at::native::CUDAFunctorOnSelf_add<float>>"
    whole = ("void cev::(anonymous namespace)::k_backward_tile<1, 256, 1, false, true>"
             "(cev_saved const*, char const*)")
    shard = ("void cev::(anonymous namespace)::k_backward_tile<1, 256, 1, true, true>"
             "(cev_saved const*, char const*)")
    rd, wr = 3_000_000, 4_000_000
    meta = {"workload": "grpo", "description": "test", "reps": 2, "kernel_source_sha": "x",
            "kernels": [dict(regex=r"^k_backward_tile<1, 256, 1, false", call="ce_backward",
                             read=rd, write=wr, roofline=True),
                        dict(regex=r"^k_backward_tile<1, 256, 1, true", call="shard",
                             read=10, write=20)]}
    json.dump(meta, open(tmp_path / "meta.json", "w"))
    # two dispatches of each; the calibration reads 2^30 B but FETCH_SIZE
    # shows half of it; WRITE_SIZE is exact
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE",
                 [(cal, 2 ** 30 / 2048), (whole, rd / 2048), (whole, rd / 2048), (shard, 7.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE",
                 [(cal, 2 ** 30 / 1024), (whole, wr / 1024), (whole, wr / 1024), (shard, 9.0)])
    _stats_csv(tmp_path / "s.csv", [(whole, 2, 1000.0), (shard, 1, 50.0), (cal, 1, 300.0)])
    bench.summarize_profile(str(tmp_path / "meta.json"), str(tmp_path / "s.csv"),
                            str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    table = capsys.readouterr().out
    assert "k_backward_tile<1, 256, 1, false, true>` (ce_backward) | 2 | 1.0 |" in table
    t = json.load(open(tmp_path / "traffic.json"))
    assert "false" in t["kernel"] and "true, true" not in t["kernel"].split("false")[0]
    assert t["read_bytes_per_launch"] == pytest.approx(rd)
    assert t["write_bytes_per_launch"] == pytest.approx(wr)
    assert t["traffic_over_algorithmic"] == pytest.approx(1.0)
    assert t["trace_average_us"] == pytest.approx(1.0)
