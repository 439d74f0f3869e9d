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
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_summary_scales_by_the_calibration_and_skips_the_shard_kernel(tmp_path,
                                                                             monkeypatch):
    import bench
    import workloads
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    cal = "void at::native::vectorized_elementwise_kernel<4, at::native::CUDAFunctorOnSelf_add<float>>"
    whole = "void cev::(anonymous namespace)::k_backward<1, 128, 2, false, true>(cev::BackwardArgs)"
    shard = "void cev::(anonymous namespace)::k_backward<1, 128, 2, true, true>(cev::BackwardArgs)"
    rows, vocab = 64, 1024
    _, labels, mask, _ = workloads.grpo_rows(rows, vocab)
    n_valid = int(((labels != -100) & (mask != 0)).sum())
    rd = n_valid * vocab * 2
    wr = rows * vocab * 2
    # the calibration reads 2^30 B but FETCH_SIZE shows half of it; WRITE_SIZE is exact
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE",
                 [(cal, 2 ** 30 / 2048), (whole, rd / 2048), (shard, 7.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE",
                 [(cal, 2 ** 30 / 1024), (whole, wr / 1024), (shard, 9.0)])
    bench.write_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), rows=rows, vocab=vocab)
    t = json.load(open(tmp_path / "traffic.json"))
    assert t["kernel"] == whole
    assert t["read_bytes_per_launch"] == pytest.approx(rd)
    assert t["write_bytes_per_launch"] == pytest.approx(wr)
    assert t["traffic_over_algorithmic"] == pytest.approx(1.0)
    assert t["kernel_source_sha"] == bench.kernel_source_hash()
