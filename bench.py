"""Throughput of the collapse-safe cross-entropy hot path on one MI355X.

One step = ce_forward (device compaction + one sweep per valid row; log p,
loss, argmax and the saved record; entropy off) followed by ce_backward (one
read of each valid row, one bf16 write of every row) on the 8192 x 152064
bf16 GRPO-shaped workload: logits 3 N(0,1) + a per-row shift U(-5, 5), labels
uniform, 819 rows masked out, g ~ N(0,1), T = 1.  Inputs are resident in HBM
before timing starts.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]

Prints one JSON line.  The roofline object describes the dominant kernel
(the backward sweep): algorithmic bytes per launch over its mean duration,
measured with HIP events on the stream the library launches on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, AMD published
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, AMD published
METRIC = "rows/s and achieved HBM GB/s (% peak), 8192x152064 bf16 fwd+bwd, 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_backward_grpo_8192x152064_bf16.json")
KERNEL_SOURCES = ["backward.hip", "cev_device.h"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "cross_entropy_vocab_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per backward launch from the committed rocprofv3 counter runs,
    if they were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


# ---------------------------------------------------------------- counters
# One workload's calls, run a few times under rocprofv3 (one counter per
# pass), and the table that turns those counter runs plus a kernel-trace run
# of the same command into per-kernel durations, bandwidth and traffic
# against algorithmic bytes.  Each kernel is matched by a regular expression
# on its name without the namespace and argument list.
COUNTER_WORKLOADS = ("grpo", "chunk", "peaked_f32", "peaked_bf16", "jsd_b0", "jsd_b05", "jsd_b1",
                     "linear", "linear_stored")


def _short_name(name):
    return name.replace("void ", "").replace("cev::(anonymous namespace)::", "").split("(")[0].strip()


def run_counter_workload(name, torch, cev, workloads, dev, reps=3):
    """Runs workload `name`'s calls `reps` times, then torch's float32 add over
    2^28 elements (2^30 bytes in, 2^30 out: the counter calibration).
    Returns the metadata the summary needs: the workload's description and
    each kernel's algorithmic bytes per launch."""
    def dev_logits(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    kernels = []
    if name == "grpo":
        w = workloads.grpo()
        R, V = w["logits"].shape
        z = dev_logits(w["logits"])
        lab, msk = torch.from_numpy(w["labels"]).to(dev), torch.from_numpy(w["row_mask"]).to(dev)
        g = torch.from_numpy(w["g"]).to(dev)
        nv = int(((w["labels"] != -100) & (w["row_mask"] != 0)).sum())
        P, Vs = 8, V // 8
        parts = torch.empty((P, R, cev.PARTIAL_BYTES), dtype=torch.uint8, device=dev)
        shard = z[:, :Vs].contiguous()
        dls = torch.empty((R, Vs), dtype=torch.bfloat16, device=dev)
        for p in range(1, P):
            cev.ce_vocab_shard_forward(z[:, p * Vs:(p + 1) * Vs], lab, p * Vs, V, 1.0, row_mask=msk,
                                       partials=parts[p])
        dl = torch.empty_like(z)
        for _ in range(reps):
            out = cev.ce_forward(z, lab, 1.0, row_mask=msk, logp=True, argmax=True)
            cev.ce_backward(z, lab, g, out["saved"], 1.0, row_mask=msk, dlogits=dl)
            cev.ce_fused(z, lab, g, 1.0, row_mask=msk, logp=True, argmax=True, dlogits=dl)
            cev.ce_vocab_shard_forward(shard, lab, 0, V, 1.0, row_mask=msk, partials=parts[0])
            mo = cev.ce_vocab_merge(parts, lab, V, 1.0, row_mask=msk, argmax=True)
            cev.ce_vocab_shard_backward(shard, lab, g, mo["saved"], 0, V, 1.0, row_mask=msk,
                                        dlogits=dls)
        desc = f"grpo-shaped {R}x{V} bf16, {nv} valid rows; one rank of 8-way vocab parallelism on {R}x{Vs}"
        kernels = [
            dict(regex=r"^k_sls_sweep<", call="ce_forward", read=nv * V * 2, write=0),
            dict(regex=r"^k_backward_tile<1, 256, 1, false", call="ce_backward",
                 read=nv * V * 2, write=R * V * 2, roofline=True),
            dict(regex=r"^k_fused_hold<", call="ce_fused", read=nv * V * 2, write=R * V * 2),
            dict(regex=r"^k_shard_sweep<", call="ce_vocab_shard_forward", read=nv * Vs * 2, write=0),
            dict(regex=r"^k_backward_tile<1, 256, 1, true", call="ce_vocab_shard_backward",
                 read=nv * Vs * 2, write=R * Vs * 2)]
    elif name == "chunk":
        w = workloads.chunk()
        R, V = w["logits"].shape
        z = dev_logits(w["logits"])
        lab, idx = torch.from_numpy(w["labels"]).to(dev), torch.from_numpy(w["indices"]).to(dev)
        gk = torch.from_numpy(np.random.default_rng(1).standard_normal(
            tuple(w["indices"].shape), dtype=np.float32)).to(dev)
        dl = torch.empty_like(z)
        for _ in range(reps):
            cev.sls_forward(z, lab, 0.7)
            lp, q, sv = cev.sls_topk_forward(z, idx, 0.7, saved=True)
            cev.sls_topk_backward(z, idx, gk, sv, q, 0.7, dlogits=dl)
        desc = f"chunked selective log-softmax {R}x{V} bf16, T = 0.7, top-8"
        kernels = [
            dict(regex=r"^k_sls_sweep<", call="sls_forward", read=R * V * 2, write=0),
            dict(regex=r"^k_topk_sweep<", call="sls_topk_forward", read=R * V * 2, write=0),
            dict(regex=r"^k_topk_backward(_tile)?<", call="sls_topk_backward", read=R * V * 2,
                 write=R * V * 2)]
    elif name in ("peaked_f32", "peaked_bf16"):
        dt = name.split("_")[1]
        w = workloads.peaked(dt)
        R, V = w["logits"].shape
        es = 2 if dt == "bf16" else 4
        z = dev_logits(w["logits"])
        lab, g = torch.from_numpy(w["labels"]).to(dev), torch.from_numpy(w["g"]).to(dev)
        dl = torch.empty_like(z)
        for _ in range(reps):
            out = cev.ce_forward(z, lab, 1.0, logp=True, entropy=True, argmax=True)
            cev.ce_backward(z, lab, g, out["saved"], 1.0, dlogits=dl)
        desc = f"peaked rows {R}x{V} {dt}, T = 1, forward with entropy and argmax"
        kernels = [
            dict(regex=r"^k_sls_sweep<", call="ce_forward", read=R * V * es, write=0),
            dict(regex=r"^k_backward_tile<", call="ce_backward", read=R * V * es, write=R * V * es)]
    elif name.startswith("jsd_"):
        beta = {"jsd_b0": 0.0, "jsd_b05": 0.5, "jsd_b1": 1.0}[name]
        w = workloads.distill()
        R, V = w["student"].shape
        st, te = dev_logits(w["student"]), dev_logits(w["teacher"])
        lab, msk = torch.from_numpy(w["labels"]).to(dev), torch.from_numpy(w["row_mask"]).to(dev)
        g = torch.from_numpy(w["g"]).to(dev)
        nv = int(((w["labels"] != -100) & (w["row_mask"] != 0)).sum())
        d = torch.empty_like(st)
        for _ in range(reps):
            out = cev.jsd_forward(st, te, 1.0, beta, labels=lab, row_mask=msk)
            cev.jsd_backward(st, te, g, out["saved"], 1.0, beta, labels=lab, row_mask=msk, dstudent=d)
        desc = f"student/teacher {R}x{V} bf16, beta = {beta:g}, {nv} valid rows"
        # the backward's bytes: both rows of each valid pair read, every
        # gradient row written (whichever of its kernels does the row)
        kernels = [
            dict(regex=r"^k_jsd_forward<", call="jsd_forward", read=2 * nv * V * 2, write=0),
            dict(regex=r"^k_jsd_(bwd_tiles|backward)<", call="jsd_backward",
                 read=2 * nv * V * 2, write=R * V * 2, per_call=True)]
    elif name in ("linear", "linear_stored"):
        R, H, V = 8192, 2560, 151936
        stored = name == "linear_stored"
        w = workloads.linear(rows=R, hidden=H, vocab=V)
        hid = torch.from_numpy(w["hidden"].view(np.int16)).to(dev).view(torch.bfloat16)
        head = torch.from_numpy(w["weight"].view(np.int16)).to(dev).view(torch.bfloat16)
        lab, msk = torch.from_numpy(w["labels"]).to(dev), torch.from_numpy(w["row_mask"]).to(dev)
        gl = torch.from_numpy(w["g"]).to(dev)
        zs = torch.empty((R, V), dtype=torch.float32, device=dev) if stored else None
        for _ in range(reps):
            out = cev.lce_forward(hid, head, lab, 1.0, row_mask=msk, argmax=True, logits=zs)
            cev.lce_backward(hid, head, lab, gl, out["saved"], 1.0, row_mask=msk,
                             workspace=out["workspace"], logits=zs)
        desc = (f"linear CE, hidden {R}x{H}, head {V}x{H} bf16, forward with argmax and the "
                f"frozen-head backward (dhidden)"
                + (", the fp32 logits stored by the forward and read back by the backward"
                   if stored else "")
                + "; bytes are each operand read once and each output written once")
        ops = R * H * 2 + V * H * 2
        nv = int(((w["labels"] != -100) & (w["row_mask"] != 0)).sum())   # rows read back
        kernels = [
            dict(regex=r"^k_lce_fwd<", call="lce_forward", read=ops,
                 write=R * V * 4 if stored else 0),
            dict(regex=r"^k_lce_dl_stored", call="lce_backward: dlogits from the stored logits",
                 read=nv * V * 4, write=R * V * 2) if stored else
            dict(regex=r"^k_lce_dl", call="lce_backward: logits again, dlogits", read=ops,
                 write=R * V * 2),
            dict(regex=r"^k_lce_gemm", call="lce_backward: dhidden, split-K partials",
                 read=R * V * 2 + V * H * 2, write=4 * R * H * 4),
            dict(regex=r"^k_splitk_reduce", call="lce_backward: split-K sum", read=4 * R * H * 4,
                 write=R * H * 4)]
    else:
        raise SystemExit(f"unknown counter workload {name!r}; one of {COUNTER_WORKLOADS}")
    src = torch.ones(2 ** 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.add(src, 1.0, out=dst)
    torch.cuda.synchronize()
    return {"workload": name, "description": desc, "reps": reps, "kernels": kernels,
            "kernel_source_sha": kernel_source_hash()}


def _stats_by_kernel(stats_csv):
    import csv
    out = {}
    with open(stats_csv) as f:
        for row in csv.DictReader(f):
            out[_short_name(row["Name"])] = dict(calls=int(row["Calls"]),
                                                 avg_us=float(row["AverageNs"]) / 1e3,
                                                 min_us=float(row["MinNs"]) / 1e3,
                                                 max_us=float(row["MaxNs"]) / 1e3,
                                                 total_us=float(row["TotalDurationNs"]) / 1e3)
    return out


def _counter_sums(csv_path, counter):
    """Sum and dispatch count of one rocprofv3 counter, by short kernel name."""
    import csv
    acc = {}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter:
                k = _short_name(row["Kernel_Name"])
                a = acc.setdefault(k, [0.0, set()])
                a[0] += float(row["Counter_Value"])
                a[1].add(row["Dispatch_Id"])
    return {k: (v[0], len(v[1])) for k, v in acc.items()}


def summarize_profile(meta_json, stats_csv, fetch_csv, write_csv):
    """Markdown summary of one counter workload: per kernel, its trace
    duration, rate on algorithmic bytes, and FETCH_SIZE / WRITE_SIZE scaled
    by the calibration copy's counters.  For the grpo workload it also writes
    the backward's traffic record that bench.py reports as roofline.traffic."""
    import re
    with open(meta_json) as f:
        meta = json.load(f)
    stats = _stats_by_kernel(stats_csv)
    fetch, write = _counter_sums(fetch_csv, "FETCH_SIZE"), _counter_sums(write_csv, "WRITE_SIZE")
    cal = [k for k in fetch if "vectorized_elementwise_kernel" in k and "_add" in k]
    if len(cal) != 1:
        raise SystemExit(f"calibration kernel not found exactly once: {cal}")
    fk, fn = fetch[cal[0]]
    wk, wn = write[cal[0]]
    f_scale = 2.0 ** 30 / (fk / fn * 1024.0)
    w_scale = 2.0 ** 30 / (wk / wn * 1024.0)
    lines = [f"Workload: {meta['description']}.", "",
             f"Calibration (torch float32 add, 2^30 B read and 2^30 B written per dispatch): "
             f"FETCH_SIZE {fk / fn:.0f} KiB, WRITE_SIZE {wk / wn:.0f} KiB per dispatch, so read "
             f"bytes = FETCH_SIZE x 1024 x {f_scale:.4f} and written bytes = WRITE_SIZE x 1024 x "
             f"{w_scale:.4f}.", "",
             "| Kernel (call) | Calls | Avg us | Min us | Algorithmic bytes | GB/s (algorithmic) | "
             "% of 8 TB/s | Read bytes (counter) | Written bytes (counter) | Counter / algorithmic |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    traffic = None
    for kinfo in meta["kernels"]:
        rx = re.compile(kinfo["regex"])
        names = [k for k in set(stats) | set(fetch) if rx.search(k)]
        if not names:
            lines.append(f"| {kinfo['regex']} ({kinfo['call']}) | 0 | - | - | - | - | - | - | - | - |")
            continue
        calls = sum(stats[k]["calls"] for k in names if k in stats)
        tot = sum(stats[k]["total_us"] for k in names if k in stats)
        mn = min(stats[k]["min_us"] for k in names if k in stats)
        # per call of the entry point: kernels matched together (e.g. the JSD
        # backward's two kernels) add up per call
        ncall = meta["reps"] if kinfo.get("per_call") else calls
        avg = tot / max(ncall, 1)
        algo = kinfo["read"] + kinfo["write"]
        gbs = algo / (avg * 1e-6) / 1e9
        rd = sum(fetch[k][0] for k in names if k in fetch) * 1024.0 * f_scale / max(ncall, 1)
        wr = sum(write[k][0] for k in names if k in write) * 1024.0 * w_scale / max(ncall, 1)
        label = " + ".join(f"`{k}`" for k in sorted(names))
        lines.append(f"| {label} ({kinfo['call']}) | {calls} | {avg:.1f} | {mn:.1f} | {algo:,} | "
                     f"{gbs:.0f} | {gbs / PEAK_HBM_GBS * 100:.1f}% | {rd:.4e} | {wr:.4e} | "
                     f"{(rd + wr) / algo:.4f} |")
        if kinfo.get("roofline"):
            traffic = dict(kernel=label, read=rd, write=wr, algo=algo, avg_us=avg)
    other = [k for k in stats if not any(re.search(ki["regex"], k) for ki in meta["kernels"])]
    if other:
        lines += ["", "Other kernels in the same process (calibration, input copies, merges):", "",
                  "| Kernel | Calls | Avg us |", "|---|---|---|"]
        lines += [f"| `{k}` | {stats[k]['calls']} | {stats[k]['avg_us']:.1f} |" for k in sorted(other)]
    print("\n".join(lines))
    if traffic is not None and meta["workload"] == "grpo":
        rec = {"kernel": traffic["kernel"], "workload": meta["description"],
               "kernel_source_sha": meta["kernel_source_sha"], "kernel_sources": KERNEL_SOURCES,
               "calibration": {"fetch_size_kib": fk / fn, "write_size_kib": wk / wn,
                               "fetch_scale": f_scale, "write_scale": w_scale},
               "read_bytes_per_launch": traffic["read"], "write_bytes_per_launch": traffic["write"],
               "bytes_per_launch": traffic["read"] + traffic["write"],
               "algorithmic_bytes_per_launch": traffic["algo"],
               "traffic_over_algorithmic": (traffic["read"] + traffic["write"]) / traffic["algo"],
               "trace_average_us": traffic["avg_us"]}
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=2)
            f.write("\n")


def bwd_bytes_all(rows, vocab, n_valid, es=2):
    """Algorithmic bytes of one ce_backward: each valid row read, every row written."""
    return n_valid * vocab * es + rows * vocab * es


def cpu_baseline(w, valid_rows, seconds=12.0, threads=None):
    """The fp64 oracle (as it stands) on a bounded sample of the same rows:
    forward (log p, loss, argmax) plus the gradient rows, chunk by chunk."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    # One GPU's share of the machine's host cores is 16 threads, whatever the
    # machine's total; the oracle uses that share (or fewer if fewer are
    # available to this process).
    threads = threads or min(16, oracle.default_threads())
    rng = np.random.default_rng(123)
    order = rng.permutation(valid_rows)
    g64 = w["g"].astype(np.float64)

    def grad_row(r):
        oracle.ce_grad_rows(w["logits"], w["labels"], g64, w["temperature"],
                            row_mask=w["row_mask"], r0=int(r), r1=int(r) + 1, threads=1)

    done = 0
    t0 = time.perf_counter()
    chunk = 2 * threads
    with ThreadPoolExecutor(threads) as ex:
        while time.perf_counter() - t0 < seconds and done < order.shape[0]:
            rows = np.sort(order[done:done + chunk])
            oracle.ce_rows(w["logits"], w["labels"], w["temperature"], row_mask=w["row_mask"],
                           rows_list=rows, threads=threads, want_entropy=False)
            list(ex.map(grad_row, rows))
            done += rows.shape[0]
    dt = time.perf_counter() - t0
    try:
        affinity = sorted(os.sched_getaffinity(0))
    except AttributeError:
        affinity = []
    return {"value": done / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "affinity_cpus": len(affinity),
            "affinity": _cpu_ranges(affinity),
            "threads_note": "capped at 16 threads, one GPU's share of the host's cores",
            "sample": f"{done} random valid rows of the 8192x152064 bf16 workload "
                      f"(forward with argmax + full gradient row each), {dt:.1f} s wall"}


def _cpu_ranges(cpus):
    """'0-15,32-47' style text for a sorted list of CPU ids."""
    out, i = [], 0
    while i < len(cpus):
        j = i
        while j + 1 < len(cpus) and cpus[j + 1] == cpus[j] + 1:
            j += 1
        out.append(f"{cpus[i]}" if i == j else f"{cpus[i]}-{cpus[j]}")
        i = j + 1
    return ",".join(out)


def bench_linear(args, torch, cev, workloads, dev):
    """lce_forward and lce_backward (frozen head: dhidden only) on the
    8192 x 2560 x 151936 bf16 shape; FLOP counts are the products' 2 R H V
    (forward) and 2 x 2 R H V (backward: logits recomputed, then dhidden)."""
    R, H, Vl = 8192, 2560, 151936
    log(f"[bench] linear CE: generating {R}x{H} hidden, {Vl}x{H} head")
    w = workloads.linear(rows=R, hidden=H, vocab=Vl)
    hid = torch.from_numpy(w["hidden"].view(np.int16)).to(dev).view(torch.bfloat16)
    head = torch.from_numpy(w["weight"].view(np.int16)).to(dev).view(torch.bfloat16)
    lab = torch.from_numpy(w["labels"]).to(dev)
    msk = torch.from_numpy(w["row_mask"]).to(dev)
    gl = torch.from_numpy(w["g"]).to(dev)
    out = cev.lce_forward(hid, head, lab, 1.0, row_mask=msk, argmax=True)
    dh, _ = cev.lce_backward(hid, head, lab, gl, out["saved"], 1.0, row_mask=msk,
                             workspace=out["workspace"])
    steps = max(2, args.steps // 4)
    for _ in range(max(1, args.warmup // 2)):
        cev.lce_forward(hid, head, lab, 1.0, row_mask=msk, argmax=True, out=out)
        cev.lce_backward(hid, head, lab, gl, out["saved"], 1.0, row_mask=msk,
                         workspace=out["workspace"], dhidden=dh)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record()
        cev.lce_forward(hid, head, lab, 1.0, row_mask=msk, argmax=True, out=out)
        e1.record()
        cev.lce_backward(hid, head, lab, gl, out["saved"], 1.0, row_mask=msk,
                         workspace=out["workspace"], dhidden=dh)
        e2.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    f_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    b_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev]))
    flop = 2.0 * R * H * Vl
    # the forward alone at 2048 rows, the other row count of the same head
    r2 = 2048
    o2 = cev.lce_forward(hid[:r2], head, lab[:r2], 1.0, row_mask=msk[:r2], argmax=True)
    e2 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    cev.lce_forward(hid[:r2], head, lab[:r2], 1.0, row_mask=msk[:r2], argmax=True, out=o2)
    e2[0].record()
    for _ in range(steps):
        cev.lce_forward(hid[:r2], head, lab[:r2], 1.0, row_mask=msk[:r2], argmax=True, out=o2)
    e2[1].record()
    torch.cuda.synchronize()
    f2_ms = e2[0].elapsed_time(e2[1]) / steps
    del o2
    log(f"[bench] linear CE: forward {f_ms:.2f} ms, backward {b_ms:.2f} ms; "
        f"forward at {r2} rows {f2_ms:.2f} ms")
    # Memory for time: the forward also stores the fp32 logits (R x V x 4
    # bytes), and the backward reads them back instead of recomputing them.
    zs = torch.empty((R, Vl), dtype=torch.float32, device=dev)
    sf_ms, sb_ms = _time_calls(torch, [
        lambda i: cev.lce_forward(hid, head, lab, 1.0, row_mask=msk, argmax=True, out=out,
                                  logits=zs),
        lambda i: cev.lce_backward(hid, head, lab, gl, out["saved"], 1.0, row_mask=msk,
                                   workspace=out["workspace"], dhidden=dh, logits=zs)], steps)
    zbytes = R * Vl * 4
    stored = {"entry": "lce_forward(logits=) + lce_backward(logits=): fp32 logits kept in HBM",
              "logits_bytes": zbytes, "forward_ms": sf_ms, "backward_ms": sb_ms,
              "step_ms": sf_ms + sb_ms, "rows_per_s": R / ((sf_ms + sb_ms) / 1e3),
              "forward_TFLOPs": flop / (sf_ms / 1e3) / 1e12,
              "backward_TFLOPs": flop / (sb_ms / 1e3) / 1e12}
    del zs
    log(f"[bench] linear CE, stored logits: forward {sf_ms:.2f} ms, backward {sb_ms:.2f} ms")
    # A trainable head: the backward also forms dhead = dlogits^T x hidden
    # (one more 2 R H V product), logits recomputed.
    dwt = torch.empty((Vl, H), dtype=torch.float32, device=dev)
    (tb_ms,) = _time_calls(torch, [
        lambda i: cev.lce_backward(hid, head, lab, gl, out["saved"], 1.0, row_mask=msk,
                                   workspace=out["workspace"], dhidden=dh, dweight=dwt)], steps)
    del dwt
    trainable = {"entry": "lce_backward(dweight=True): dlogits, dhidden and dhead",
                 "backward_ms": tb_ms, "backward_TFLOPs": 3 * flop / (tb_ms / 1e3) / 1e12}
    log(f"[bench] linear CE, trainable head: backward {tb_ms:.2f} ms")
    res = {"entry": "lce_forward + lce_backward (frozen head: dhidden only), logits never "
                    "stored; 2560 x 151936 head as in the unsloth-zoo #2080 Speed section",
           "shape": {"rows": R, "hidden": H, "vocab": Vl}, "steps": steps,
           "ms_per_step": wall, "rows_per_s": R / (wall / 1e3),
           "forward_ms": f_ms, "backward_ms": b_ms,
           "forward_TFLOPs": flop / (f_ms / 1e3) / 1e12,
           "backward_TFLOPs": 2 * flop / (b_ms / 1e3) / 1e12,
           "step_TFLOPs": 3 * flop / ((f_ms + b_ms) / 1e3) / 1e12,
           "forward_2048_rows_ms": f2_ms,
           "forward_2048_rows_TFLOPs": flop * r2 / R / (f2_ms / 1e3) / 1e12,
           "stored_logits": stored,
           "trainable_head": trainable,
           "roofline": {"bound": "mfma", "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "achieved": 3 * flop / ((f_ms + b_ms) / 1e3) / 1e12,
                        "frac": 3 * flop / ((f_ms + b_ms) / 1e3) / 1e12 / PEAK_BF16_TFLOPS}}
    del hid, head, out, dh
    torch.cuda.empty_cache()
    return res


def bench_jsd(args, torch, cev, workloads, dev):
    """jsd_forward + jsd_backward on the 2048 x 151936 bf16 student/teacher
    pair at beta 0, 0.5 and 1.  Algorithmic bytes: the forward reads each
    valid row of both matrices once; the backward reads them once more and
    writes every gradient row."""
    log("[bench] jsd: generating 2048x151936 bf16 student and teacher")
    w = workloads.distill()
    R, V = w["student"].shape
    st = torch.from_numpy(w["student"].view(np.int16)).to(dev).view(torch.bfloat16)
    te = torch.from_numpy(w["teacher"].view(np.int16)).to(dev).view(torch.bfloat16)
    lab = torch.from_numpy(w["labels"]).to(dev)
    msk = torch.from_numpy(w["row_mask"]).to(dev)
    g = torch.from_numpy(w["g"]).to(dev)
    n_valid = int(((w["labels"] != -100) & (w["row_mask"] != 0)).sum())
    fwd_bytes = 2 * n_valid * V * 2
    bwd_bytes = 2 * n_valid * V * 2 + R * V * 2
    steps = max(3, args.steps // 2)
    res = {"entry": "jsd_forward + jsd_backward (student gradient), 2048 x 151936 bf16 "
                    "student/teacher rows as in the unsloth-zoo #2079 Numbers",
           "shape": {"rows": R, "vocab": V, "valid_rows": n_valid},
           "algorithmic_bytes": {"forward": fwd_bytes, "backward": bwd_bytes}}
    dl = torch.empty_like(st)
    for beta in (0.0, 0.5, 1.0):
        out = cev.jsd_forward(st, te, 1.0, beta, labels=lab, row_mask=msk)
        t_end = time.perf_counter() + 0.05          # warm up for 50 ms (GPU clocks)
        while time.perf_counter() < t_end:
            cev.jsd_forward(st, te, 1.0, beta, labels=lab, row_mask=msk, out=out)
            cev.jsd_backward(st, te, g, out["saved"], 1.0, beta, labels=lab, row_mask=msk,
                             dstudent=dl)
            torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        for e0, e1, e2 in ev:
            e0.record()
            cev.jsd_forward(st, te, 1.0, beta, labels=lab, row_mask=msk, out=out)
            e1.record()
            cev.jsd_backward(st, te, g, out["saved"], 1.0, beta, labels=lab, row_mask=msk,
                             dstudent=dl)
            e2.record()
        torch.cuda.synchronize()
        f_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
        b_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev]))
        res[f"beta_{beta:g}"] = {"forward_ms": f_ms, "backward_ms": b_ms,
                                 "forward_GBps": fwd_bytes / (f_ms / 1e3) / 1e9,
                                 "backward_GBps": bwd_bytes / (b_ms / 1e3) / 1e9,
                                 "rows_per_s": R / ((f_ms + b_ms) / 1e3)}
        log(f"[bench] jsd beta={beta:g}: forward {f_ms:.3f} ms, backward {b_ms:.3f} ms")
    # the backward at beta = 0 (k_jsd_bwd_tiles) is bound by HBM; the
    # forwards and the backward in between are bound by VALU issue
    bb = res["beta_0"]
    res["roofline"] = {"bound": "hbm", "kernel": "k_jsd_bwd_tiles (beta 0)", "unit": "GB/s",
                       "achieved": bb["backward_GBps"], "peak": PEAK_HBM_GBS,
                       "frac": bb["backward_GBps"] / PEAK_HBM_GBS,
                       "valu_bound": ["k_jsd_forward (every beta)",
                                      "k_jsd_bwd_tiles (0 < beta < 1)"]}
    del st, te, dl
    torch.cuda.empty_cache()
    return res


def _time_calls(torch, calls, iters, warmup_s=0.05):
    """Mean GPU time in ms of each call in `calls` (functions of the iteration
    index): each call runs iters times back to back between two HIP events
    recorded on the library's stream, as a training or serving loop issues
    it, so the time includes the dispatch gaps between its own launches but
    no host work.  The calls first run in order, back to back, for at least
    warmup_s seconds: after the host-side input generation the GPU has idled,
    and its clocks take a while to come back up."""
    t_end = time.perf_counter() + warmup_s
    n = 0
    while n < 3 or time.perf_counter() < t_end:
        for c in calls:
            c(n)
        torch.cuda.synchronize()
        n += 1
    out = []
    for c in calls:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(iters):
            c(i)
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / iters)
    return out


def bench_configs(args, torch, cev, workloads, dev):
    """The other workloads of the scope table, timed on their own entry
    points: the tiny and sparse-supervision cases (launch-bound, in us), the
    chunked selective log-softmax and its top-K form on 4096 x 32768 bf16
    (three input copies in rotation, so the 256 MB Infinity Cache cannot hold
    the next call's input), and the peaked-row stress rows in fp32 and bf16 at
    T = 1 and 0.9 (forward with entropy and argmax, then the backward)."""
    iters = max(10, args.steps)
    res = {}

    def dev_logits(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    for name, w in (("tiny_64x4096_f32", workloads.tiny()),
                    ("sparse_1922x4096_f32", workloads.sparse())):
        z = dev_logits(w["logits"])
        lab = torch.from_numpy(w["labels"]).to(dev)
        g = torch.from_numpy(w["g"]).to(dev)
        T = w["temperature"]
        out = cev.ce_forward(z, lab, T, logp=True, argmax=True)
        dl = torch.empty_like(z)
        f, b = _time_calls(torch, [
            lambda i: cev.ce_forward(z, lab, T, logp=True, argmax=True, out=out),
            lambda i: cev.ce_backward(z, lab, g, out["saved"], T, dlogits=dl)], iters)
        res[name] = {"calls": "ce_forward (compaction + sweep) + ce_backward",
                     "valid_rows": int(out["n_valid"].item()),
                     "ce_forward_us": f * 1e3, "ce_backward_us": b * 1e3}
        log(f"[bench] {name}: forward {f * 1e3:.1f} us, backward {b * 1e3:.1f} us")

    # Few long rows: ce_forward splits each row over several workgroups and
    # merges their partial records (the workspace the binding allocates holds
    # them).
    w = workloads.grpo(rows=8)
    z = dev_logits(w["logits"])
    lab = torch.from_numpy(w["labels"]).to(dev)
    out = cev.ce_forward(z, lab, 1.0, logp=True, argmax=True)
    (f,) = _time_calls(torch, [lambda i: cev.ce_forward(z, lab, 1.0, logp=True, argmax=True,
                                                         out=out)], iters)
    nb = z.shape[0] * z.shape[1] * 2
    res["split_8x152064_bf16"] = {"calls": "ce_forward (split rows: partial records + merge)",
                                  "ce_forward_us": f * 1e3,
                                  "ce_forward_GBps": nb / (f / 1e3) / 1e9}
    log(f"[bench] split 8 rows: ce_forward {f * 1e3:.1f} us")
    del z

    w = workloads.chunk()
    R, V = w["logits"].shape
    copies = [dev_logits(w["logits"])]
    copies += [copies[0].clone() for _ in range(2)]
    lab = torch.from_numpy(w["labels"]).to(dev)
    idx = torch.from_numpy(w["indices"]).to(dev)
    T = w["temperature"]
    gk = torch.from_numpy(np.random.default_rng(1).standard_normal(
        tuple(w["indices"].shape), dtype=np.float32)).to(dev)
    tk = cev.sls_topk_forward(copies[0], idx, T, saved=True)
    dl = torch.empty_like(copies[0])
    f, k, kb = _time_calls(torch, [
        lambda i: cev.sls_forward(copies[i % 3], lab, T),
        lambda i: cev.sls_topk_forward(copies[(i + 1) % 3], idx, T),
        lambda i: cev.sls_topk_backward(copies[0], idx, gk, tk[2], tk[1], T, dlogits=dl)], iters)
    nbytes = R * V * 2
    res["chunk_4096x32768_bf16"] = {
        "calls": "sls_forward (T = 0.7); sls_topk_forward (K = 8); sls_topk_backward (K = 8, "
                 "g ~ N(0, 1) per index)", "bytes_per_call": nbytes,
        "ideal_us_at_peak": nbytes / PEAK_HBM_GBS / 1e3,
        "sls_forward_us": f * 1e3, "sls_forward_GBps": nbytes / (f / 1e3) / 1e9,
        "sls_topk_forward_us": k * 1e3, "sls_topk_forward_GBps": nbytes / (k / 1e3) / 1e9,
        "sls_topk_backward_us": kb * 1e3,
        "sls_topk_backward_GBps": 2 * nbytes / (kb / 1e3) / 1e9}
    log(f"[bench] chunk: sls_forward {f * 1e3:.1f} us, sls_topk_forward {k * 1e3:.1f} us, "
        f"sls_topk_backward {kb * 1e3:.1f} us")
    del copies, dl

    for dt in ("f32", "bf16"):
        w = workloads.peaked(dt)
        R, V = w["logits"].shape
        ES = 2 if dt == "bf16" else 4
        z = dev_logits(w["logits"])
        lab = torch.from_numpy(w["labels"]).to(dev)
        g = torch.from_numpy(w["g"]).to(dev)
        dl = torch.empty_like(z)
        for T in (1.0, 0.9):
            out = cev.ce_forward(z, lab, T, logp=True, entropy=True, argmax=True)
            f, b = _time_calls(torch, [
                lambda i: cev.ce_forward(z, lab, T, logp=True, entropy=True, argmax=True,
                                         out=out),
                lambda i: cev.ce_backward(z, lab, g, out["saved"], T, dlogits=dl)], iters)
            fb, bb = R * V * ES, 2 * R * V * ES
            res[f"peaked_{R}x{V}_{dt}_T{T:g}"] = {
                "calls": "ce_forward (entropy, argmax) + ce_backward",
                "ce_forward_us": f * 1e3, "ce_backward_us": b * 1e3,
                "ce_forward_GBps": fb / (f / 1e3) / 1e9, "ce_backward_GBps": bb / (b / 1e3) / 1e9,
                "step_frac_of_peak": (fb + bb) / ((f + b) / 1e3) / 1e9 / PEAK_HBM_GBS}
            log(f"[bench] peaked {dt} T={T:g}: forward {f * 1e3:.1f} us, backward {b * 1e3:.1f} us")
        del z, dl
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="back-to-back steps for at least this long before the counted warmup")
    ap.add_argument("--rows", type=int, default=8192)
    ap.add_argument("--vocab", type=int, default=152064)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain elementwise kernel over 1 GiB in / 1 GiB out, "
                         "the reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--no-jsd", action="store_true",
                    help="skip the student/teacher JSD measurement (2048 x 151936)")
    ap.add_argument("--no-linear", action="store_true",
                    help="skip the linear cross-entropy measurement (8192 x 2560 x 151936)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (tiny, chunked + top-K, sparse, peaked)")
    ap.add_argument("--counters", choices=COUNTER_WORKLOADS,
                    help="run only this workload's calls (for rocprofv3 counter and trace "
                         "passes) and write its metadata to --counter-meta")
    ap.add_argument("--counter-meta", default=None,
                    help="metadata file written by --counters and read by --summarize")
    ap.add_argument("--summarize", nargs=3, metavar=("STATS_CSV", "FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: print the markdown summary of a counter workload from "
                         "its kernel-trace stats and its FETCH_SIZE and WRITE_SIZE runs")
    args = ap.parse_args()
    if args.summarize:
        summarize_profile(args.counter_meta, *args.summarize)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(rows shard across GPUs with no communication inside the op).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import cross_entropy_vocab_amd as cev
    import workloads

    dev = torch.device("cuda:0")
    if args.counters:
        meta = run_counter_workload(args.counters, torch, cev, workloads, dev)
        if args.counter_meta:
            with open(args.counter_meta, "w") as f:
                json.dump(meta, f, indent=2)
        print(json.dumps({"counters": args.counters, "kernels": len(meta["kernels"])}))
        return
    log(f"[bench] generating {args.rows}x{args.vocab} bf16 workload")
    w = workloads.grpo(rows=args.rows, vocab=args.vocab)
    R, V = w["logits"].shape
    logits = torch.from_numpy(w["logits"].view(np.int16)).to(dev).view(torch.bfloat16)
    labels = torch.from_numpy(w["labels"]).to(dev)
    mask = torch.from_numpy(w["row_mask"]).to(dev)
    g = torch.from_numpy(w["g"]).to(dev)
    T = w["temperature"]
    n_valid = int(((w["labels"] != -100) & (w["row_mask"] != 0)).sum())
    out = cev.ce_forward(logits, labels, T, row_mask=mask, logp=True, argmax=True)
    dl = torch.empty((R, V), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step():
        cev.ce_forward(logits, labels, T, row_mask=mask, logp=True, argmax=True, out=out)
        cev.ce_backward(logits, labels, g, out["saved"], T, row_mask=mask, dlogits=dl)

    # The GPU idled during the host-side input generation and its clocks take
    # a while to come back: settle them with back-to-back steps (synchronized
    # every 10) for at least --settle-ms before the counted warmup.
    log(f"[bench] settling clocks for {args.settle_ms:.0f} ms, then warmup {args.warmup}")
    t_settle = time.perf_counter()
    settle_steps = 0
    while settle_steps < 10 or (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        step()
        settle_steps += 1
        if settle_steps % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(out["n_valid"].item()) == n_valid

    # K back-to-back steps timed by the wall clock between synchronizations
    # (value); the same K steps again with HIP events recorded on the
    # library's stream (torch's current stream) between the calls, for the
    # per-call times (the host runs ahead of the GPU, so each event pair
    # brackets one call's kernels plus the short dispatch gap); then the K
    # steps once more by the wall clock, an A/A rerun whose gap to the first
    # is the run-to-run noise.
    def timed_steps():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps * 1e3

    log(f"[bench] timing {args.steps} steps")
    ms_step = timed_steps()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e0, e1, e2 in ev:
        e0.record()
        cev.ce_forward(logits, labels, T, row_mask=mask, logp=True, argmax=True, out=out)
        e1.record()
        cev.ce_backward(logits, labels, g, out["saved"], T, row_mask=mask, dlogits=dl)
        e2.record()
    torch.cuda.synchronize()
    fwd_ms = [e0.elapsed_time(e1) for e0, e1, _ in ev]
    bwd_ms = [e1.elapsed_time(e2) for _, e1, e2 in ev]
    fwd = float(np.mean(fwd_ms))
    bwd = float(np.mean(bwd_ms))
    ms_step_aa = timed_steps()

    # Scrub A/B for the backward: the same call timed right after ce_forward
    # (as in the step), after a 1 GiB read that leaves none of the logits in
    # the 256 MB Infinity Cache (a read, so that no dirty lines of the scrub
    # itself are written back during the backward), after that scrub and then
    # ce_forward, and right after another ce_backward.  The scrubbed time is
    # the backward's rate from HBM alone.
    scrub = torch.ones(2 ** 28, dtype=torch.float32, device=dev)
    conds = ("after_forward", "after_scrub", "after_scrub_then_forward", "after_backward")
    scrub_ab = {k: [] for k in conds}
    for i in range(len(conds) * max(4, args.steps // 2)):
        key = conds[i % len(conds)]
        if key in ("after_scrub", "after_scrub_then_forward"):
            scrub_sum = scrub.sum()
        if key in ("after_forward", "after_scrub_then_forward"):
            cev.ce_forward(logits, labels, T, row_mask=mask, logp=True, argmax=True, out=out)
        if key == "after_backward":
            cev.ce_backward(logits, labels, g, out["saved"], T, row_mask=mask, dlogits=dl)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cev.ce_backward(logits, labels, g, out["saved"], T, row_mask=mask, dlogits=dl)
        e1.record()
        torch.cuda.synchronize()
        scrub_ab[key].append(e0.elapsed_time(e1))
    del scrub, scrub_sum
    scrub_ab = {k: float(np.median(v)) for k, v in scrub_ab.items()}
    scrub_ab["scrub"] = "1 GiB float32 read (torch sum)"
    scrub_ab["hbm_only_GBps"] = bwd_bytes_all(R, V, n_valid) / (scrub_ab["after_scrub"] / 1e3) / 1e9

    # The same step as one call (g known up front): ce_fused.
    fout = cev.ce_fused(logits, labels, g, T, row_mask=mask, logp=True, argmax=True,
                        dlogits=dl)
    for _ in range(args.warmup):
        cev.ce_fused(logits, labels, g, T, row_mask=mask, logp=True, argmax=True, out=fout)
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in fev:
        e0.record()
        cev.ce_fused(logits, labels, g, T, row_mask=mask, logp=True, argmax=True, out=fout)
        e1.record()
    torch.cuda.synchronize()
    fused_wall = (time.perf_counter() - t0) / args.steps * 1e3
    fused_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in fev]))

    # One rank's share of an 8-way vocab-parallel step: its contiguous
    # [R, V/8] shard, the shard sweep, the merge of all 8 shards' records
    # (the other 7 made once, untimed, standing in for the all-gather), and
    # the shard backward.
    P = 8
    Vs = V // P
    shard = logits[:, :Vs].contiguous()
    parts = torch.empty((P, R, cev.PARTIAL_BYTES), dtype=torch.uint8, device=dev)
    for p in range(1, P):
        cev.ce_vocab_shard_forward(logits[:, p * Vs:(p + 1) * Vs], labels, p * Vs, V, T,
                                   row_mask=mask, partials=parts[p])
    dls = torch.empty((R, Vs), dtype=torch.bfloat16, device=dev)

    def shard_step(ev=None):
        if ev:
            ev[0].record()
        cev.ce_vocab_shard_forward(shard, labels, 0, V, T, row_mask=mask, partials=parts[0])
        if ev:
            ev[1].record()
        mo = cev.ce_vocab_merge(parts, labels, V, T, row_mask=mask, argmax=True)
        if ev:
            ev[2].record()
        cev.ce_vocab_shard_backward(shard, labels, g, mo["saved"], 0, V, T, row_mask=mask,
                                    dlogits=dls)
        if ev:
            ev[3].record()

    for _ in range(args.warmup):
        shard_step()
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in sev:
        shard_step(e)
    torch.cuda.synchronize()
    shard_wall = (time.perf_counter() - t0) / args.steps * 1e3
    s_fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in sev]))
    s_mrg = float(np.mean([e[1].elapsed_time(e[2]) for e in sev]))
    s_bwd = float(np.mean([e[2].elapsed_time(e[3]) for e in sev]))
    del shard, dls, parts

    del logits, dl, out, fout
    torch.cuda.empty_cache()
    linear = None if args.no_linear else bench_linear(args, torch, cev, workloads, dev)
    jsd = None if args.no_jsd else bench_jsd(args, torch, cev, workloads, dev)
    configs = None if args.no_configs else bench_configs(args, torch, cev, workloads, dev)

    ES = 2
    fwd_bytes = n_valid * V * ES                    # valid rows read once
    bwd_bytes = n_valid * V * ES + R * V * ES       # valid rows re-read, every row written
    step_bytes = fwd_bytes + bwd_bytes
    rows_per_s = R / (ms_step / 1e3)
    achieved = bwd_bytes / (bwd / 1e3) / 1e9
    traffic = measured_traffic()
    res = {
        "metric": METRIC,
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"grpo-shaped {R}x{V} bf16 logits, {R - n_valid} rows masked, "
                               "ce_forward (argmax, no entropy) + ce_backward, T=1",
                   "rows": R, "vocab": V, "valid_rows": n_valid},
        "hbm_GBps": step_bytes / (ms_step / 1e3) / 1e9,
        "hbm_frac_of_peak": step_bytes / (ms_step / 1e3) / 1e9 / PEAK_HBM_GBS,
        "step_algorithmic_bytes": step_bytes,
        "aa_rerun": {"ms_per_step": ms_step_aa,
                     "relative_difference": (ms_step_aa - ms_step) / ms_step},
        "clock_settle": {"ms": settle_ms, "steps": settle_steps,
                         "note": "back-to-back steps before the counted warmup"},
        "backward_scrub_ab_ms": scrub_ab,
        "kernels_ms": {"ce_forward": fwd, "ce_backward": bwd,
                       "ce_forward_median": float(np.median(fwd_ms)),
                       "ce_forward_p10_p90": [float(np.percentile(fwd_ms, 10)),
                                              float(np.percentile(fwd_ms, 90))],
                       "ce_backward_median": float(np.median(bwd_ms)),
                       "ce_backward_p10_p90": [float(np.percentile(bwd_ms, 10)),
                                               float(np.percentile(bwd_ms, 90))],
                       "ce_backward_min": float(np.min(bwd_ms)),
                       "ce_backward_max": float(np.max(bwd_ms)),
                       "ce_forward_GBps": fwd_bytes / (fwd / 1e3) / 1e9,
                       "ce_backward_GBps": achieved},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "k_backward_tile (ce_backward)", "bytes_per_launch": bwd_bytes},
        "cpu_baseline": None,
        "fused": {"entry": "ce_fused: the same outputs in one call for a g known up front; "
                           "each valid row swept once, 43% of it held on chip and the rest "
                           "read again at once, every dlogits row written once",
                  "ms_per_step": fused_wall, "kernel_ms": fused_ms,
                  "rows_per_s": R / (fused_wall / 1e3),
                  "algorithmic_bytes": fwd_bytes + R * V * ES,
                  "GBps": (fwd_bytes + R * V * ES) / (fused_ms / 1e3) / 1e9,
                  "frac_of_peak": (fwd_bytes + R * V * ES) / (fused_ms / 1e3) / 1e9 / PEAK_HBM_GBS},
        "linear_ce": linear,
        "jsd": jsd,
        "configs": configs,
        "vocab_shard": {"entry": f"one rank of {P}-way vocab parallelism: "
                                 "ce_vocab_shard_forward on its contiguous shard, ce_vocab_merge "
                                 f"of {P} shards' records, ce_vocab_shard_backward",
                        "shard": [R, Vs], "ms_per_step": shard_wall,
                        "kernels_ms": {"shard_forward": s_fwd, "merge": s_mrg,
                                       "shard_backward": s_bwd},
                        "shard_forward_GBps": n_valid * Vs * ES / (s_fwd / 1e3) / 1e9,
                        "shard_backward_GBps": (n_valid + R) * Vs * ES / (s_bwd / 1e3) / 1e9},
    }
    log(f"[bench] {ms_step:.3f} ms/step (A/A rerun {ms_step_aa:.3f}), fwd {fwd:.3f} ms, bwd {bwd:.3f} ms; "
        f"fused {fused_wall:.3f} ms/step; vocab shard {shard_wall:.3f} ms/step "
        f"(fwd {s_fwd:.3f}, merge {s_mrg:.3f}, bwd {s_bwd:.3f})")
    if args.copy_calibration:
        # torch's elementwise add: reads exactly 2^30 bytes, writes exactly 2^30 bytes
        src = torch.ones(2 ** 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.add(src, 1.0, out=dst)
        torch.cuda.synchronize()
        res["copy_calibration"] = {"kernel": "torch elementwise add (float32)",
                                   "read_bytes": 2 ** 30, "write_bytes": 2 ** 30}
        del src, dst
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)")
        vr = np.flatnonzero((w["labels"] != -100) & (w["row_mask"] != 0))
        res["cpu_baseline"] = cpu_baseline(w, vr, seconds=args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
