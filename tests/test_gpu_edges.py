"""Edge cases of the HIP path against the oracle: tiny and odd vocabularies,
misaligned and padded rows, empty inputs, all-ignored and bad labels, argmax
ties, top-K duplicates and ignored entries, determinism, guard bands."""
import numpy as np
import pytest
import torch

import cross_entropy_vocab_amd as cev
import oracle
import workloads
from tolerance import RTOL, assert_close, assert_nonpositive, assert_row_sums

pytestmark = pytest.mark.gpu


def _rand_case(rows, V, dtype="f32", T=1.0, seed=0, scale=3.0, n_ignored=0, mask_frac=0.0):
    rng = np.random.default_rng(seed)
    z = (rng.standard_normal((rows, V)) * scale).astype(np.float32)
    logits = workloads.bf16_bits(z) if dtype == "bf16" else z
    labels = rng.integers(0, V, rows).astype(np.int64)
    if n_ignored:
        labels[rng.permutation(rows)[:n_ignored]] = -100
    mask = None
    if mask_frac:
        mask = (rng.random(rows) >= mask_frac).astype(np.uint8)
    g = rng.standard_normal(rows).astype(np.float32)
    return dict(logits=logits, labels=labels, row_mask=mask, temperature=T, g=g)


def _check_against_oracle(w, got, name):
    kind = "bf16" if w["logits"].dtype == np.uint16 else "f32"
    tol = RTOL[kind]
    V = w["logits"].shape[1]
    ref = oracle.ce_rows(w["logits"], w["labels"], w["temperature"], row_mask=w.get("row_mask"))
    dref = oracle.ce_grad_rows(w["logits"], w["labels"], np.asarray(w["g"], np.float64),
                               w["temperature"], row_mask=w.get("row_mask"))
    vr, _ = oracle.valid_rows(w["labels"], w.get("row_mask"), V)
    n = int(got["n_valid"][0])
    assert n == vr.shape[0] and np.array_equal(got["valid_rows"][:n], vr), name
    assert_close(f"{name} logp", got["logp"], ref["logp"], tol["logp"])
    assert_close(f"{name} loss", got["loss"], ref["loss"], tol["loss"])
    assert_close(f"{name} entropy", got["entropy"], ref["entropy"], tol["entropy"], 1e-30)
    assert np.array_equal(got["argmax"], ref["argmax"]), name
    valid = np.zeros(w["logits"].shape[0], dtype=bool)
    valid[vr] = True
    assert_nonpositive(name, got["logp"], valid)
    assert_close(f"{name} dlogits", got["dlogits"], dref, tol["dlogits"], 2.0 ** -126)
    assert_row_sums(f"{name} dlogits", got["dlogits"], tol["dlogits"])


@pytest.mark.parametrize("V", [1, 2, 3, 5, 7, 8, 9, 15, 16, 17, 31, 33, 63, 64, 65, 127, 511,
                               512, 513, 1023, 2049, 4097])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_and_odd_vocab(V, dtype):
    from gpu_helpers import run_ce
    w = _rand_case(9, V, dtype, T=0.8, seed=V, n_ignored=2)
    got = run_ce(w)
    _check_against_oracle(w, got, f"V={V} {dtype}")
    if V == 1:
        valid = w["labels"] != -100
        assert np.all(got["logp"][valid] == 0) and np.all(np.signbit(got["logp"][valid]))
        assert np.all(got["dlogits"] == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V,stride", [(1000, 1003), (4093, 4100), (32768, 32775), (777, 777)])
def test_padded_and_misaligned_rows(dtype, V, stride):
    """Row starts at every alignment modulo 16 bytes; padding holds NaN
    canaries that must not leak into any output."""
    from gpu_helpers import DEV, run_ce, strided_dev
    w = _rand_case(11, V, dtype, seed=stride, n_ignored=1)
    dev = strided_dev(w["logits"], stride)
    got = run_ce(w, logits_dev=dev)
    _check_against_oracle(w, got, f"V={V} stride={stride} {dtype}")


def test_dlogits_padded_stride_untouched():
    from gpu_helpers import DEV, to_dev
    w = _rand_case(6, 300, "bf16", seed=3)
    logits = to_dev(w["logits"])
    labels = to_dev(w["labels"])
    g = to_dev(w["g"])
    out = cev.ce_forward(logits, labels, 1.0)
    big = torch.full((6, 307), 12345, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    dl = big[:, :300]
    cev.ce_backward(logits, labels, g, out["saved"], 1.0, dlogits=dl)
    ref = cev.ce_backward(logits, labels, g, out["saved"], 1.0)
    torch.cuda.synchronize()
    assert torch.equal(dl.view(torch.int16), ref.view(torch.int16))
    assert torch.all(big.view(torch.int16)[:, 300:] == 12345)


def test_empty_rows():
    from gpu_helpers import DEV
    logits = torch.empty((0, 100), dtype=torch.float32, device=DEV)
    labels = torch.empty(0, dtype=torch.int64, device=DEV)
    out = cev.ce_forward(logits, labels, 1.0)
    assert out["loss"].shape == (0,)
    dl = cev.ce_backward(logits, labels, torch.empty(0, device=DEV), out["saved"], 1.0)
    assert dl.shape == (0, 100)
    assert cev.sls_forward(logits, labels)["logp"].shape == (0,)
    idx = torch.empty((0, 4), dtype=torch.int64, device=DEV)
    assert cev.sls_topk_forward(logits, idx).shape == (0, 4)


def test_all_rows_ignored():
    from gpu_helpers import run_ce
    w = _rand_case(20, 5000, "bf16", seed=5, n_ignored=20)
    got = run_ce(w)
    assert int(got["n_valid"][0]) == 0
    assert np.all(got["loss"] == 0) and np.all(got["logp"] == 0)
    assert np.all(got["argmax"] == -1) and np.all(got["dlogits"] == 0)


def test_all_rows_masked_and_mixed_mask():
    from gpu_helpers import run_ce
    w = _rand_case(40, 3000, "f32", seed=6, mask_frac=0.5, n_ignored=5)
    got = run_ce(w)
    _check_against_oracle(w, got, "mixed mask")
    w["row_mask"][:] = 0
    got = run_ce(w)
    assert int(got["n_valid"][0]) == 0 and np.all(got["dlogits"] == 0)


def test_bad_labels_set_status_and_are_ignored():
    from gpu_helpers import run_ce, run_sls
    w = _rand_case(12, 700, "f32", seed=7)
    w["labels"][3] = 700
    w["labels"][8] = -5
    got = run_ce(w)
    assert got["status"] & cev.STATUS_BAD_LABEL
    _check_against_oracle(w, got, "bad labels")
    assert got["argmax"][3] == -1 and got["logp"][8] == 0
    s = run_sls(w)
    assert s["status"] & cev.STATUS_BAD_LABEL


def test_argmax_ties_lowest_index():
    """Ties of the row maximum, on and off the target, resolve to the lowest
    column, compared on the stored values."""
    from gpu_helpers import run_ce
    rng = np.random.default_rng(8)
    rows, V = 16, 40000
    z = (rng.standard_normal((rows, V)) * 0.3).astype(np.float32)
    labels = rng.integers(0, V, rows).astype(np.int64)
    for r in range(rows):
        cols = np.sort(rng.choice(V, 3, replace=False))
        z[r, cols] = 7.0
        if r % 4 == 0:
            labels[r] = cols[1]          # target ties a lower column
        elif r % 4 == 1:
            labels[r] = cols[0]          # target is the lowest tied column
        elif r % 4 == 2:
            z[r, labels[r]] = 7.0        # target joins the tie
    for dtype in ("f32", "bf16"):
        logits = workloads.bf16_bits(z) if dtype == "bf16" else z.copy()
        w = dict(logits=logits, labels=labels, row_mask=None, temperature=0.9,
                 g=np.ones(rows, np.float32))
        got = run_ce(w)
        stored = workloads.stored_values(logits)
        assert np.array_equal(got["argmax"], np.argmax(stored, axis=1)), dtype
        _check_against_oracle(w, got, f"ties {dtype}")


def test_deterministic_bits():
    from gpu_helpers import run_ce
    w = workloads.grpo(rows=24, vocab=152064)
    a = run_ce(w)
    b = run_ce(w)
    for k in ("logp", "loss", "entropy", "argmax", "saved", "dlogits"):
        assert np.array_equal(np.asarray(a[k]).view(np.uint8), np.asarray(b[k]).view(np.uint8)), k


def test_output_guard_bands():
    """Outputs written into the middle of larger buffers touch nothing else."""
    from gpu_helpers import DEV, to_dev
    w = _rand_case(10, 2000, "bf16", seed=9, n_ignored=3)
    logits = to_dev(w["logits"])
    labels = to_dev(w["labels"])
    pad = 64
    buf = {
        "loss": torch.full((10 + 2 * pad,), 77.0, device=DEV),
        "logp": torch.full((10 + 2 * pad,), 77.0, device=DEV),
        "entropy": torch.full((10 + 2 * pad,), 77.0, device=DEV),
        "argmax": torch.full((10 + 2 * pad,), 77, dtype=torch.int64, device=DEV),
        "valid_rows": torch.full((10 + 2 * pad,), 77, dtype=torch.int64, device=DEV),
    }
    saved = torch.full((10 + 2 * pad, 16), 77, dtype=torch.uint8, device=DEV)
    nv = torch.full((1 + 2 * pad,), 77, dtype=torch.int64, device=DEV)
    out = {k: v[pad:pad + 10] for k, v in buf.items()}
    out["saved"] = saved[pad:pad + 10]
    out["n_valid"] = nv[pad:pad + 1]
    cev.ce_forward(logits, labels, 1.0, entropy=True, argmax=True, out=out)
    torch.cuda.synchronize()
    for k, v in buf.items():
        assert torch.all(v[:pad] == 77) and torch.all(v[pad + 10:] == 77), k
    assert torch.all(saved[:pad] == 77) and torch.all(saved[pad + 10:] == 77)
    assert torch.all(nv[:pad] == 77) and torch.all(nv[pad + 1:] == 77)
    n = int(out["n_valid"].item())
    vrows = out["valid_rows"][:n].cpu().numpy()
    assert np.array_equal(vrows, np.flatnonzero(w["labels"] != -100))


def test_topk_duplicates_ignored_and_bad_indices():
    from gpu_helpers import run_topk
    w = _rand_case(10, 5000, "bf16", T=0.7, seed=10, mask_frac=0.2)
    rng = np.random.default_rng(11)
    idx = rng.integers(0, 5000, (10, 12)).astype(np.int64)
    idx[:, 3] = idx[:, 1]          # duplicate column
    idx[2, 5] = -100               # ignored entry
    idx[4, 0] = 5000               # out of range
    idx[6, 7] = -3                 # out of range
    got, st = run_topk(w, idx)
    want, wst = oracle.topk_rows(w["logits"], idx, 0.7, row_mask=w["row_mask"])
    assert st & cev.STATUS_BAD_INDEX or w["row_mask"][4] == 0 and w["row_mask"][6] == 0
    assert_close("topk dup", got, want, RTOL["bf16"]["topk"])
    assert_nonpositive("topk dup", got)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_topk_register_path_boundary(dtype):
    """K = 64 (indices held in lanes) and K = 65 (indices in LDS) on rows that
    start at every alignment (padded stride, NaN canaries), with gathered
    columns in the unaligned head, the ragged tail and the last full step,
    duplicates, an ignored entry and out-of-range ones: both against the
    oracle, and the two paths agreeing bit for bit on the shared indices."""
    from gpu_helpers import DEV, strided_dev, to_dev, to_host
    R, V = 16, 3001
    w = _rand_case(R, V, dtype, T=0.8, seed=21, mask_frac=0.2)
    rng = np.random.default_rng(22)
    idx = np.stack([rng.choice(V, 64, replace=False) for _ in range(R)]).astype(np.int64)
    idx[:, 0] = np.arange(R) % 7           # head columns
    idx[:, 1] = V - 1 - np.arange(R) % 3   # ragged tail
    idx[:, 2] = idx[:, 5]                  # duplicate
    idx[3, 9] = -100                       # ignored
    idx[5, 10] = V                         # out of range
    idx[7, 11] = -2                        # out of range
    idx65 = np.concatenate([idx, np.full((R, 1), -100, np.int64)], axis=1)
    logits = strided_dev(w["logits"], V + 3)
    mask = to_dev(w["row_mask"])
    got = {}
    for K, ix in ((64, idx), (65, idx65)):
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        lp, q, saved = cev.sls_topk_forward(logits, to_dev(ix), 0.8, row_mask=mask, status=status,
                                            saved=True)
        torch.cuda.synchronize()
        got[K] = (to_host(lp), to_host(q), saved.cpu().numpy(), int(status.item()))
        assert got[K][3] & cev.STATUS_BAD_INDEX, K
        want, _ = oracle.topk_rows(w["logits"], ix, 0.8, row_mask=w["row_mask"])
        assert_close(f"topk K={K}", got[K][0], want, RTOL[dtype]["topk"])
        assert_nonpositive(f"topk K={K}", got[K][0])
    assert np.array_equal(got[64][0], got[65][0][:, :64])
    assert np.array_equal(got[64][1], got[65][1][:, :64])
    assert np.all(got[65][0][:, 64] == 0) and np.all(got[65][1][:, 64] == 0)
    assert np.array_equal(got[64][2], got[65][2])


def test_topk_large_k_and_peaked():
    """K = 100 gathered columns on peaked rows: the peak's own log p keeps its
    tiny complement (never 0, never positive)."""
    from gpu_helpers import run_topk
    w = workloads.peaked("f32", 0.9, rows=12, vocab=20000)
    rng = np.random.default_rng(12)
    idx = np.stack([rng.choice(20000, 100, replace=False) for _ in range(12)]).astype(np.int64)
    idx[:, 50] = w["labels"]
    idx[idx[:, 49] == w["labels"], 49] = (w["labels"][idx[:, 49] == w["labels"]] + 1) % 20000
    got, st = run_topk(w, idx)
    want, _ = oracle.topk_rows(w["logits"], idx, 0.9)
    assert_close("topk K=100", got, want, RTOL["f32"]["topk"])
    assert np.all(got[:, 50] < 0)


def test_topk_index_equals_label_matches_sls():
    from gpu_helpers import run_sls, run_topk
    w = _rand_case(30, 32768, "bf16", T=0.7, seed=13)
    idx = np.stack([w["labels"], (w["labels"] + 7) % 32768], axis=1)
    got, _ = run_topk(w, idx)
    s = run_sls(w, entropy=False, argmax=False)
    assert_close("topk vs sls", got[:, 0], s["logp"], 1e-6)


def test_temperature_scaling_identity():
    """T = 0.5 on z equals T = 1 on 2z (both exact), up to fp32 rounding of log2(e)/T."""
    from gpu_helpers import run_ce
    w = _rand_case(8, 9000, "f32", T=0.5, seed=14)
    a = run_ce(w)
    w2 = dict(w, logits=w["logits"] * np.float32(2.0), temperature=1.0)
    b = run_ce(w2)
    assert_close("T scaling logp", a["logp"], b["logp"].astype(np.float64), 2e-6)
    assert np.array_equal(a["argmax"], b["argmax"])


def _ce_raw(w, workspace_bytes, eps=0.0):
    """ce_forward through the C ABI with an explicit workspace size (0 = none),
    so the whole-row and the split-row sweeps can both be exercised."""
    from gpu_helpers import DEV, to_dev
    from cross_entropy_vocab_amd import _lib
    logits = to_dev(w["logits"])
    labels = to_dev(w["labels"])
    R, V = w["logits"].shape
    dt = 1 if w["logits"].dtype == np.uint16 else 0
    mask = None if w.get("row_mask") is None else to_dev(w["row_mask"])
    loss = torch.empty(R, device=DEV)
    logp = torch.empty(R, device=DEV)
    ent = torch.empty(R, device=DEV)
    arg = torch.empty(R, dtype=torch.int64, device=DEV)
    saved = torch.empty((R, 16), dtype=torch.uint8, device=DEV)
    vr = torch.empty(R, dtype=torch.int64, device=DEV)
    nv = torch.empty(1, dtype=torch.int64, device=DEV)
    ws = torch.empty(max(workspace_bytes, 1), dtype=torch.uint8, device=DEV)
    rc = _lib.get().ce_forward(logits.data_ptr(), R, V, V, dt, labels.data_ptr(), -100,
                               float(w["temperature"]), float(eps),
                               None if mask is None else mask.data_ptr(), loss.data_ptr(),
                               saved.data_ptr(), logp.data_ptr(), ent.data_ptr(), arg.data_ptr(),
                               vr.data_ptr(), nv.data_ptr(),
                               ws.data_ptr() if workspace_bytes else None, workspace_bytes, None,
                               torch.cuda.current_stream().cuda_stream)
    assert rc == 0, rc
    torch.cuda.synchronize()
    return dict(loss=loss.cpu().numpy(), logp=logp.cpu().numpy(), entropy=ent.cpu().numpy(),
                argmax=arg.cpu().numpy(), saved=saved.cpu().numpy(), n_valid=int(nv.item()),
                valid_rows=vr.cpu().numpy())


@pytest.mark.parametrize("rows,V,dtype,T", [(1, 152064, "bf16", 1.0), (3, 151936, "f32", 0.9),
                                            (12, 152064, "bf16", 1.0), (15, 65537, "f32", 0.7),
                                            (7, 40001, "bf16", 1.3)])
def test_split_rows_match_oracle_and_whole_rows(rows, V, dtype, T):
    """Few long rows: the split-row sweep (partials + fixed-order merge) and the
    whole-row sweep both match the oracle, and the integer outputs agree."""
    w = _rand_case(rows, V, dtype, T=T, seed=rows + V, n_ignored=rows // 5)
    if rows >= 3:
        w["logits"][1] = w["logits"][0]        # duplicated row: identical outputs
        w["labels"][1] = w["labels"][0] if w["labels"][0] != -100 else 5
        w["labels"][0] = w["labels"][1]
    import cross_entropy_vocab_amd as cev
    full = cev.workspace_size(rows, V, 1 if dtype == "bf16" else 0)
    split = _ce_raw(w, full)
    whole = _ce_raw(w, 0)
    tol = RTOL[dtype]
    ref = oracle.ce_rows(w["logits"], w["labels"], T)
    for got, kind in ((split, "split"), (whole, "whole")):
        assert_close(f"{kind} logp", got["logp"], ref["logp"], tol["logp"])
        assert_close(f"{kind} loss", got["loss"], ref["loss"], tol["loss"])
        assert_close(f"{kind} entropy", got["entropy"], ref["entropy"], tol["entropy"], 1e-30)
        assert np.array_equal(got["argmax"], ref["argmax"]), kind
    assert split["n_valid"] == whole["n_valid"]
    assert np.array_equal(split["valid_rows"][:split["n_valid"]],
                          whole["valid_rows"][:whole["n_valid"]])
    # saved records: same maximum bits and flags; sums agree to rounding
    s1 = split["saved"].view(np.float32).reshape(rows, 4)
    s2 = whole["saved"].view(np.float32).reshape(rows, 4)
    assert np.array_equal(s1[:, 0], s2[:, 0]) and np.array_equal(s1[:, 3], s2[:, 3])
    # log2 d enters dlogits as an exponent: 1e-6 absolute is 7e-7 relative in p
    assert_close("log2 d", s1[:, 1], s2[:, 1].astype(np.float64), 1e-6, 1e-6)
    if rows >= 3:
        assert split["logp"][0] == split["logp"][1] and split["argmax"][0] == split["argmax"][1]
    # a second split call is bit-identical
    again = _ce_raw(w, full)
    assert np.array_equal(again["saved"], split["saved"])
    assert np.array_equal(again["logp"].view(np.uint32), split["logp"].view(np.uint32))


def _run_fused(w, logits_dev=None, dl_stride=None, entropy=True):
    from gpu_helpers import DEV, to_dev, to_host
    logits = logits_dev if logits_dev is not None else to_dev(w["logits"])
    labels = to_dev(w["labels"])
    mask = None if w.get("row_mask") is None else to_dev(w["row_mask"])
    g = to_dev(np.asarray(w["g"], np.float32))
    R, V = w["logits"].shape
    dl = None
    if dl_stride is not None:
        dl = torch.zeros((R, dl_stride), dtype=logits.dtype, device=DEV)[:, :V]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = cev.ce_fused(logits, labels, g, w["temperature"], row_mask=mask, entropy=entropy,
                       argmax=True, valid_rows=True, dlogits=dl, status=status)
    torch.cuda.synchronize()
    res = {k: to_host(v) for k, v in out.items() if v is not None and k != "workspace"}
    res["status"] = int(status.item())
    return res


def _fused_regions_case():
    """bf16 rows of 77101 columns, targets in every part of ce_fused's row
    layout: 9637 vectors of 8 make 75 wave steps of 128 vectors (steps 0-31
    held in registers, 32-63 in LDS, 64-74 read twice), 37 remainder vectors
    and 5 tail columns; one row peaked on a target in the LDS-held part, one
    ignored."""
    w = _rand_case(11, 77101, "bf16", T=0.9, seed=44)
    w["labels"][:] = [100, 20000, 33000, 60000, 66000, 76000, 76900, 77098, 77100, 40000, -100]
    z = workloads.bf16_to_f32(w["logits"])
    z[9, 40000] = z[9].max() + 30.0
    w["logits"] = workloads.bf16_bits(z)
    return w


FUSED_CASES = {
    "regions_11x77101_bf16_T0.9": _fused_regions_case,
    "grpo_40x152064_bf16": lambda: workloads.grpo(rows=40, vocab=152064),
    "peaked_16x151936_bf16_T0.9": lambda: workloads.peaked("bf16", 0.9, rows=16),
    "peaked_12x151936_f32_T1_two_pass": lambda: workloads.peaked("f32", 1.0, rows=12),
    "tiny_64x4096_f32": lambda: workloads.tiny(),
    "sparse_1922x4096_f32": lambda: workloads.sparse(),
    "chunk_20x32768_bf16_T0.7": lambda: workloads.chunk(rows=20, vocab=32768),
    "small_9x300_f32_two_pass": lambda: _rand_case(9, 300, "f32", seed=1, n_ignored=2),
}


@pytest.mark.parametrize("name", sorted(FUSED_CASES))
def test_ce_fused_matches_oracle(name):
    """ce_fused against the oracle on every output, in both its fused form
    (16-byte-aligned rows: one workgroup sweeps, closes and re-reads each row)
    and its fallback to ce_forward + ce_backward (other alignments)."""
    w = FUSED_CASES[name]()
    got = _run_fused(w)
    _check_against_oracle(w, got, f"fused {name}")
    assert got["status"] == 0


def test_ce_fused_tail_columns_and_padded_strides():
    """V not a multiple of 8 with 16-byte aligned padded rows (one pass, tail
    columns in the registers), and the same with an unaligned stride (two pass);
    padding columns of dlogits stay untouched."""
    from gpu_helpers import strided_dev
    for V, stride in ((32781, 32784), (32781, 32781), (40007, 40016)):
        w = _rand_case(10, V, "bf16", T=0.8, seed=V + stride, n_ignored=2)
        w["labels"][3] = V - 1            # target in the tail columns
        w["labels"][4] = V - 3
        got = _run_fused(w, logits_dev=strided_dev(w["logits"], stride), dl_stride=stride)
        _check_against_oracle(w, got, f"fused V={V} stride={stride}")


def test_ce_fused_equals_separate_calls():
    """The one-pass result matches ce_forward + ce_backward (summation order
    differs: log p to 1e-6, bf16 dlogits to one rounding step)."""
    from gpu_helpers import run_ce
    w = workloads.grpo(rows=48, vocab=152064)
    a = _run_fused(w, entropy=False)
    b = run_ce(w, entropy=False)
    assert_close("fused vs two-pass logp", a["logp"], b["logp"].astype(np.float64), 1e-6)
    assert np.array_equal(a["argmax"], b["argmax"])
    assert np.array_equal(a["valid_rows"][:int(a["n_valid"][0])],
                          b["valid_rows"][:int(b["n_valid"][0])])
    assert_close("fused vs two-pass dlogits", a["dlogits"], b["dlogits"], 8e-3, 2.0 ** -126)
    again = _run_fused(w, entropy=False)
    assert np.array_equal(again["dlogits"], a["dlogits"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mask_views_at_every_byte_offset(dtype):
    """The kernels read a row's mask byte as the aligned 4-byte word holding
    it: a mask that is a view starting at byte offsets 0-3 of a larger buffer,
    with a row count that is not a multiple of 4, must give the same results
    as the oracle for ce_forward/ce_backward, sls_forward and sls_topk_forward
    (the bytes around the view are the opposite of the row's own)."""
    from gpu_helpers import DEV, to_dev, to_host
    rows, V = 13, 3000
    w = _rand_case(rows, V, dtype, T=0.9, seed=31, mask_frac=0.4, n_ignored=2)
    host_mask = w["row_mask"]
    ref = oracle.ce_rows(w["logits"], w["labels"], w["temperature"], row_mask=host_mask)
    kind = "bf16" if dtype == "bf16" else "f32"
    tol = RTOL[kind]
    idx = np.stack([np.arange(4) * 7 + r for r in range(rows)]).astype(np.int64)
    tref, _ = oracle.topk_rows(w["logits"], idx, w["temperature"], row_mask=host_mask)
    logits = to_dev(w["logits"])
    labels = to_dev(w["labels"])
    g = to_dev(w["g"])
    for off in range(4):
        buf = np.empty(rows + 8, dtype=np.uint8)
        buf[:] = 1 - np.resize(host_mask, rows + 8)          # neighbours disagree
        buf[off:off + rows] = host_mask
        mask = to_dev(buf)[off:off + rows]
        assert mask.is_contiguous() and mask.data_ptr() % 4 == off % 4
        out = cev.ce_forward(logits, labels, w["temperature"], row_mask=mask, argmax=True)
        dl = cev.ce_backward(logits, labels, g, out["saved"], w["temperature"], row_mask=mask)
        s = cev.sls_forward(logits, labels, w["temperature"], row_mask=mask)
        tk = cev.sls_topk_forward(logits, to_dev(idx), w["temperature"], row_mask=mask)
        torch.cuda.synchronize()
        name = f"{dtype} mask offset {off}"
        assert_close(f"{name} loss", to_host(out["loss"]), ref["loss"], tol["loss"])
        assert_close(f"{name} sls logp", to_host(s["logp"]), ref["logp"], tol["logp"])
        assert_close(f"{name} topk logp", to_host(tk), tref, tol["logp"])
        assert np.array_equal(to_host(out["argmax"]), ref["argmax"]), name
        valid = (host_mask != 0) & (w["labels"] != -100)
        d = to_host(dl)
        assert np.all(d[~valid] == 0) and np.all(np.any(d[valid] != 0, axis=1)), name

def test_ce_fused_unaligned_rows_without_workspace():
    """ce_fused on rows that are not 16-byte aligned (its fallback to
    ce_forward + ce_backward) with no list outputs and no workspace, through
    the C ABI: accepted as the aligned form is, and equal to the oracle; the
    same call with a large input (every row swept in place, no list)."""
    import ctypes
    from gpu_helpers import DEV, strided_dev, to_dev, to_host
    from cross_entropy_vocab_amd import _lib
    lib = _lib.get()
    for rows, V, stride, dt in ((24, 4099, 4101, "f32"), (260, 152064, 152067, "bf16")):
        w = _rand_case(rows, V, dt, T=0.9, seed=rows, n_ignored=3, mask_frac=0.1)
        logits = strided_dev(w["logits"], stride)
        assert logits.stride(0) == stride and (stride * logits.element_size()) % 16 != 0
        lab = to_dev(w["labels"])
        mask = to_dev(w["row_mask"])
        g = to_dev(w["g"])
        loss = torch.empty(rows, dtype=torch.float32, device=DEV)
        logp = torch.empty(rows, dtype=torch.float32, device=DEV)
        argmax = torch.empty(rows, dtype=torch.int64, device=DEV)
        saved = torch.empty((rows, 16), dtype=torch.uint8, device=DEV)
        dl = torch.empty((rows, V), dtype=logits.dtype, device=DEV)
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        code = cev.CEV_BF16 if dt == "bf16" else cev.CEV_F32
        rc = lib.ce_fused(logits.data_ptr(), rows, V, stride, code, lab.data_ptr(), -100,
                          w["temperature"], 0.0, mask.data_ptr(), g.data_ptr(), loss.data_ptr(),
                          saved.data_ptr(), logp.data_ptr(), None, argmax.data_ptr(),
                          dl.data_ptr(), V, None, None, None, 0, status.data_ptr(),
                          ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream))
        assert rc == 0, rc
        torch.cuda.synchronize()
        kind = "bf16" if dt == "bf16" else "f32"
        tol = RTOL[kind]
        ref = oracle.ce_rows(w["logits"], w["labels"], w["temperature"], row_mask=w["row_mask"],
                             want_entropy=False)
        assert_close(f"fused unaligned {rows}x{V} loss", to_host(loss), ref["loss"], tol["loss"])
        assert_close(f"fused unaligned {rows}x{V} logp", to_host(logp), ref["logp"], tol["logp"])
        assert np.array_equal(to_host(argmax), ref["argmax"])
        sample = np.arange(0, rows, max(1, rows // 12))
        g64 = np.asarray(w["g"], np.float64)
        dref = np.concatenate([oracle.ce_grad_rows(w["logits"], w["labels"], g64, w["temperature"],
                                                   row_mask=w["row_mask"], r0=int(r), r1=int(r) + 1)
                               for r in sample])
        assert_close(f"fused unaligned {rows}x{V} dlogits", to_host(dl)[sample], dref,
                     tol["dlogits"], atol=2.0 ** -126)
        assert int(status.item()) == 0
