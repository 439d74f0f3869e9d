"""The vocab-parallel form on one GPU: the columns of each row are cut into P
shards (views of one matrix standing in for P ranks), each shard swept into
partial records, the records stacked (the all-gather) and merged, and the
backward run shard by shard.  The merged outputs are those of the whole row,
so the oracle is the plain one on the full matrix."""
import numpy as np
import pytest
import torch

import cross_entropy_vocab_amd as cev
import oracle
import workloads
from tolerance import FLOOR, RTOL, assert_close, assert_nonpositive, assert_row_sums

pytestmark = pytest.mark.gpu


def _kind(w):
    return "bf16" if w["logits"].dtype == np.uint16 else "f32"


def even_bounds(V, P):
    return [V * p // P for p in range(P + 1)]


def run_sharded(w, bounds, eps=0.0, entropy=True, logits_dev=None, skip=()):
    """Shard forward on every shard (except those in `skip`), merge, shard
    backward into one full-width dlogits; numpy outputs."""
    from gpu_helpers import DEV, to_dev, to_host
    R, V = w["logits"].shape
    logits = logits_dev if logits_dev is not None else to_dev(w["logits"])
    labels = to_dev(w["labels"])
    mask = None if w.get("row_mask") is None else to_dev(w["row_mask"])
    g = to_dev(np.asarray(w["g"], np.float32))
    T = w["temperature"]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    parts = []
    for p, (c0, c1) in enumerate(zip(bounds[:-1], bounds[1:])):
        if p in skip:
            continue
        parts.append(cev.ce_vocab_shard_forward(logits[:, c0:c1], labels, c0, V, T,
                                                row_mask=mask, entropy=entropy,
                                                value_sum=eps != 0.0, status=status))
    out = cev.ce_vocab_merge(torch.stack(parts), labels, V, T, row_mask=mask,
                             label_smoothing=eps, entropy=entropy, argmax=True, status=status)
    dl = torch.full((R, V), float("nan"), dtype=logits.dtype, device=DEV)
    for c0, c1 in zip(bounds[:-1], bounds[1:]):
        cev.ce_vocab_shard_backward(logits[:, c0:c1], labels, g, out["saved"], c0, V, T,
                                    row_mask=mask, label_smoothing=eps, dlogits=dl[:, c0:c1],
                                    status=status)
    torch.cuda.synchronize()
    res = {k: (None if v is None else to_host(v)) for k, v in out.items()}
    res["dlogits"] = to_host(dl)
    res["status"] = int(status.item())
    return res


def check_against_oracle(w, got, name, eps=0.0, entropy=True):
    tol = RTOL[_kind(w)]
    T = w["temperature"]
    V = w["logits"].shape[1]
    ref = oracle.ce_rows(w["logits"], w["labels"], T, row_mask=w.get("row_mask"),
                         label_smoothing=eps)
    vr, _ = oracle.valid_rows(w["labels"], w.get("row_mask"), V)
    valid = np.zeros(w["logits"].shape[0], bool)
    valid[vr] = True
    assert_close(f"{name} logp", got["logp"], ref["logp"], tol["logp"])
    assert_close(f"{name} loss", got["loss"], ref["loss"], tol["loss"])
    if entropy:
        assert_close(f"{name} entropy", got["entropy"], ref["entropy"], tol["entropy"], 1e-30)
    assert np.array_equal(got["argmax"], ref["argmax"]), name
    assert_nonpositive(name, got["logp"], valid)
    dref = oracle.ce_grad_rows(w["logits"], w["labels"], np.asarray(w["g"], np.float64), T,
                               row_mask=w.get("row_mask"), label_smoothing=eps)
    if eps == 0.0:
        assert_close(f"{name} dlogits", got["dlogits"], dref, tol["dlogits"], FLOOR)
    else:
        from test_gpu_smoothing_topk import TERM_RTOL, _assert_within, _smoothed_grad_bound
        mag, _ = _smoothed_grad_bound(w, eps)
        _assert_within(f"{name} dlogits", got["dlogits"], dref,
                       tol["dlogits"] * np.abs(dref) + TERM_RTOL * mag + FLOOR)
    assert_row_sums(f"{name} dlogits", got["dlogits"], tol["dlogits"])
    assert np.all(got["dlogits"][~valid] == 0)


CASES = {
    "grpo_40x152064_bf16_P8": (lambda: workloads.grpo(rows=40, vocab=152064),
                               lambda V: even_bounds(V, 8)),
    "chunk_24x32781_bf16_T0.7_ragged_P3": (
        lambda: dict(workloads.chunk(rows=24, vocab=32781),
                     g=np.random.default_rng(5).standard_normal(24).astype(np.float32)),
        lambda V: [0, 10000, 10003, V]),
    "peaked_24x151936_f32_T0.9_P4": (lambda: workloads.peaked("f32", 0.9, rows=24),
                                     lambda V: even_bounds(V, 4)),
    "peaked_16x151936_bf16_T1_P5": (lambda: workloads.peaked("bf16", 1.0, rows=16),
                                    lambda V: [0, 7, 30001, 30002, 100000, V]),
    "tiny_64x4096_f32_P2": (lambda: workloads.tiny(), lambda V: even_bounds(V, 2)),
    "sparse_1922x4096_f32_P7": (lambda: workloads.sparse(), lambda V: even_bounds(V, 7)),
}


@pytest.mark.parametrize("eps", [0.0, 0.1])
@pytest.mark.parametrize("name", sorted(CASES))
def test_sharded_matches_oracle(name, eps):
    from gpu_helpers import say
    make, bounds = CASES[name]
    w = make()
    say(f"[vocab-parallel] {name} eps={eps}")
    got = run_sharded(w, bounds(w["logits"].shape[1]), eps=eps)
    check_against_oracle(w, got, name, eps=eps)
    assert got["status"] == 0


def test_one_shard_is_bit_identical_to_ce_forward():
    """P = 1 runs the same row sweep as ce_forward and a merge that adds only
    exact zeros: every output bit matches."""
    from gpu_helpers import run_ce
    w = workloads.grpo(rows=200, vocab=20011)
    got = run_sharded(w, [0, 20011])
    ce = run_ce(w)
    for k in ("logp", "loss", "entropy", "argmax", "saved", "dlogits"):
        assert np.array_equal(got[k], ce[k]), k


def test_shard_boundaries_targets_and_cross_shard_ties():
    """Labels on the first and last column of every shard; row maxima tied
    across shards (the lowest global column wins, on and off the target)."""
    from gpu_helpers import DEV
    V, P = 1000, 4
    b = [0, 250, 251, 640, V]
    rng = np.random.default_rng(61)
    z = (2.0 * rng.standard_normal((16, V))).astype(np.float32)
    labels = np.array([0, 249, 250, 251, 639, 640, 999, 500, 3, 700, 100, 900, 251, 0, 999, 640],
                      np.int64)
    z[8, [10, 300, 700]] = 20.0                # tie in three shards, off the target
    z[9, [20, 700]] = 21.0                     # tie, the target (700) is not the lowest
    z[10, [100, 800]] = 22.0                   # tie, the target (100) is the lowest
    z[11, [5, 900]] = 23.0                     # tie with the target in the last shard
    z[12, 251] = 30.0                          # peaked target on a shard's first column
    # row 2's label (250) is the only column of shard [250, 251)
    w = dict(logits=z, labels=labels, row_mask=None, temperature=0.9,
             g=rng.standard_normal(16).astype(np.float32))
    got = run_sharded(w, b)
    check_against_oracle(w, got, "boundaries")
    assert list(got["argmax"][8:12]) == [10, 20, 100, 5]


def test_misaligned_shards_and_strides():
    """Shard starts at every alignment modulo 16 bytes (element head path),
    a padded row stride with NaN canaries."""
    from gpu_helpers import strided_dev
    for dtype in ("f32", "bf16"):
        rng = np.random.default_rng(71)
        z = (3.0 * rng.standard_normal((12, 5003))).astype(np.float32)
        w = dict(logits=workloads.bf16_bits(z) if dtype == "bf16" else z,
                 labels=rng.integers(0, 5003, 12).astype(np.int64), row_mask=None,
                 temperature=1.1, g=rng.standard_normal(12).astype(np.float32))
        w["labels"][3] = -100
        got = run_sharded(w, [0, 1, 3, 6, 13, 1001, 2999, 5003],
                          logits_dev=strided_dev(w["logits"], 5011))
        check_against_oracle(w, got, f"misaligned {dtype}")


def test_inconsistent_partials_are_flagged():
    """A missing shard leaves the rows whose label it held without an owner:
    those rows get the ignored-row outputs and CEV_STATUS_BAD_PARTS; rows whose
    label is elsewhere merge normally (over the columns present)."""
    from gpu_helpers import DEV, to_dev, to_host
    w = workloads.tiny()
    V = w["logits"].shape[1]
    b = even_bounds(V, 4)
    logits = to_dev(w["logits"])
    labels = to_dev(w["labels"])
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    parts = [cev.ce_vocab_shard_forward(logits[:, c0:c1], labels, c0, V, 1.0)
             for c0, c1 in zip(b[:-1], b[1:]) if c0 != b[2]]
    out = cev.ce_vocab_merge(torch.stack(parts), labels, V, 1.0, argmax=True, status=status)
    torch.cuda.synchronize()
    lab = w["labels"]
    orphan = (lab >= b[2]) & (lab < b[3])
    assert status.item() & cev.STATUS_BAD_PARTS
    assert np.all(to_host(out["loss"])[orphan] == 0)
    assert np.all(to_host(out["argmax"])[orphan] == -1)
    sv = out["saved"].cpu().numpy().view(np.int32).reshape(-1, 4)
    assert np.all(sv[orphan, 3] == 0) and np.all(sv[(lab != -100) & ~orphan, 3] == 1)
    # a shard computed under a row mask that drops a valid row marks it invalid
    r0 = int(np.flatnonzero(lab != -100)[0])
    mask = torch.ones(64, dtype=torch.uint8, device=DEV)
    mask[r0] = 0
    parts = [cev.ce_vocab_shard_forward(logits[:, c0:c1], labels, c0, V, 1.0,
                                        row_mask=mask if p == 1 else None)
             for p, (c0, c1) in enumerate(zip(b[:-1], b[1:]))]
    status.zero_()
    out = cev.ce_vocab_merge(torch.stack(parts), labels, V, 1.0, status=status)
    torch.cuda.synchronize()
    assert status.item() & cev.STATUS_BAD_PARTS
    assert to_host(out["loss"])[r0] == 0


def test_bad_labels_and_determinism():
    from gpu_helpers import DEV
    rng = np.random.default_rng(81)
    z = (3.0 * rng.standard_normal((9, 3000))).astype(np.float32)
    labels = rng.integers(0, 3000, 9).astype(np.int64)
    labels[2] = 3000
    labels[5] = -7
    w = dict(logits=z, labels=labels, row_mask=None, temperature=1.0,
             g=rng.standard_normal(9).astype(np.float32))
    got = run_sharded(w, even_bounds(3000, 3))
    assert got["status"] & cev.STATUS_BAD_LABEL
    assert got["loss"][2] == 0 and got["argmax"][5] == -1
    assert np.all(got["dlogits"][[2, 5]] == 0)
    w2 = dict(w, labels=np.where((labels < 0) | (labels >= 3000), -100, labels))
    check_against_oracle(w2, got, "bad labels")
    again = run_sharded(w, even_bounds(3000, 3))
    for k in ("loss", "logp", "entropy", "argmax", "saved", "dlogits"):
        assert np.array_equal(again[k], got[k]), k
