"""The fp64 oracle against closed forms, 120-digit brute force, invariants,
library routines and the values the pages print (tests/golden/)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import pinlib
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("check", pinlib.ALL_CHECKS + pinlib.LINEAR_CHECKS,
                         ids=lambda c: c.__name__)
def test_pin(check):
    check()


@pytest.mark.parametrize("check", pinlib.JSD_CHECKS, ids=lambda c: c.__name__)
def test_jsd_pin(check):
    check()


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _naive_fp32_logp(z, t):
    """Plain fp32 log_softmax at the target: x_t - (m + log sum e^{x - m})."""
    x = z.astype(np.float32)
    m = x.max()
    s = np.sum(np.exp(x - m), dtype=np.float32)
    return np.float32(x[t] - (m + np.log(s)))


def _naive_fp64_logp(z, t):
    x = z.astype(np.float64)
    m = x.max()
    return x[t] - (m + math.log(np.sum(np.exp(x - m))))


def _naive_target_grad(z, t, ftype):
    """Plain softmax at the target minus one, in the given float type:
    e^{x_t - m} / sum_j e^{x_j - m} - 1."""
    x = z.astype(ftype)
    e = np.exp(x - x.max())
    return ftype(e[t] / np.sum(e, dtype=ftype) - ftype(1))


def test_golden_collapse_thresholds():
    """The pages put the collapse at a target lead of about 16.6 over the
    log-sum-exp of the other classes in fp32 and about 36.7 in fp64: beyond it
    softmax at the target rounds to 1, so its gradient p_t - 1 reads exactly 0.
    The oracle's target gradient (-q) and loss stay at the closed form."""
    gold = _golden("collapse_thresholds.json")
    assert math.log(2.0 ** 24) == pytest.approx(gold["fp32_lead"], abs=0.05)
    assert math.log(2.0 ** 53) == pytest.approx(gold["fp64_lead"], abs=0.05)
    # V = 2: the lead over the others' log-sum-exp is the margin itself
    for ftype, key in ((np.float32, "fp32_lead"), (np.float64, "fp64_lead")):
        for lead, collapsed in ((gold[key] - 0.3, False), (gold[key] + 0.3, True)):
            z = np.array([0.0, lead], dtype=np.float32)
            assert (_naive_target_grad(z, 1, ftype) == 0) == collapsed, (key, lead)
            o = oracle.ce_rows(z[None, :], np.array([1]), 1.0, threads=1)
            lead32 = float(z[1])
            assert abs(o["q"][0] - math.exp(-lead32) / (1 + math.exp(-lead32))) <= \
                1e-15 * o["q"][0]
            expect = -math.log1p(math.exp(-lead32))
            assert o["logp"][0] < 0 and abs(o["logp"][0] - expect) <= 1e-15 * abs(expect)


def _lead_over_others(z, t):
    """x_t - log sum_{j != t} e^{x_j} in fp64 (T = 1), with a max shift."""
    x = z.astype(np.float64)
    o = np.delete(x, t)
    m = o.max()
    return x[t] - (m + math.log(np.sum(np.exp(o - m))))


def test_golden_negative_control_margins():
    """Peaked rows at the pages' margins (17, 20, 30, 50 over equal others, at
    V in {1003, 40001, 151936}): plain fp32 softmax puts exactly 0 gradient on the
    target wherever the lead over the others' log-sum-exp passes ln 2^24, and not
    below it; the oracle's loss and target gradient stay at the closed form."""
    gold = _golden("collapse_thresholds.json")
    thr = math.log(2.0 ** 24)
    seen = set()
    for V in gold["vocab_sizes"]:
        for M in gold["margins"]:
            z = np.zeros(V, dtype=np.float32)
            z[5] = M
            lead = _lead_over_others(z, 5)
            if abs(lead - thr) < 0.05:
                continue
            collapsed = lead > thr
            seen.add(collapsed)
            assert (_naive_target_grad(z, 5, np.float32) == 0) == collapsed, (V, M)
            o = oracle.ce_rows(z[None, :], np.array([5]), 1.0, threads=1)
            expect = -math.log1p((V - 1) * math.exp(-M))
            assert o["logp"][0] < 0 and o["q"][0] > 0
            assert abs(o["logp"][0] - expect) <= 1e-13 * abs(expect)
            # the pages' after-fix CE loss error bound (absolute) is far above ours
            assert abs(o["loss"][0] + expect) <= gold["ce_loss_abs_error_after_fix"]
    assert seen == {False, True}


def test_golden_sparse_supervision_shape():
    """The sparse-supervision workload: 1922 kept rows of which 256 are supervised,
    V = 4096; vocabulary-sized fp32 storage 30.03125 MiB dense vs 4 MiB sparse."""
    gold = _golden("sparse_supervision.json")
    w = workloads.sparse()
    rows, V = w["logits"].shape
    assert rows == gold["kept_rows"] and V == gold["vocab"]
    vr, st = oracle.valid_rows(w["labels"], None, V)
    assert st == 0 and vr.shape[0] == gold["supervised_rows"]
    assert rows * V * 4 / 2 ** 20 == gold["dense_fp32_MiB"]
    assert vr.shape[0] * V * 4 / 2 ** 20 == gold["sparse_fp32_MiB"]


def test_negative_control_on_peaked_workload():
    """P8 on the peaked workload's recipe: wherever the target's lead over the
    others' log-sum-exp passes ln 2^24 (fp32) or ln 2^53 (fp64), plain softmax
    gives a target gradient of exactly 0; the oracle's loss and q stay > 0."""
    w = workloads.peaked("f32", 1.0, rows=24, vocab=2000)
    o = oracle.ce_rows(w["logits"], w["labels"], 1.0)
    assert np.all(o["loss"] > 0) and np.all(o["q"] > 0)
    n32 = n64 = 0
    for r in range(24):
        z = w["logits"][r]
        t = w["labels"][r]
        lead = _lead_over_others(z, t)
        if lead > math.log(2.0 ** 24) + 0.05:
            assert _naive_target_grad(z, t, np.float32) == 0
            n32 += 1
        if lead > math.log(2.0 ** 53) + 0.05:
            assert _naive_target_grad(z, t, np.float64) == 0
            n64 += 1
    assert n32 > 0 and n64 > 0
