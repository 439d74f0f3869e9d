"""Generalized JSD / KL between student and teacher rows (jsd_forward,
jsd_backward) against the fp64 oracle (oracle/jsd.py).

Error model of the GPU arithmetic, per column j (derived, not fitted): the
exponent arguments (z - m)/T are rounded to fp32 and exp2 / log1p / expm1 err
by a few ulp, and the per-row log-normalisers log1p(S) are fp32 copies of
fp64 sums of fp32 terms, so log p_j and every quantity built from it errs by
about eps_j = 3e-7 (2 + |ls_j| + |lt_j|): relative for the probabilities,
absolute for log-differences such as delta = lt - ls (whose error does not
shrink with delta).  The loss sum_j p_j f(delta_j) then errs by at most
sum_j eps_j p_j (1 + |f_j|) (its terms accumulate in fp32 over one 16-byte
vector, then in fp64).  A gradient entry is the difference of two terms -- ps - pt
(beta = 0), ps (-delta) and ps L (beta = 1), ps r and ps K (in between) -- so
it errs relative to those terms plus the carried error of L or K; the
student's argmax entry is minus the sum of the others, so it errs like them
together.  fp32 outputs add one rounding, bf16 outputs 2^-8 relative (round
to nearest even), and entries below 2^-126 may be flushed (the weight |g|/T
is folded into the exponent, so an entry flushes only when it is itself that
small); in the loss, a term whose probability is below the fp32 normal
range may be lost entirely.
"""
import numpy as np
import pytest
import torch

import cross_entropy_vocab_amd as cev
import oracle.jsd as oj
import workloads
from tolerance import FLOOR

pytestmark = pytest.mark.gpu

BETAS = (0.0, 0.1, 0.5, 1.0)


def _kind(w):
    return "bf16" if w["student"].dtype == np.uint16 else "f32"


def run_jsd(w, beta, ss=None, ts=None):
    from gpu_helpers import DEV, strided_dev, to_dev, to_host
    st = to_dev(w["student"]) if ss is None else strided_dev(w["student"], ss)
    te = to_dev(w["teacher"]) if ts is None else strided_dev(w["teacher"], ts)
    labels = None if w.get("labels") is None else to_dev(w["labels"])
    mask = None if w.get("row_mask") is None else to_dev(w["row_mask"])
    g = to_dev(np.asarray(w["g"], np.float32))
    T = w["temperature"]
    out = cev.jsd_forward(st, te, T, beta, labels=labels, row_mask=mask)
    d = cev.jsd_backward(st, te, g, out["saved"], T, beta, labels=labels, row_mask=mask)
    torch.cuda.synchronize()
    return dict(loss=to_host(out["loss"]), dstudent=to_host(d),
                saved=out["saved"].cpu().numpy())


def _valid(w):
    R = w["student"].shape[0]
    v = np.ones(R, bool)
    if w.get("row_mask") is not None:
        v &= w["row_mask"] != 0
    if w.get("labels") is not None:
        v &= w["labels"] != -100
    return v


def row_bounds(zs, zt, g, T, beta):
    """(loss, its bound, d_ref, per-entry bound) for one valid row."""
    loss, K, ls, lt, r = oj.jsd_row(zs, zt, T, beta)
    ps, pt = np.exp(ls), np.exp(lt)
    eps = 3e-7 * (2.0 + np.abs(ls) + np.abs(lt))
    delta = lt - ls
    if beta == 0.0:
        terms = pt * np.abs(delta)
        sens = pt * (1 + np.abs(delta))
    elif beta == 1.0:
        terms = ps * np.abs(delta)
        sens = ps * (1 + np.abs(delta))
    else:
        q = delta + r
        terms = beta * pt * np.abs(q) + (1 - beta) * ps * np.abs(r)
        sens = beta * pt * (1 + np.abs(q)) + (1 - beta) * ps * (1 + np.abs(r))
    tiny = 2.0 ** -126
    if beta == 0.0:
        lost = np.sum(np.where(pt < tiny, terms, 0.0))
    elif beta == 1.0:
        lost = np.sum(np.where(ps < tiny, terms, 0.0))
    else:
        lost = np.sum(np.where(pt < tiny, beta * pt * np.abs(q), 0.0) +
                      np.where(ps < tiny, (1 - beta) * ps * np.abs(r), 0.0))
    bl = float(np.sum(eps * sens)) + 1e-6 * abs(loss) + float(lost)
    w = abs(g) / T
    if beta == 0.0:
        bd = w * eps * (ps + pt)
    elif beta == 1.0:
        bd = w * ps * (eps * (1 + np.abs(delta) + abs(loss)) + 2 * bl)
    else:
        bk = float(np.sum(eps * ps * (1 + np.abs(r)))) + 1e-6 * abs(K)
        bd = w * (1 - beta) * ps * (eps * (1 + np.abs(r) + abs(K)) + 2 * bk + 6e-8 * abs(K))
    a = int(np.argmax(oj._widen(zs)))
    dref = oj.jsd_grad_row(zs, zt, g, T, beta)
    # entries (or, at beta = 0, the two products) below the fp32 normal range
    # may be flushed to zero before they enter the argmax entry's sum
    tiny = 2.0 ** -126
    if beta == 0.0:
        flushed = np.where(w * ps < tiny, w * ps, 0.0) + np.where(w * pt < tiny, w * pt, 0.0)
    else:
        flushed = np.where(np.abs(dref) < tiny, np.abs(dref), 0.0)
    bd[a] = 0.0
    flushed[a] = 0.0
    bd[a] = np.sum(bd) + np.sum(flushed)   # minus the sum of the others: their errors add
    return loss, bl, dref, bd


def check(w, got, beta, name, rows=None):
    T = w["temperature"]
    valid = _valid(w)
    R = w["student"].shape[0]
    rows = range(R) if rows is None else rows
    out_rtol = 4e-3 if _kind(w) == "bf16" else 1.2e-7
    worst_l = worst_d = 0.0
    for r in rows:
        if not valid[r]:
            assert got["loss"][r] == 0 and np.all(got["dstudent"][r] == 0), (name, r)
            continue
        loss, bl, dref, bd = row_bounds(w["student"][r], w["teacher"][r], float(w["g"][r]), T,
                                        beta)
        el = abs(got["loss"][r] - loss)
        assert el <= bl + 1e-30, (name, beta, r, "loss", got["loss"][r], loss, bl)
        worst_l = max(worst_l, el / (bl + 1e-30))
        ed = np.abs(got["dstudent"][r] - dref)
        bound = out_rtol * np.abs(dref) + bd + 2 * FLOOR
        i = int(np.argmax(ed / bound))
        assert np.all(ed <= bound), (name, beta, r, "dstudent", i, got["dstudent"][r][i], dref[i],
                                     bound[i])
        worst_d = max(worst_d, float(np.max(ed / bound)))
        assert got["loss"][r] >= -bl, (name, r)
    return worst_l, worst_d


CASES = {
    "distill_64x4099_f32_ragged": lambda: workloads.distill(rows=64, vocab=4099, dtype="f32",
                                                             peaked_frac=0.25),
    "distill_40x32768_bf16_T0.9": lambda: workloads.distill(rows=40, vocab=32768, dtype="bf16",
                                                             temperature=0.9, peaked_frac=0.2),
    "distill_24x151936_f32_peaked": lambda: workloads.distill(rows=24, vocab=151936, dtype="f32",
                                                               peaked_frac=0.75),
    "distill_24x151936_bf16_peaked_T0.7": lambda: workloads.distill(
        rows=24, vocab=151936, dtype="bf16", temperature=0.7, peaked_frac=0.75),
    "distill_32x7_f32": lambda: workloads.distill(rows=32, vocab=7, dtype="f32", peaked_frac=0.5),
}


@pytest.mark.parametrize("beta", BETAS)
@pytest.mark.parametrize("name", sorted(CASES))
def test_jsd_matches_oracle(name, beta):
    from gpu_helpers import say
    w = CASES[name]()
    say(f"[jsd] {name} beta={beta}")
    got = run_jsd(w, beta)
    wl, wd = check(w, got, beta, name)
    say(f"  worst loss error / bound {wl:.3f}, dstudent {wd:.3f}")


def test_jsd_identical_rows_are_zero():
    """Student == teacher: loss 0 and a zero gradient up to rounding, on
    peaked rows too (every beta)."""
    w = workloads.distill(rows=16, vocab=5000, dtype="f32", peaked_frac=0.5)
    w = dict(w, teacher=w["student"].copy(), labels=None, row_mask=None)
    for beta in BETAS:
        got = run_jsd(w, beta)
        assert np.all(np.abs(got["loss"]) <= 1e-6), (beta, got["loss"])
        assert np.all(np.abs(got["dstudent"]) <= 1e-7), beta


def test_jsd_tiny_vocab_and_ties():
    """V = 1 (every divergence 0), V = 2, and rows whose maximum is tied across
    several columns (the first one is the argmax)."""
    from gpu_helpers import say
    rng = np.random.default_rng(91)
    for V in (1, 2, 3):
        zs = rng.standard_normal((8, V)).astype(np.float32)
        zt = rng.standard_normal((8, V)).astype(np.float32)
        w = dict(student=zs, teacher=zt, labels=None, row_mask=None, temperature=1.0,
                 g=np.ones(8, np.float32))
        for beta in BETAS:
            check(w, run_jsd(w, beta), beta, f"V={V}")
    zs = rng.standard_normal((6, 300)).astype(np.float32)
    zt = rng.standard_normal((6, 300)).astype(np.float32)
    zs[0, [3, 100, 299]] = 9.0
    zs[1, [0, 1]] = 30.0
    zt[1, [0, 1]] = 30.0
    zs[2, [7, 8]] = 80.0
    zt[2, 150] = 60.0
    w = dict(student=zs, teacher=zt, labels=None, row_mask=None, temperature=0.8,
             g=rng.uniform(0.5, 1.5, 6).astype(np.float32))
    for beta in BETAS:
        got = run_jsd(w, beta)
        check(w, got, beta, "ties")
        sv = got["saved"].view(np.int32).reshape(6, 12)
        assert list(sv[:3, 6]) == [3, 0, 7]
    say("[jsd] ties ok")


def test_jsd_strides_masks_and_zero_sums():
    """Padded row strides (NaN canaries in the padding), masks and ignored
    labels, and every gradient row summing to zero up to output rounding."""
    for dtype, pad in (("f32", 4), ("bf16", 8)):
        w = workloads.distill(rows=48, vocab=3001, dtype=dtype, peaked_frac=0.3, temperature=1.3)
        V = 3001
        for beta in (0.0, 0.3, 1.0):
            got = run_jsd(w, beta, ss=V + pad + (-(V + pad)) % pad, ts=V + 2 * pad + (-(V + 2 * pad)) % pad)
            check(w, got, beta, f"strided {dtype}")
            d = got["dstudent"].astype(np.float64)
            rt = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
            assert np.all(np.abs(d.sum(1)) <= rt * np.abs(d).sum(1) + V * FLOOR), (dtype, beta)
            # rows that do not start 16-byte aligned take the scalar path
            odd = run_jsd(w, beta, ss=V + 1, ts=V + 3)
            check(w, odd, beta, f"unaligned {dtype}")


def test_jsd_peaked_rows_keep_signal():
    """Rows peaked by 20-80 with the teacher peaked elsewhere: the loss is
    large and positive and the gradient moves mass off the student's peak
    (wherever the error bound resolves that entry's sign: in between the KL
    ends a nearly disjoint pair is at the loss's maximum, where the gradient
    vanishes to far below the size of its terms); with the teacher peaked at
    the same column the gradient is tiny, zero-sum and not exactly zero (no
    collapse)."""
    w = workloads.distill(rows=32, vocab=151936, dtype="f32", peaked_frac=1.0)
    w = dict(w, labels=None, row_mask=None)
    T = w["temperature"]
    for beta in BETAS:
        got = run_jsd(w, beta)
        check(w, got, beta, "peaked")
        zs = w["student"].astype(np.float64)
        zt = w["teacher"].astype(np.float64)
        same = np.argmax(zs, 1) == np.argmax(zt, 1)
        d = got["dstudent"]
        a = np.argmax(zs, 1)
        if beta < 1.0:
            resolved = 0
            for r in np.nonzero(~same)[0]:
                _, _, dref, bd = row_bounds(w["student"][r], w["teacher"][r],
                                            float(w["g"][r]), T, beta)
                if dref[a[r]] > bd[a[r]] + 2 * FLOOR:
                    assert d[r, a[r]] > 0, (beta, r, d[r, a[r]], dref[a[r]])
                    resolved += 1
            assert resolved >= (~same).sum() // 2, (beta, resolved)
        assert np.all(np.abs(d[same]).max(1) > 0), beta
        if beta in (0.0, 1.0):
            assert np.all(got["loss"][~same] > 1.0), beta
        else:
            # nearly disjoint supports: the maximum, the binary entropy of beta
            h = -beta * np.log(beta) - (1 - beta) * np.log(1 - beta)
            assert np.all(np.abs(got["loss"][~same] - h) <= 1e-3 * h), (beta, got["loss"][~same])


def test_jsd_determinism():
    w = workloads.distill(rows=20, vocab=20011, dtype="bf16", peaked_frac=0.3)
    for beta in (0.0, 0.5):
        a = run_jsd(w, beta)
        b = run_jsd(w, beta)
        for k in ("loss", "dstudent", "saved"):
            assert np.array_equal(a[k], b[k]), (beta, k)


def test_jsd_record_carries_argmax_entry():
    """The forward stores the student-argmax gradient entry (per unit of g/T)
    for beta < 1 unless the student's mass off its argmax is below V 2^-80,
    where the fp32 sums behind it lose terms; the backward then takes those
    rows one workgroup each.  Checked against the oracle's mass and entry."""
    w = workloads.distill(rows=40, vocab=3001, dtype="f32", peaked_frac=0.5)
    w = dict(w, labels=None, row_mask=None)
    V = 3001
    T = w["temperature"]
    for beta in BETAS:
        got = run_jsd(w, beta)
        check(w, got, beta, "record")
        rec = got["saved"].view(np.int32).reshape(40, 12)
        flags = rec[:, 7]
        garg = got["saved"].view(np.float32).reshape(40, 12)[:, 5]
        seen = set()
        for r in range(40):
            zs, zt = w["student"][r], w["teacher"][r]
            _, _, ls, _, _ = oj.jsd_row(zs, zt, T, beta)
            a = int(np.argmax(oj._widen(zs)))
            g0 = -np.expm1(ls[a])
            assert flags[r] & 1, (beta, r)
            if beta == 1.0:
                assert not flags[r] & 2, (beta, r)
                continue
            lim = V * 2.0 ** -80
            if g0 >= 2 * lim:
                assert flags[r] & 2, (beta, r, g0)
                # g = T: the entry per unit of g/T, against the entry's error bound
                _, _, dref, bd = row_bounds(zs, zt, T, T, beta)
                assert abs(garg[r] - dref[a]) <= 1.2e-7 * abs(dref[a]) + bd[a] + FLOOR, (beta, r)
                seen.add(True)
            elif g0 <= lim / 2:
                assert not flags[r] & 2, (beta, r, g0)
                seen.add(False)
        if beta < 1.0:
            assert seen == {True, False}, (beta, seen)


def test_jsd_near_end_betas():
    """beta within 1e-6 of either end takes the mixture path: the teacher's
    weight beta rides in its exponent as log2(1e-6), and 1 - beta folds into
    the backward's exponent; both against the oracle's error model."""
    from gpu_helpers import say
    for name in ("distill_64x4099_f32_ragged", "distill_24x151936_bf16_peaked_T0.7"):
        w = CASES[name]()
        for beta in (1e-6, 1.0 - 1e-6):
            got = run_jsd(w, beta)
            wl, wd = check(w, got, beta, name)
            say(f"[jsd] {name} beta={beta}: worst loss error / bound {wl:.3f}, dstudent {wd:.3f}")
