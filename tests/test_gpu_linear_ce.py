"""Linear cross-entropy (logits = hidden x head^T on the matrix cores) against
the fp64 oracle.

Exact-contraction inputs: every hidden and head value lies on a 1/16 grid
(peaked rows on a 1/256 grid) with magnitude below 1, so every product and
every partial sum of a logit is exactly representable in fp32, whatever order
the MFMA accumulates in.  The GPU's logits then equal the oracle's, and loss,
log p, entropy and argmax are held to the same bars as ce_forward.  dlogits is
kept in bf16 by design, so dlogits is held to the bf16 bar (4e-3 relative plus
2^-126) and dhidden / dhead to that bar carried through the product:
4.5e-3 sum |dlogits| |operand| + 2^-126 sum |operand| (one bf16 rounding,
2^-8 relative, plus fp32 accumulation over at most V / 16 MFMA steps, below
6e-4 here; the floor covers fp32-subnormal probabilities flushed to 0).

Random bf16 inputs: the logits carry the fp32 accumulation error of the
product, at most (H / 16 + 2) 2^-24 sum_k |h_k w_jk| per logit (one rounding
per 16-deep MFMA step), which moves the loss by at most twice that over T.
"""
import numpy as np
import pytest
import torch

import cross_entropy_vocab_amd as cev
import oracle
import workloads
from tolerance import FLOOR, RTOL, SUBNORMAL, assert_close

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def grid_case(R, H, V, seed, T=1.0, peaked=0, n_ignored=0, mask_frac=0.0, margins=(17, 30, 50, 80)):
    """Exact-contraction inputs (bf16 bit patterns) and labels."""
    rng = np.random.default_rng([seed, 4242])
    w = (rng.integers(-15, 16, (V, H)) / 16.0).astype(np.float32)
    h = (rng.integers(-15, 16, (R, H)) / 16.0).astype(np.float32)
    labels = rng.integers(0, V, R).astype(np.int64)
    rows = rng.permutation(R)
    for i, r in enumerate(rows[:peaked]):
        # h = (m / 16) w_t: logits are exact multiples of 2^-12; pick m so the
        # target leads the others by at least the wanted margin.
        t = labels[r]
        zt = float(w[t].astype(np.float64) @ w[t])
        others = w.astype(np.float64) @ w[t]
        others[t] = -np.inf
        gap = zt - others.max()
        want = margins[i % len(margins)]
        m = int(min(17, max(1, np.ceil(want * 16 * T / gap))))
        h[r] = (m / 16.0) * w[t]
    labels[rows[peaked:peaked + n_ignored]] = -100
    mask = None
    if mask_frac:
        mask = (rng.random(R) >= mask_frac).astype(np.uint8)
    g = rng.standard_normal(R).astype(np.float32)
    return dict(hidden=workloads.bf16_bits(h), weight=workloads.bf16_bits(w), labels=labels,
                row_mask=mask, temperature=T, g=g)


def padded_dev(bits, stride):
    from gpu_helpers import DEV
    R, H = bits.shape
    buf = np.full((R, stride), 0x7FC1, dtype=np.uint16)     # NaN canaries in the padding
    buf[:, :H] = bits
    return torch.from_numpy(buf.view(np.int16)).to(DEV).view(torch.bfloat16)[:, :H]


def run_lce(w, eps=0.0, entropy=True, dweight=True, hs=None, ws=None, logits=None):
    from gpu_helpers import DEV, to_dev, to_host
    R, H = w["hidden"].shape
    V = w["weight"].shape[0]
    hid = to_dev(w["hidden"]) if hs is None else padded_dev(w["hidden"], hs)
    wt = to_dev(w["weight"]) if ws is None else padded_dev(w["weight"], ws)
    labels = to_dev(w["labels"])
    mask = None if w.get("row_mask") is None else to_dev(w["row_mask"])
    g = to_dev(np.asarray(w["g"], np.float32))
    T = w["temperature"]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = cev.lce_forward(hid, wt, labels, T, row_mask=mask, label_smoothing=eps,
                          entropy=entropy, argmax=True, status=status, logits=logits)
    dh, dw = cev.lce_backward(hid, wt, labels, g, out["saved"], T, row_mask=mask,
                              label_smoothing=eps, dweight=dweight, status=status,
                              workspace=out["workspace"], logits=out["logits"])
    torch.cuda.synchronize()
    ldd = (V + 63) // 64 * 64
    dl = out["workspace"][:R * ldd * 2].view(torch.bfloat16).view(R, ldd)
    res = {k: to_host(v) for k, v in out.items() if v is not None and k != "workspace"}
    res.update(dhidden=dh.cpu().numpy(), dweight=None if dw is None else dw.cpu().numpy(),
               dlogits=to_host(dl), status=int(status.item()))
    return res


def check_exact(w, got, name, eps=0.0, entropy=True):
    T = w["temperature"]
    R, H = w["hidden"].shape
    V = w["weight"].shape[0]
    tol = RTOL["f32"]
    ref = oracle.linear_ce_rows(w["hidden"], w["weight"], w["labels"], T,
                                row_mask=w.get("row_mask"), label_smoothing=eps)
    # (rows peaked past ~90 nats have fp32-subnormal log p: half a subnormal step)
    assert_close(f"{name} logp", got["logp"], ref["logp"], tol["logp"], SUBNORMAL)
    assert_close(f"{name} loss", got["loss"], ref["loss"], tol["loss"], SUBNORMAL)
    if entropy:
        # A row peaked on a non-target class has q ~ 1 and H ~ log S tiny: the
        # fp32-accumulated S (relative error ~1e-7) then moves H by ~1e-7
        # absolute whatever its size, so such rows also get 2e-6 q absolute.
        err = np.abs(got["entropy"] - ref["entropy"])
        bound = tol["entropy"] * np.abs(ref["entropy"]) + 2e-6 * ref["q"] + 1e-30
        assert np.all(err <= bound), (name, "entropy", float(np.max(err / bound)))
    assert np.array_equal(got["argmax"], ref["argmax"]), name
    # the saved maximum is the exact largest logit
    z = oracle.linear_logits(w["hidden"], w["weight"])
    vr, _ = oracle.valid_rows(w["labels"], w.get("row_mask"), V)
    mz = got["saved"].view(np.float32).reshape(R, 4)[:, 0]
    assert np.array_equal(mz[vr].astype(np.float64), z[vr].max(axis=1)), name
    # dlogits (bf16 scratch) at the bf16 bar; its padding columns are zero
    dref = oracle.ce_grad_rows(z, w["labels"], np.asarray(w["g"], np.float64), T,
                               row_mask=w.get("row_mask"), label_smoothing=eps)
    # smoothing makes some entries differences of two terms: the fp32 value errs
    # relative to the terms (TERM_RTOL of their size), then bf16 rounds it
    from test_gpu_smoothing_topk import TERM_RTOL
    mag = np.abs(oracle.ce_grad_rows(z, w["labels"], np.asarray(w["g"], np.float64), T,
                                     row_mask=w.get("row_mask")))
    gt = np.zeros(R)
    gt[vr] = np.abs(np.asarray(w["g"], np.float64)[vr]) / T
    mag += gt[:, None] * (eps / V)
    mag[vr, w["labels"][vr]] += gt[vr] * eps
    err = np.abs(got["dlogits"][:, :V] - dref)
    bound = RTOL["bf16"]["dlogits"] * np.abs(dref) + TERM_RTOL * mag + FLOOR
    assert np.all(err <= bound), (name, "dlogits", float(np.max(err / bound)))
    assert np.all(got["dlogits"][:, V:] == 0)
    grads = oracle.linear_ce_grads(w["hidden"], w["weight"], w["labels"],
                                   np.asarray(w["g"], np.float64), T, row_mask=w.get("row_mask"),
                                   label_smoothing=eps)
    hw = oracle._widen(w["weight"])
    hh = oracle._widen(w["hidden"])
    # each dlogits entry carries the bf16 bar's 2^-126 floor too (fp32-subnormal
    # probabilities of peaked rows flush to 0), summed through the product
    valid = np.zeros(R)
    valid[vr] = 1.0
    bh = 4.5e-3 * (np.abs(dref) @ np.abs(hw)) + FLOOR * (valid[:, None] * np.abs(hw).sum(0)) \
        + FLOOR
    err = np.abs(got["dhidden"] - grads["dhidden"])
    i = np.unravel_index(np.argmax(err / bh), err.shape)
    assert np.all(err <= bh), (name, "dhidden", float(np.max(err / bh)), i,
                               float(np.abs(dref[i[0]]).max()))
    if got["dweight"] is not None:
        bw = 4.5e-3 * (np.abs(dref).T @ np.abs(hh)) + FLOOR * (valid @ np.abs(hh))[None, :] \
            + FLOOR
        err = np.abs(got["dweight"] - grads["dweight"])
        assert np.all(err <= bw), (name, "dweight", float(np.max(err / bw)))


EXACT = {
    "200x128x1000": dict(R=200, H=128, V=1000, seed=1, n_ignored=9),
    "300x256x4099_T0.7": dict(R=300, H=256, V=4099, seed=2, T=0.7, mask_frac=0.1),
    "130x512x32769_peaked_T0.9": dict(R=130, H=512, V=32769, seed=3, T=0.9, peaked=60),
    "64x64x7": dict(R=64, H=64, V=7, seed=4, n_ignored=3),
    "1x192x300": dict(R=1, H=192, V=300, seed=5),
    "257x1024x2053_peaked": dict(R=257, H=1024, V=2053, seed=6, peaked=40, mask_frac=0.05),
}


@pytest.mark.parametrize("name", sorted(EXACT))
def test_lce_exact_contraction(name):
    from gpu_helpers import say
    say(f"[lce exact] {name}")
    w = grid_case(**EXACT[name])
    got = run_lce(w)
    check_exact(w, got, name)
    assert got["status"] == 0


def test_lce_exact_smoothing_and_strides():
    from gpu_helpers import say
    say("[lce exact] smoothing 0.1, padded strides")
    w = grid_case(R=150, H=192, V=3001, seed=7, T=1.1, peaked=30, n_ignored=5)
    got = run_lce(w, eps=0.1, hs=200, ws=264)
    check_exact(w, got, "smoothing+strides", eps=0.1)


def test_lce_exact_wide_hidden_stride():
    """A hidden row stride of 2^24 + 64 elements: the operand copies that read
    hidden (both logit products, and the head gradient's B operand) take
    clamped per-lane addresses instead of an SGPR base with 32-bit offsets."""
    from gpu_helpers import say
    say("[lce exact] hidden stride 2^24 + 64")
    w = grid_case(R=3, H=64, V=300, seed=9, n_ignored=1)
    got = run_lce(w, hs=(1 << 24) + 64)
    check_exact(w, got, "wide hidden stride")


def test_lce_bad_labels_and_determinism():
    w = grid_case(R=70, H=64, V=500, seed=8)
    w["labels"][3] = 500
    w["labels"][9] = -5
    got = run_lce(w)
    assert got["status"] & cev.STATUS_BAD_LABEL
    assert got["loss"][3] == 0 and got["argmax"][9] == -1
    assert np.all(got["dhidden"][[3, 9]] == 0)
    w2 = dict(w, labels=np.where((w["labels"] < 0) | (w["labels"] >= 500), -100, w["labels"]))
    check_exact(w2, got, "bad labels")
    again = run_lce(w)
    for k in ("loss", "logp", "entropy", "argmax", "saved", "dhidden", "dweight"):
        assert np.array_equal(again[k], got[k]), k


def test_lce_random_bf16_bound():
    """Realistic bf16 inputs: the loss within the derived fp32-product bound,
    argmax among the columns the bound cannot separate from the maximum."""
    from gpu_helpers import say
    say("[lce random] 200x2560x6000 bf16")
    w = workloads.linear(rows=200, hidden=2560, vocab=6000, peaked_frac=0.25)
    R, H = w["hidden"].shape
    T = w["temperature"]
    got = run_lce(w, dweight=False)
    ref = oracle.linear_ce_rows(w["hidden"], w["weight"], w["labels"], T, row_mask=w["row_mask"])
    z = oracle.linear_logits(w["hidden"], w["weight"])
    absz = np.abs(oracle._widen(w["hidden"])) @ np.abs(oracle._widen(w["weight"])).T
    dz = (H / 16 + 2) * U * absz.max(axis=1)               # per-row logit error bound
    vr, _ = oracle.valid_rows(w["labels"], w["row_mask"], w["weight"].shape[0])
    err = np.abs(got["loss"][vr] - ref["loss"][vr])
    bound = 2e-6 * np.abs(ref["loss"][vr]) + 2 * dz[vr] / T
    assert np.all(err <= bound), float(np.max(err / bound))
    for r in vr:
        top = z[r].max()
        assert z[r, got["argmax"][r]] >= top - 2 * dz[r], r
    say(f"  worst loss error / bound: {float(np.max(err / bound)):.3f}")


STORED = {
    "1x192x300": dict(R=1, H=192, V=300, seed=5),
    "70x64x3": dict(R=70, H=64, V=3, seed=10, n_ignored=2),
    "200x128x1000": dict(R=200, H=128, V=1000, seed=1, n_ignored=9),
    "300x256x4099_T0.7": dict(R=300, H=256, V=4099, seed=2, T=0.7, mask_frac=0.1),
    "64x64x7": dict(R=64, H=64, V=7, seed=4, n_ignored=3),
    "257x1024x2053_peaked": dict(R=257, H=1024, V=2053, seed=6, peaked=40, mask_frac=0.05),
}


@pytest.mark.parametrize("name", sorted(STORED))
def test_lce_stored_logits_exact(name):
    """The forward's stored logits equal the exact product (the oracle's), and
    a backward that reads them back gives the recomputing backward's dlogits,
    dhidden and dhead bit for bit (both apply one formula to one fp32 value)."""
    from gpu_helpers import say
    say(f"[lce stored logits] {name}")
    w = grid_case(**STORED[name])
    V = w["weight"].shape[0]
    ref = run_lce(w)
    got = run_lce(w, logits=True)
    z = oracle.linear_logits(w["hidden"], w["weight"])
    assert np.array_equal(got["logits"].astype(np.float64), z), name
    for k in ("loss", "logp", "entropy", "argmax", "saved", "dlogits", "dhidden", "dweight"):
        assert np.array_equal(got[k], ref[k]), (name, k)
    check_exact(w, got, name + " stored")
    assert got["status"] == 0


def test_lce_stored_logits_strided_smoothing():
    """A caller-owned logits buffer with a padded row stride (its padding left
    untouched) under label smoothing and padded operand strides."""
    from gpu_helpers import DEV, say
    say("[lce stored logits] stride 3012, smoothing 0.1")
    w = grid_case(R=150, H=192, V=3001, seed=7, T=1.1, peaked=30, n_ignored=5)
    R, V = 150, 3001
    buf = torch.full((R, 3012), 7.5, dtype=torch.float32, device=DEV)
    ref = run_lce(w, eps=0.1, hs=200, ws=264)
    got = run_lce(w, eps=0.1, hs=200, ws=264, logits=buf[:, :V])
    z = oracle.linear_logits(w["hidden"], w["weight"])
    assert np.array_equal(buf[:, :V].cpu().numpy().astype(np.float64), z)
    assert bool((buf[:, V:] == 7.5).all())
    for k in ("loss", "logp", "entropy", "argmax", "saved", "dlogits", "dhidden", "dweight"):
        assert np.array_equal(got[k], ref[k]), k


def test_lce_stored_logits_random_bf16_identical():
    """Random bf16 inputs: the stored logits are the forward's own fp32 sums,
    and the backward reading them matches the recomputing one bit for bit
    (the product is summed in one order by both)."""
    from gpu_helpers import say
    say("[lce stored logits] random 200x2560x6000 bf16")
    w = workloads.linear(rows=200, hidden=2560, vocab=6000, peaked_frac=0.25)
    ref = run_lce(w, dweight=True)
    got = run_lce(w, dweight=True, logits=True)
    for k in ("loss", "logp", "entropy", "argmax", "saved", "dlogits", "dhidden", "dweight"):
        assert np.array_equal(got[k], ref[k]), k
    # the stored logits within the product's fp32 bound of the exact ones
    H = w["hidden"].shape[1]
    z = oracle.linear_logits(w["hidden"], w["weight"])
    absz = np.abs(oracle._widen(w["hidden"])) @ np.abs(oracle._widen(w["weight"])).T
    assert np.all(np.abs(got["logits"] - z) <= (H / 16 + 2) * U * absz + 1e-30)


def test_lce_caller_owned_dweight():
    """A caller-owned dhead buffer (NaN-filled beforehand) receives the same
    values, bit for bit, as the one the binding allocates."""
    from gpu_helpers import DEV, to_dev
    w = grid_case(R=90, H=128, V=1100, seed=12, n_ignored=4)
    hid, wt = to_dev(w["hidden"]), to_dev(w["weight"])
    labels, g = to_dev(w["labels"]), to_dev(np.asarray(w["g"], np.float32))
    out = cev.lce_forward(hid, wt, labels, 1.0)
    _, dw = cev.lce_backward(hid, wt, labels, g, out["saved"], 1.0, dweight=True,
                             workspace=out["workspace"])
    mine = torch.full((1100, 128), float("nan"), dtype=torch.float32, device=DEV)
    _, dw2 = cev.lce_backward(hid, wt, labels, g, out["saved"], 1.0, dweight=mine,
                              workspace=out["workspace"])
    torch.cuda.synchronize()
    assert dw2 is mine
    assert torch.equal(mine, dw)
