"""Label smoothing (ce_forward / ce_backward / ce_fused) and the top-K backward
(sls_topk_forward's q and saved record, sls_topk_backward) against the fp64
oracle, element by element.

Where the result is a difference of two terms (p_j - eps/V next to a smoothed
label; G_j q_j - p_j (Gs - G_j) at a gathered column) the fp32 arithmetic errs
relative to the terms, not to their difference, so those elements are held to
the dtype's bound on |ref| plus 2e-6 of the terms' magnitude (about ten times
the few fp32 roundings involved); every other element keeps the plain bound."""
import numpy as np
import pytest
import torch

import cross_entropy_vocab_amd as cev
import oracle
import workloads
from tolerance import FLOOR, RTOL, assert_close, assert_row_sums

pytestmark = pytest.mark.gpu

TERM_RTOL = 2e-6


def _kind(w):
    return "bf16" if w["logits"].dtype == np.uint16 else "f32"


def _rand_case(rows, V, dtype="f32", T=1.0, seed=0, scale=3.0, n_ignored=0, mask_frac=0.0):
    rng = np.random.default_rng([seed, 77])
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


def _assert_within(name, got, ref, bound):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bad = ~(err <= bound)
    if np.any(bad):
        i = np.unravel_index(np.argmax(np.where(bad, err - bound, -np.inf)), err.shape)
        raise AssertionError(f"{name}: {int(bad.sum())} of {bad.size} outside the bound; worst "
                             f"at {i}: got {got[i]!r} ref {ref[i]!r} bound {bound[i]!r}")


# ---------------------------------------------------------------------------
# label smoothing

def _smoothed_grad_bound(w, eps):
    """|ref| rtol + (|unsmoothed gradient| + |g/T| eps/V, and + |g/T| eps at the
    target) * TERM_RTOL + the subnormal floor."""
    R, V = w["logits"].shape
    T = w["temperature"]
    g = np.asarray(w["g"], np.float64)
    d0 = oracle.ce_grad_rows(w["logits"], w["labels"], g, T, row_mask=w.get("row_mask"))
    vr, _ = oracle.valid_rows(w["labels"], w.get("row_mask"), V)
    gt = np.zeros(R)
    gt[vr] = np.abs(g[vr]) / T
    mag = np.abs(d0) + gt[:, None] * (eps / V)
    mag[vr, w["labels"][vr]] += gt[vr] * eps
    return mag, vr


SMOOTH_CASES = {
    "tiny_64x4096_f32": lambda: workloads.tiny(),
    "grpo_40x152064_bf16_mask": lambda: workloads.grpo(rows=40, vocab=152064),
    "chunk_24x32781_bf16_T0.7": lambda: dict(workloads.chunk(rows=24, vocab=32781),
                                             g=np.random.default_rng(5).standard_normal(24)
                                             .astype(np.float32)),
    "peaked_24x151936_f32_T0.9": lambda: workloads.peaked("f32", 0.9, rows=24),
    "peaked_16x151936_bf16_T1": lambda: workloads.peaked("bf16", 1.0, rows=16),
    "odd_9x17_f32": lambda: _rand_case(9, 17, "f32", T=0.8, seed=17, n_ignored=2),
    "odd_9x3_bf16": lambda: _rand_case(9, 3, "bf16", T=1.2, seed=3, n_ignored=1),
    "single_9x1_f32": lambda: _rand_case(9, 1, "f32", seed=1, n_ignored=2),
}


@pytest.mark.parametrize("eps", [0.1, 1.0])
@pytest.mark.parametrize("name", sorted(SMOOTH_CASES))
def test_label_smoothing_matches_oracle(name, eps):
    from gpu_helpers import run_ce, say
    w = SMOOTH_CASES[name]()
    if "g" not in w:
        w["g"] = np.random.default_rng(9).standard_normal(w["logits"].shape[0]).astype(np.float32)
    say(f"[smoothing] {name} eps={eps}")
    tol = RTOL[_kind(w)]
    T = w["temperature"]
    got = run_ce(w, label_smoothing=eps)
    plain = run_ce(w)
    ref = oracle.ce_rows(w["logits"], w["labels"], T, row_mask=w.get("row_mask"),
                         label_smoothing=eps)
    e_loss = assert_close(f"{name} smoothed loss", got["loss"], ref["loss"], tol["loss"])
    # smoothing changes only the loss and the gradient: log p, entropy, argmax
    # and the saved record are bit-identical to the unsmoothed call
    for k in ("logp", "entropy", "argmax", "saved", "valid_rows", "n_valid"):
        assert np.array_equal(got[k], plain[k]), k
    dref = oracle.ce_grad_rows(w["logits"], w["labels"], np.asarray(w["g"], np.float64), T,
                               row_mask=w.get("row_mask"), label_smoothing=eps)
    mag, vr = _smoothed_grad_bound(w, eps)
    _assert_within(f"{name} smoothed dlogits", got["dlogits"], dref,
                   tol["dlogits"] * np.abs(dref) + TERM_RTOL * mag + FLOOR)
    assert_row_sums(f"{name} smoothed dlogits", got["dlogits"], tol["dlogits"])
    valid = np.zeros(w["logits"].shape[0], bool)
    valid[vr] = True
    assert np.all(got["dlogits"][~valid] == 0) and np.all(got["loss"][~valid] == 0)
    assert got["status"] == 0
    say(f"  max rel err smoothed loss {e_loss:.2e}")


@pytest.mark.parametrize("rows,V,dtype", [(3, 151936, "f32"), (12, 152064, "bf16")])
def test_label_smoothing_split_rows(rows, V, dtype):
    """Few long rows take the split sweep, whose merge sums the parts' value
    sums; the smoothed loss matches the oracle and the whole-row sweep."""
    from test_gpu_edges import _ce_raw
    w = _rand_case(rows, V, dtype, T=0.9, seed=rows, n_ignored=rows // 8)
    full = cev.workspace_size(rows, V, 1 if dtype == "bf16" else 0)
    split = _ce_raw(w, full, eps=0.2)
    whole = _ce_raw(w, 0, eps=0.2)
    ref = oracle.ce_rows(w["logits"], w["labels"], 0.9, label_smoothing=0.2)
    tol = RTOL[dtype]
    assert_close("split smoothed loss", split["loss"], ref["loss"], tol["loss"])
    assert_close("whole smoothed loss", whole["loss"], ref["loss"], tol["loss"])


@pytest.mark.parametrize("name", ["grpo_40x152064_bf16_mask", "peaked_24x151936_f32_T0.9",
                                  "odd_9x17_f32"])
def test_label_smoothing_fused(name):
    """ce_fused with smoothing: its loss and dlogits match the oracle and agree
    with the separate calls."""
    from gpu_helpers import to_dev, to_host
    w = SMOOTH_CASES[name]()
    if "g" not in w:
        w["g"] = np.random.default_rng(9).standard_normal(w["logits"].shape[0]).astype(np.float32)
    eps = 0.1
    tol = RTOL[_kind(w)]
    T = w["temperature"]
    mask = None if w.get("row_mask") is None else to_dev(w["row_mask"])
    out = cev.ce_fused(to_dev(w["logits"]), to_dev(w["labels"]), to_dev(w["g"]), T,
                       row_mask=mask, label_smoothing=eps)
    torch.cuda.synchronize()
    ref = oracle.ce_rows(w["logits"], w["labels"], T, row_mask=w.get("row_mask"),
                         label_smoothing=eps)
    assert_close(f"{name} fused smoothed loss", to_host(out["loss"]), ref["loss"], tol["loss"])
    dref = oracle.ce_grad_rows(w["logits"], w["labels"], np.asarray(w["g"], np.float64), T,
                               row_mask=w.get("row_mask"), label_smoothing=eps)
    mag, _ = _smoothed_grad_bound(w, eps)
    dl = to_host(out["dlogits"])
    _assert_within(f"{name} fused smoothed dlogits", dl, dref,
                   tol["dlogits"] * np.abs(dref) + TERM_RTOL * mag + FLOOR)
    assert_row_sums(f"{name} fused smoothed dlogits", dl, tol["dlogits"])


# ---------------------------------------------------------------------------
# top-K backward

def _topk_bound(w, idx, g, ignore_index=-100):
    """Per-element bound for the top-K gradient: rtol |ref| everywhere, plus
    TERM_RTOL (|G_j| q_j + p_j |Gs - G_j|) / T at each gathered column."""
    R, V = w["logits"].shape
    T = w["temperature"]
    mask = w.get("row_mask")
    lp, q, _ = oracle.topk_rows(w["logits"], idx, T, row_mask=mask, want_q=True)
    extra = np.zeros((R, V))
    for r in range(R):
        if mask is not None and mask[r] == 0:
            continue
        ok = (idx[r] != ignore_index) & (idx[r] >= 0) & (idx[r] < V)
        gs = float(np.sum(g[r][ok], dtype=np.float64))
        for j in np.unique(idx[r][ok]):
            sel = ok & (idx[r] == j)
            gj = float(np.sum(g[r][sel], dtype=np.float64))
            k = int(np.argmax(sel))
            pj = float(np.exp(lp[r, k]))
            extra[r, j] = (abs(gj) * q[r, k] + pj * abs(gs - gj)) / T
    return extra


def _check_topk(w, idx, g, got, name, ignore_index=-100):
    tol = RTOL[_kind(w)]
    T = w["temperature"]
    mask = w.get("row_mask")
    lp_ref, q_ref, st = oracle.topk_rows(w["logits"], idx, T, row_mask=mask, want_q=True)
    assert_close(f"{name} topk logp", got["logp"], lp_ref, tol["topk"])
    assert_close(f"{name} topk q", got["q"], q_ref, tol["topk"])
    dref = oracle.topk_grad_rows(w["logits"], idx, np.asarray(g, np.float64), T, row_mask=mask)
    extra = _topk_bound(w, idx, g)
    _assert_within(f"{name} topk dlogits", got["dlogits"], dref,
                   tol["dlogits"] * np.abs(dref) + TERM_RTOL * extra + FLOOR)
    assert_row_sums(f"{name} topk dlogits", got["dlogits"], tol["dlogits"])
    if mask is not None:
        assert np.all(got["dlogits"][mask == 0] == 0)
    return st


def test_topk_backward_chunk_workload():
    from gpu_helpers import run_topk_fb, say
    w = workloads.chunk(rows=40, vocab=32768)
    g = np.random.default_rng([6, 40]).standard_normal(w["indices"].shape).astype(np.float32)
    say("[topk bwd] chunk 40x32768 bf16 K=8 T=0.7")
    got = run_topk_fb(w, w["indices"], g)
    assert _check_topk(w, w["indices"], g, got, "chunk") == 0 and got["status"] == 0


def test_topk_backward_duplicates_ignored_bad_and_masked():
    from gpu_helpers import run_topk_fb
    w = _rand_case(10, 5000, "bf16", T=0.7, seed=10, mask_frac=0.2)
    w["row_mask"][0] = 1
    w["row_mask"][4] = 1
    rng = np.random.default_rng(11)
    idx = rng.integers(0, 5000, (10, 12)).astype(np.int64)
    idx[:, 3] = idx[:, 1]          # duplicate column: its g values add
    idx[0, 4] = idx[0, 1]          # three entries at one column
    idx[2, 5] = -100               # ignored entry
    idx[4, 0] = 5000               # out of range
    idx[6, 7] = -3                 # out of range
    g = rng.standard_normal((10, 12)).astype(np.float32)
    got = run_topk_fb(w, idx, g)
    _check_topk(w, idx, g, got, "dup")
    assert got["status"] & cev.STATUS_BAD_INDEX


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_topk_backward_lane_form_boundary(dtype):
    """K = 64 (tiles with the entries held in lanes) and K = 65 (the general
    kernel): against the oracle, and equal bit for bit on the shared entries,
    with duplicates (three at one column), an ignored entry, bad entries,
    masked rows, and gathered columns in the first and last vector of a row
    and on a tile boundary."""
    from gpu_helpers import run_topk_fb
    R, V = 12, 12288
    w = _rand_case(R, V, dtype, T=0.9, seed=51, mask_frac=0.25)
    w["row_mask"][:4] = 1
    w["row_mask"][5] = 0
    rng = np.random.default_rng(52)
    idx = np.stack([rng.choice(V, 64, replace=False) for _ in range(R)]).astype(np.int64)
    idx[:, 0] = 0
    idx[:, 1] = V - 1
    tile = 512 * (8 if dtype == "bf16" else 4)    # columns per 256 x 2 tile
    idx[:, 2] = tile * (1 + np.arange(R) % 2) - np.arange(R) % 2   # a tile's last or first column
    idx[:, 3] = idx[:, 5]
    idx[0, 4] = idx[0, 5]
    idx[2, 9] = -100
    idx[3, 10] = V
    g = rng.standard_normal((R, 64)).astype(np.float32)
    got64 = run_topk_fb(w, idx, g)
    _check_topk(w, idx, g, got64, "K=64")
    idx65 = np.concatenate([idx, np.full((R, 1), -100, np.int64)], axis=1)
    g65 = np.concatenate([g, rng.standard_normal((R, 1)).astype(np.float32)], axis=1)
    got65 = run_topk_fb(w, idx65, g65)
    _check_topk(w, idx65, g65, got65, "K=65")
    assert got64["status"] & cev.STATUS_BAD_INDEX and got65["status"] & cev.STATUS_BAD_INDEX
    assert np.array_equal(got64["dlogits"], got65["dlogits"])


def test_topk_backward_peaked_large_k():
    """K = 100 on peaked rows with the peak gathered: the peak's gradient is
    G q - p (Gs - G) without cancellation in 1 - p."""
    from gpu_helpers import run_topk_fb
    w = workloads.peaked("f32", 0.9, rows=12, vocab=20000)
    rng = np.random.default_rng(12)
    idx = np.stack([rng.choice(20000, 100, replace=False) for _ in range(12)]).astype(np.int64)
    idx[:, 50] = w["labels"]
    clash = idx[:, 49] == w["labels"]
    idx[clash, 49] = (w["labels"][clash] + 1) % 20000
    g = rng.standard_normal((12, 100)).astype(np.float32)
    g[:3] = 0.0
    g[:3, 50] = 1.0                # rows whose only weight sits on the peak
    got = run_topk_fb(w, idx, g)
    _check_topk(w, idx, g, got, "peaked K=100")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("stride,dstride", [(1003, 1001), (1003, 1003), (1000, 1000)])
def test_topk_backward_strides(dtype, stride, dstride):
    """Rows at every alignment (element path when logits and dlogits rows
    disagree modulo 16 bytes, vector path with a peeled head otherwise),
    padding untouched."""
    from gpu_helpers import run_topk_fb, strided_dev
    w = _rand_case(11, 1000, dtype, T=1.1, seed=stride + dstride)
    rng = np.random.default_rng(stride)
    idx = rng.integers(0, 1000, (11, 6)).astype(np.int64)
    idx[:, 0] = [0, 1, 2, 3, 996, 997, 998, 999, 7, 8, 500]   # head and tail columns
    g = rng.standard_normal((11, 6)).astype(np.float32)
    got = run_topk_fb(w, idx, g, logits_dev=strided_dev(w["logits"], stride), dl_stride=dstride)
    _check_topk(w, idx, g, got, f"strides {stride}/{dstride}")


def test_topk_backward_k1_label_equals_ce_backward():
    """K = 1 at the label with weight g is ce_backward with weight -g (the
    gradient of log p_t is minus that of the loss)."""
    from gpu_helpers import run_ce, run_topk_fb
    w = _rand_case(16, 32768, "f32", T=0.8, seed=21)
    g = np.random.default_rng(22).standard_normal((16, 1)).astype(np.float32)
    got = run_topk_fb(w, w["labels"][:, None], g)
    ce = run_ce(dict(w, g=-g[:, 0]), entropy=False, argmax=False)
    assert_close("K=1 vs ce logp", got["logp"][:, 0], ce["logp"].astype(np.float64), 1e-6)
    # each kernel rounds its own log2 d (about 16 here, fp32 spacing 2^-19) and
    # its own exponent offset: up to ~4 such roundings apart, ~5e-6 in p
    assert_close("K=1 vs ce dlogits", got["dlogits"], ce["dlogits"], 1e-5, FLOOR)


def test_topk_backward_k1024_many_duplicates_and_determinism():
    from gpu_helpers import run_topk_fb
    w = _rand_case(4, 3000, "bf16", T=1.0, seed=31)
    rng = np.random.default_rng(32)
    idx = rng.integers(0, 3000, (4, 1024)).astype(np.int64)
    idx[1, ::7] = -100
    g = rng.standard_normal((4, 1024)).astype(np.float32)
    got = run_topk_fb(w, idx, g)
    _check_topk(w, idx, g, got, "K=1024")
    again = run_topk_fb(w, idx, g)
    assert np.array_equal(again["dlogits"], got["dlogits"])
    assert np.array_equal(again["q"], got["q"])


def test_topk_backward_zero_weights_and_empty():
    from gpu_helpers import DEV, run_topk_fb, to_dev
    w = _rand_case(5, 700, "f32", seed=41)
    idx = np.random.default_rng(42).integers(0, 700, (5, 3)).astype(np.int64)
    got = run_topk_fb(w, idx, np.zeros((5, 3), np.float32))
    assert np.all(got["dlogits"] == 0)
    logits = torch.empty((0, 700), device=DEV)
    i0 = torch.empty((0, 3), dtype=torch.int64, device=DEV)
    lp, q, sv = cev.sls_topk_forward(logits, i0, saved=True)
    dl = cev.sls_topk_backward(logits, i0, torch.empty((0, 3), device=DEV), sv, q)
    assert lp.shape == (0, 3) and dl.shape == (0, 700)
