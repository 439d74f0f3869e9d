"""The full-size workloads in the launch configuration the benchmark times,
against the oracle on every row: log p, loss, entropy and argmax of all rows
in one (threaded) oracle call, and every dlogits element with the oracle's
gradient rows streamed in chunks of 256 rows, so that no full fp64 gradient
matrix is ever held.  Plus properties that hold at any size (bit-exact
compaction, log p <= 0 with the sign bit set, strictly positive loss on
peaked rows, zero dlogits row sums).  The worst relative errors are printed."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tolerance import FLOOR, RTOL, SUBNORMAL, assert_close, assert_nonpositive

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

CHUNK = 256


def _sample_rows(rng, valid, n_valid_rows, n_invalid_rows):
    v = np.flatnonzero(valid)
    iv = np.flatnonzero(~valid)
    pick = list(rng.choice(v, min(n_valid_rows, v.size), replace=False))
    pick += [v[0], v[-1]]
    if iv.size:
        pick += list(rng.choice(iv, min(n_invalid_rows, iv.size), replace=False))
    return np.unique(np.asarray(pick, dtype=np.int64))


def _row_sums_ok(dl: torch.Tensor, tol, chunk=256):
    """|sum_j dl_j| <= tol * sum_j |dl_j| + V 2^-126 on every row (fp64 on the GPU)."""
    R, V = dl.shape
    for a in range(0, R, chunk):
        d = dl[a:a + chunk].double()
        s = d.sum(1).abs()
        bound = tol * d.abs().sum(1) + V * FLOOR
        bad = s > bound
        assert not bool(bad.any()), f"rows {[a + i for i in torch.nonzero(bad).flatten()[:5].tolist()]}"


def _forward_all_rows(name, w, out, tol, entropy, argmax=True):
    """Every row's forward outputs against one oracle call over all rows;
    returns the oracle's results and the worst relative errors."""
    from gpu_helpers import to_host
    T = w["temperature"]
    ref = oracle.ce_rows(w["logits"], w["labels"], T, row_mask=w.get("row_mask"),
                         want_entropy=entropy, want_argmax=argmax)
    errs = {"logp": assert_close(f"{name} logp", to_host(out["logp"]), ref["logp"], tol["logp"])}
    if out.get("loss") is not None:
        errs["loss"] = assert_close(f"{name} loss", to_host(out["loss"]), ref["loss"], tol["loss"])
    if entropy:
        # an entropy below the fp32 normal range is exact only to the
        # subnormal spacing
        errs["entropy"] = assert_close(f"{name} entropy", to_host(out["entropy"]), ref["entropy"],
                                       tol["entropy"], SUBNORMAL)
    if argmax:
        assert np.array_equal(to_host(out["argmax"]), ref["argmax"]), f"{name} argmax"
    return ref, errs


def _dlogits_all_rows(name, w, dl, tol, g=None):
    """Every dlogits element against the oracle's gradient rows, CHUNK rows at
    a time; returns the worst relative error."""
    from gpu_helpers import to_host
    R = dl.shape[0]
    g64 = np.asarray(w["g"] if g is None else g, np.float64)
    worst = 0.0
    for r0 in range(0, R, CHUNK):
        r1 = min(R, r0 + CHUNK)
        dref = oracle.ce_grad_rows(w["logits"], w["labels"], g64, w["temperature"],
                                   row_mask=w.get("row_mask"), r0=r0, r1=r1)
        got = to_host(dl[r0:r1])
        worst = max(worst, assert_close(f"{name} dlogits rows {r0}:{r1}", got, dref, tol, FLOOR))
        del dref, got
    return worst


def _ce_full(name, w, entropy, tol):
    from gpu_helpers import say, to_dev, to_host
    import cross_entropy_vocab_amd as cev
    R, V = w["logits"].shape
    logits = to_dev(w["logits"])
    labels = to_dev(w["labels"])
    mask = None if w.get("row_mask") is None else to_dev(w["row_mask"])
    g = to_dev(np.asarray(w["g"], np.float32))
    T = w["temperature"]
    out = cev.ce_forward(logits, labels, T, row_mask=mask, entropy=entropy, argmax=True)
    dl = cev.ce_backward(logits, labels, g, out["saved"], T, row_mask=mask)
    torch.cuda.synchronize()
    vr, _ = oracle.valid_rows(w["labels"], w.get("row_mask"), V)
    n = int(out["n_valid"].item())
    assert n == vr.size and np.array_equal(out["valid_rows"][:n].cpu().numpy(), vr)
    valid = np.zeros(R, dtype=bool)
    valid[vr] = True
    logp = to_host(out["logp"])
    loss = to_host(out["loss"])
    assert_nonpositive("logp", logp, valid)
    assert np.all(loss[valid] >= 0) and np.all(loss[~valid] == 0)
    _row_sums_ok(dl, tol["dlogits"])
    _, errs = _forward_all_rows(name, w, out, tol, entropy)
    errs["dlogits"] = _dlogits_all_rows(name, w, dl, tol["dlogits"])
    say(f"  {name}: {n} of {R} rows valid, all rows vs oracle, worst relative error " +
        ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    return out, logp, loss, valid


def test_grpo_full_8192x152064_bf16():
    from gpu_helpers import say
    say("[full] grpo 8192x152064 bf16, 819 rows masked")
    w = workloads.grpo()
    _ce_full("grpo", w, entropy=False, tol=RTOL["bf16"])


@pytest.fixture(scope="module", params=["f32", "bf16"])
def peaked_full(request):
    return workloads.peaked(request.param, 1.0)


@pytest.mark.parametrize("T", [1.0, 0.9])
def test_peaked_full_2048x151936(peaked_full, T):
    """Every margin in {5,17,20,30,50,80}: loss stays strictly positive (no
    collapse) and every row matches the oracle."""
    from gpu_helpers import say
    w = dict(peaked_full, temperature=T)
    kind = "bf16" if w["logits"].dtype == np.uint16 else "f32"
    say(f"[full] peaked 2048x151936 {kind} T={T}")
    out, logp, loss, valid = _ce_full(f"peaked {kind} T={T}", w, entropy=True, tol=RTOL[kind])
    assert np.all(loss > 0) and np.all(logp < 0), "a peaked row collapsed to 0"


def test_chunk_full_4096x32768_bf16_sls_and_topk():
    from gpu_helpers import DEV, say, to_dev, to_host
    import cross_entropy_vocab_amd as cev
    say("[full] chunk 4096x32768 bf16 T=0.7, sls + top-8")
    w = workloads.chunk()
    logits = to_dev(w["logits"])
    labels = to_dev(w["labels"])
    idx = to_dev(w["indices"])
    s = cev.sls_forward(logits, labels, 0.7, argmax=True)
    lp = cev.sls_topk_forward(logits, idx, 0.7)
    torch.cuda.synchronize()
    logp = to_host(s["logp"])
    tk = to_host(lp)
    assert_nonpositive("sls", logp, np.ones(4096, dtype=bool))
    assert_nonpositive("topk", tk)
    ref = oracle.ce_rows(w["logits"], w["labels"], 0.7, want_entropy=False)
    e1 = assert_close("sls logp", logp, ref["logp"], RTOL["bf16"]["logp"])
    assert np.array_equal(to_host(s["argmax"]), ref["argmax"])
    tref, _ = oracle.topk_rows(w["logits"], w["indices"], 0.7)
    e2 = assert_close("topk", tk, tref, RTOL["bf16"]["topk"])
    say(f"  all 4096 rows vs oracle, worst relative error sls logp {e1:.2e}, top-8 logp {e2:.2e}")


def test_compaction_many_rows():
    """Compaction across many tiles (300000 rows, so each workgroup owns
    several 1024-row sub-tiles): bit-exact against numpy.flatnonzero."""
    from gpu_helpers import DEV, to_dev
    import cross_entropy_vocab_amd as cev
    rng = np.random.default_rng(21)
    R, V = 300000, 6
    z = rng.standard_normal((R, V)).astype(np.float32)
    labels = rng.integers(0, V, R).astype(np.int64)
    labels[rng.random(R) < 0.3] = -100
    mask = (rng.random(R) > 0.2).astype(np.uint8)
    out = cev.ce_forward(to_dev(z), to_dev(labels), 1.0, row_mask=to_dev(mask))
    torch.cuda.synchronize()
    want = np.flatnonzero((labels != -100) & (mask != 0))
    n = int(out["n_valid"].item())
    assert n == want.size
    assert np.array_equal(out["valid_rows"][:n].cpu().numpy(), want)


def test_chunk_full_topk_backward():
    """Top-8 backward over the full chunk workload: every row's gradient sums
    to zero; sampled rows match the oracle (gathered columns with the
    difference-of-terms bound)."""
    from gpu_helpers import DEV, say, to_dev, to_host
    from test_gpu_smoothing_topk import TERM_RTOL, _assert_within, _topk_bound
    import cross_entropy_vocab_amd as cev
    say("[full] chunk 4096x32768 bf16 T=0.7, top-8 forward + backward")
    w = workloads.chunk()
    g = np.random.default_rng([6, 4096]).standard_normal((4096, 8)).astype(np.float32)
    logits = to_dev(w["logits"])
    idx = to_dev(w["indices"])
    lp, q, sv = cev.sls_topk_forward(logits, idx, 0.7, saved=True)
    dl = cev.sls_topk_backward(logits, idx, to_dev(g), sv, q, 0.7)
    torch.cuda.synchronize()
    _row_sums_ok(dl, RTOL["bf16"]["dlogits"])
    rows = _sample_rows(np.random.default_rng(5), np.ones(4096, bool), 24, 0)
    dsel = to_host(dl[torch.from_numpy(rows).to(DEV)])
    sub = dict(w, logits=w["logits"][rows], indices=w["indices"][rows])
    dref = oracle.topk_grad_rows(sub["logits"], sub["indices"], g[rows].astype(np.float64), 0.7)
    extra = _topk_bound(sub, sub["indices"], g[rows])
    tol = RTOL["bf16"]["dlogits"]
    _assert_within("topk dlogits", dsel, dref, tol * np.abs(dref) + TERM_RTOL * extra + FLOOR)
    qref = oracle.topk_rows(sub["logits"], sub["indices"], 0.7, want_q=True)[1]
    assert_close("topk q", to_host(q)[rows], qref, RTOL["bf16"]["topk"])


def test_grpo_full_vocab_parallel_p8():
    """The grpo workload as 8 vocab shards of 19008 columns (one rank's shard
    shape): the merged outputs agree with the unsharded call and with the
    oracle on every row, and so does every gradient element."""
    from gpu_helpers import DEV, say, to_dev, to_host
    import cross_entropy_vocab_amd as cev
    say("[full] grpo 8192x152064 bf16 as 8 vocab shards")
    w = workloads.grpo()
    R, V = w["logits"].shape
    P, Vs = 8, V // 8
    logits = to_dev(w["logits"])
    labels = to_dev(w["labels"])
    mask = to_dev(w["row_mask"])
    g = to_dev(w["g"])
    parts = torch.empty((P, R, cev.PARTIAL_BYTES), dtype=torch.uint8, device=DEV)
    for p in range(P):
        cev.ce_vocab_shard_forward(logits[:, p * Vs:(p + 1) * Vs], labels, p * Vs, V, 1.0,
                                   row_mask=mask, partials=parts[p])
    out = cev.ce_vocab_merge(parts, labels, V, 1.0, row_mask=mask, argmax=True)
    dl = torch.empty_like(logits)
    for p in range(P):
        cev.ce_vocab_shard_backward(logits[:, p * Vs:(p + 1) * Vs], labels, g, out["saved"],
                                    p * Vs, V, 1.0, row_mask=mask, dlogits=dl[:, p * Vs:(p + 1) * Vs])
    ce = cev.ce_forward(logits, labels, 1.0, row_mask=mask, argmax=True)
    torch.cuda.synchronize()
    logp, cel = to_host(out["logp"]), to_host(ce["logp"])
    assert_close("sharded vs whole logp", logp, cel.astype(np.float64), 1e-6)
    assert np.array_equal(to_host(out["argmax"]), to_host(ce["argmax"]))
    _row_sums_ok(dl, RTOL["bf16"]["dlogits"])
    _, errs = _forward_all_rows("sharded", w, out, RTOL["bf16"], entropy=False)
    errs["dlogits"] = _dlogits_all_rows("sharded", w, dl, RTOL["bf16"]["dlogits"])
    say("  all rows vs oracle, worst relative error " +
        ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))


def test_linear_full_8192x2560x151936():
    """lce_forward + lce_backward (frozen head) at the benchmarked shape, 2% of
    the rows peaked at the accuracy margins.  Every row: log p <= 0, loss >= 0,
    ignored rows 0 / -1 / zero dhidden, bf16 dlogits rows summing to zero.
    Sampled rows against the fp64 oracle under the random-bf16 product bound:
    each logit may err by dz = (H / 16 + 2) 2^-24 max_j sum_k |h_k w_jk| (one
    fp32 rounding per 16-deep MFMA step), which moves log p, the loss and every
    probability by at most 2 dz / T relative."""
    from gpu_helpers import DEV, say, to_dev, to_host
    import cross_entropy_vocab_amd as cev
    say("[full] linear 8192x2560x151936 bf16, frozen head")
    w = workloads.linear(peaked_frac=0.02)
    R, H = w["hidden"].shape
    V = w["weight"].shape[0]
    T = w["temperature"]
    hid, head = to_dev(w["hidden"]), to_dev(w["weight"])
    labels, mask = to_dev(w["labels"]), to_dev(w["row_mask"])
    g = to_dev(w["g"])
    out = cev.lce_forward(hid, head, labels, T, row_mask=mask, argmax=True)
    dh, dw = cev.lce_backward(hid, head, labels, g, out["saved"], T, row_mask=mask,
                              workspace=out["workspace"])
    torch.cuda.synchronize()
    assert dw is None
    ldd = (V + 63) // 64 * 64
    dl = out["workspace"][:R * ldd * 2].view(torch.bfloat16).view(R, ldd)
    vr, _ = oracle.valid_rows(w["labels"], w["row_mask"], V)
    valid = np.zeros(R, bool)
    valid[vr] = True
    logp, loss = to_host(out["logp"]), to_host(out["loss"])
    arg = to_host(out["argmax"])
    dhn = dh.cpu().numpy()
    assert_nonpositive("logp", logp, valid)
    assert np.all(loss[valid] >= 0) and np.all(loss[~valid] == 0)
    assert np.all(arg[~valid] == -1) and np.all(dhn[~valid] == 0)
    _row_sums_ok(dl[:, :V], RTOL["bf16"]["dlogits"])
    assert bool((dl[:, V:] == 0).all())

    rng = np.random.default_rng(11)
    rows = _sample_rows(rng, valid, 16, 3)
    rows = np.unique(np.concatenate([rows, w["peak_rows"][:6]]))
    ref = oracle.linear_ce_rows(w["hidden"], w["weight"], w["labels"], T,
                                row_mask=w["row_mask"], rows_list=rows, want_entropy=False)
    z = oracle.linear_logits(w["hidden"], w["weight"], rows)
    h64, w64 = oracle._widen(w["hidden"][rows]), oracle._widen(w["weight"])
    dz = (H / 16 + 2) * 2.0 ** -24 * (np.abs(h64) @ np.abs(w64).T).max(axis=1)
    rel = 2 * dz / T
    vs = valid[rows]
    err = np.abs(loss[rows] - ref["loss"][rows])
    bound = 2e-6 * np.abs(ref["loss"][rows]) + rel * np.abs(ref["loss"][rows]) + 2 * dz / T
    assert np.all(err[vs] <= bound[vs]), float(np.max(err[vs] / bound[vs]))
    err = np.abs(logp[rows] - ref["logp"][rows])
    assert np.all(err[vs] <= bound[vs]), float(np.max(err[vs] / bound[vs]))
    for i, r in enumerate(rows):
        if vs[i]:
            assert z[i, arg[r]] >= z[i].max() - 2 * dz[i], r
    grads = oracle.linear_ce_grads(w["hidden"], w["weight"], w["labels"], w["g"], T,
                                   row_mask=w["row_mask"], rows_list=rows)
    dref = oracle.ce_grad_rows(z, np.ascontiguousarray(w["labels"][rows]),
                               np.asarray(w["g"], np.float64)[rows], T,
                               row_mask=np.ascontiguousarray(w["row_mask"][rows]))
    dsel = to_host(dl[torch.from_numpy(rows).to(DEV), :V])
    # bf16 bar plus the probabilities' 2 dz / T from the product
    bdl = (RTOL["bf16"]["dlogits"] + 1.01 * rel[:, None]) * np.abs(dref) + FLOOR
    assert np.all(np.abs(dsel - dref) <= bdl), float(np.max(np.abs(dsel - dref) / bdl))
    # dhidden: the same per-entry bar carried through the product, fp32
    # accumulation over V / 16 MFMA steps (below 6e-4 relative), and the
    # floor of every flushed entry
    bh = (4.5e-3 + 1.01 * rel[:, None]) * (np.abs(dref) @ np.abs(w64)) \
        + FLOOR * vs[:, None] * np.abs(w64).sum(0) + FLOOR
    err = np.abs(dhn[rows] - grads["dhidden"])
    assert np.all(err <= bh), float(np.max(err / bh))
    say(f"  sampled {rows.size} rows; max logit error bound dz {dz.max():.2e}; "
        f"worst dhidden error / bound {float(np.max(err / bh)):.3f}")

    # The same call pair with the fp32 logits stored by the forward and read
    # back by the backward: every output bit for bit as recomputed, and the
    # stored logits of the sampled rows within the product bound of the exact
    # ones.
    say("[full] linear 8192x2560x151936 bf16, logits stored")
    zs = torch.empty((R, V), dtype=torch.float32, device=DEV)
    o2 = cev.lce_forward(hid, head, labels, T, row_mask=mask, argmax=True, logits=zs)
    dh2, _ = cev.lce_backward(hid, head, labels, g, o2["saved"], T, row_mask=mask,
                              workspace=o2["workspace"], logits=zs)
    torch.cuda.synchronize()
    for k in ("loss", "logp", "argmax", "saved"):
        assert torch.equal(o2[k], out[k]), k
    dl2 = o2["workspace"][:R * ldd * 2].view(torch.int16).view(R, ldd)
    assert torch.equal(dl2, out["workspace"][:R * ldd * 2].view(torch.int16).view(R, ldd))
    assert torch.equal(dh2, dh)
    zsel = zs[torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(zsel - z) <= dz[:, None]), float(np.max(np.abs(zsel - z) - dz[:, None]))
    del zs, o2, dh2


@pytest.fixture(scope="module")
def distill_full():
    return workloads.distill(peaked_frac=0.02)


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0])
def test_jsd_full_2048x151936_bf16(distill_full, beta):
    """jsd_forward + jsd_backward at the 2048 x 151936 bf16 shape of the
    unsloth-zoo #2079 Numbers, 2% of the rows peaked by 20-80: every row has a
    finite loss >= -bound, masked rows are zero, gradient rows sum to zero up
    to bf16 rounding; sampled rows (random, peaked, masked) against the fp64
    oracle under the error model of tests/test_gpu_jsd.py."""
    from gpu_helpers import DEV, say, to_dev, to_host
    import cross_entropy_vocab_amd as cev
    from test_gpu_jsd import _valid, check
    w = distill_full
    R, V = w["student"].shape
    say(f"[full] jsd 2048x151936 bf16 beta={beta}")
    st, te = to_dev(w["student"]), to_dev(w["teacher"])
    labels, mask, g = to_dev(w["labels"]), to_dev(w["row_mask"]), to_dev(w["g"])
    out = cev.jsd_forward(st, te, 1.0, beta, labels=labels, row_mask=mask)
    d = cev.jsd_backward(st, te, g, out["saved"], 1.0, beta, labels=labels, row_mask=mask)
    torch.cuda.synchronize()
    loss = to_host(out["loss"])
    valid = _valid(w)
    assert np.all(np.isfinite(loss)) and np.all(loss[~valid] == 0)
    assert np.all(loss[valid] > -1e-5)
    _row_sums_ok(d, 2.0 ** -8)
    rng = np.random.default_rng(12)
    rows = _sample_rows(rng, valid, 12, 3)
    rows = np.unique(np.concatenate([rows, w["peak_rows"][:6]]))
    dsel = to_host(d[torch.from_numpy(rows).to(DEV)])
    sub = dict(student=w["student"][rows], teacher=w["teacher"][rows], labels=w["labels"][rows],
               row_mask=w["row_mask"][rows], g=w["g"][rows], temperature=1.0)
    wl, wd = check(sub, dict(loss=loss[rows], dstudent=dsel), beta, "full jsd")
    say(f"  sampled {rows.size} rows; worst loss error / bound {wl:.3f}, dstudent {wd:.3f}")


def test_grpo_full_fused():
    """ce_fused (g known up front) on the full grpo workload, in the launch
    configuration bench.py times: every row agrees with ce_forward +
    ce_backward (log p to 1e-6 relative, argmax exactly) and with the oracle
    (every output and gradient element); masked rows are zero."""
    from gpu_helpers import DEV, say, to_dev, to_host
    import cross_entropy_vocab_amd as cev
    say("[full] ce_fused grpo 8192x152064 bf16")
    w = workloads.grpo()
    R, V = w["logits"].shape
    logits, labels = to_dev(w["logits"]), to_dev(w["labels"])
    mask, g = to_dev(w["row_mask"]), to_dev(w["g"])
    out = cev.ce_fused(logits, labels, g, 1.0, row_mask=mask, argmax=True)
    torch.cuda.synchronize()
    dl = out["dlogits"]
    two = cev.ce_forward(logits, labels, 1.0, row_mask=mask, argmax=True)
    torch.cuda.synchronize()
    logp, logp2 = to_host(out["logp"]), to_host(two["logp"])
    assert_close("fused vs two calls logp", logp, logp2.astype(np.float64), 1e-6)
    assert np.array_equal(to_host(out["argmax"]), to_host(two["argmax"]))
    vr, _ = oracle.valid_rows(w["labels"], w["row_mask"], V)
    n = vr.size
    valid = np.zeros(R, bool)
    valid[vr] = True
    _row_sums_ok(dl, RTOL["bf16"]["dlogits"])
    assert bool((dl[torch.from_numpy(np.flatnonzero(~valid)).to(DEV)] == 0).all())
    _, errs = _forward_all_rows("fused", w, out, RTOL["bf16"], entropy=False)
    errs["dlogits"] = _dlogits_all_rows("fused", w, dl, RTOL["bf16"]["dlogits"])
    say(f"  {n} valid rows, all rows vs oracle, worst relative error " +
        ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))


def test_longest_rows_2p27_bf16():
    """Rows of V = 2^27 + 5 bf16 columns (index arithmetic far past 2^26, a
    ragged tail, ce_forward's split-row path with few rows): 3 rows, one
    ignored, one peaked by 30 with its target in the last (tail) column, one
    with its target past 2^26.  Forward outputs against the oracle on every
    row; dlogits against the oracle's full gradient rows at 2^20 random
    columns plus the target and the tail, and zero row sums."""
    from gpu_helpers import DEV, say, to_dev, to_host
    import cross_entropy_vocab_amd as cev
    V = (1 << 27) + 5
    say(f"[full] 3 rows x {V} bf16")
    rng = np.random.default_rng(27)
    z = np.empty((3, V), np.float32)
    for r in range(3):
        z[r] = 3.0 * rng.standard_normal(V, dtype=np.float32)
    labels = np.array([V - 1, -100, (1 << 26) + 12345], np.int64)
    z[0, V - 1] = z[0].max() + 30.0
    w = dict(logits=workloads.bf16_bits(z), labels=labels, row_mask=None, temperature=1.0,
             g=np.array([0.8, 1.0, -1.3], np.float32))
    del z
    logits, lab = to_dev(w["logits"]), to_dev(labels)
    g = to_dev(w["g"])
    out = cev.ce_forward(logits, lab, 1.0, entropy=True, argmax=True)
    dl = cev.ce_backward(logits, lab, g, out["saved"], 1.0)
    torch.cuda.synchronize()
    ref = oracle.ce_rows(w["logits"], labels, 1.0)
    tol = RTOL["bf16"]
    assert_close("logp", to_host(out["logp"]), ref["logp"], tol["logp"])
    assert_close("loss", to_host(out["loss"]), ref["loss"], tol["loss"])
    assert_close("entropy", to_host(out["entropy"]), ref["entropy"], tol["entropy"], 1e-30)
    assert np.array_equal(to_host(out["argmax"]), ref["argmax"])
    assert to_host(out["loss"])[0] > 0
    _row_sums_ok(dl, tol["dlogits"])
    assert bool((dl[1] == 0).all())
    cols = np.unique(np.concatenate([rng.integers(0, V, 1 << 20), [0, V - 5, V - 1, labels[2]]]))
    cidx = torch.from_numpy(cols).to(DEV)
    g64 = np.asarray(w["g"], np.float64)
    for r in (0, 2):
        dref = oracle.ce_grad_rows(w["logits"], labels, g64, 1.0, r0=r, r1=r + 1)[0]
        got = to_host(dl[r][cidx])
        assert_close(f"dlogits row {r}", got, dref[cols], tol["dlogits"], FLOOR)
        del dref
