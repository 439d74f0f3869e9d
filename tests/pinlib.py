"""Checks that pin the fp64 oracle to facts fixed outside of it.

Each check takes an oracle library handle (``lib=None`` means the real one) so
that tests/test_oracle_mutants.py can run the same checks against deliberately
broken copies of the oracle and show that every planted mistake is caught.

Sources of truth used here, none of them the oracle itself:
  * closed forms (uniform rows, equal-others peaked rows, V = 2 logistic, V = 1);
  * 120-digit brute force with mpmath straight from the definitions
    log p_t = x_t - log sum_j e^{x_j}, H = -sum p log p,
    dL/dz_j = (g/T)(p_j - [j = t]), and mpmath central differences of the loss;
  * invariants (shift, column permutation, temperature scaling, zero row sum);
  * library routines (numpy.argmax, numpy.flatnonzero).
"""
from __future__ import annotations

import math

import mpmath as mp
import numpy as np

import oracle
from workloads import bf16_bits, bf16_to_f32

# 120 digits: the peaked brute-force rows need log p_t ~ e^{-115} resolved
# after an O(100) cancellation, so 50 digits would not be enough.
mp.mp.dps = 120


# ----------------------------------------------------------------- references
def mp_row(z, t, T, g=1.0):
    """Brute-force log p_t, loss, entropy, dlogits, and log p at every column,
    for one row of stored values z (float array) at 50 digits, unshifted."""
    x = [mp.mpf(float(v)) / mp.mpf(T) for v in z]
    Z = mp.fsum(mp.e ** xi for xi in x)
    lse = mp.log(Z)
    logp_all = [xi - lse for xi in x]
    p = [mp.e ** lp for lp in logp_all]
    H = -mp.fsum(pj * lp for pj, lp in zip(p, logp_all))
    w = mp.mpf(g) / mp.mpf(T)
    dl = [w * (p[j] - (1 if j == t else 0)) for j in range(len(z))]
    return dict(logp=logp_all[t], loss=-logp_all[t], entropy=H, dl=dl, logp_all=logp_all)


def mp_loss_of(z, t, T):
    x = [mp.mpf(v) / mp.mpf(T) for v in z]
    return mp.log(mp.fsum(mp.e ** xi for xi in x)) - x[t]


def rel(a, b):
    a = float(a)
    b = float(b)
    if a == b:
        return 0.0
    return abs(a - b) / max(abs(b), 1e-300)


# --------------------------------------------------------------------- P1..P4
def check_uniform(lib=None):
    """All-equal row: log p = -log V, H = log V, argmax 0 (lowest index),
    dl_j = (g/T)(1/V - [j = t])."""
    for V in (3, 7, 4096, 151936):
        for T in (1.0, 0.9, 0.7):
            z = np.full((1, V), 3.25, dtype=np.float32)
            t = V // 3
            lab = np.array([t], dtype=np.int64)
            o = oracle.ce_rows(z, lab, T, lib=lib, threads=1)
            assert rel(o["logp"][0], -math.log(V)) < 1e-14, (V, T, o["logp"][0])
            # plain sequential fp64 summation of V terms: error bound ~ V * eps
            assert rel(o["entropy"][0], math.log(V)) < 1e-14 + 2.3e-16 * V, (V, T, o["entropy"][0])
            assert o["argmax"][0] == 0
            g = np.array([1.5])
            d = oracle.ce_grad_rows(z, lab, g, T, lib=lib, threads=1)[0]
            w = 1.5 / T
            expect = np.full(V, w / V)
            expect[t] = w * (1.0 / V - 1.0)
            assert np.max(np.abs(d - expect) / np.abs(expect)) < 1e-14 + 2.3e-16 * V, (V, T)


def check_peaked_closed_form(lib=None):
    """Target at margin M above V-1 equal others:
    log p_t = -softplus(log(V-1) - M/T); dl_t = -(g/T) sigmoid(log(V-1) - M/T);
    dl_j = (g/T) e^{-M/T} / (1 + (V-1) e^{-M/T}); H from p_t and the equal others."""
    for V in (2, 1003, 40001):
        for T in (1.0, 0.9):
            for M in (5.0, 17.0, 20.0, 30.0, 36.75, 40.0, 50.0, 80.0, 300.0):
                z = np.zeros((1, V), dtype=np.float32)
                t = (7 * V) // 11
                z[0, t] = M
                lab = np.array([t], dtype=np.int64)
                o = oracle.ce_rows(z, lab, T, lib=lib, threads=1)
                a = mp.log(V - 1) - mp.mpf(M) / mp.mpf(T)
                sp = mp.log1p(mp.e ** a)
                assert rel(o["logp"][0], -sp) < 1e-13, (V, T, M, o["logp"][0], sp)
                assert rel(o["loss"][0], sp) < 1e-13
                # closed form with -log p_t = log1p((V-1) e^{-M/T}) and
                # -log p_o = M/T - log p_t, so nothing rounds to 1 at 50 digits
                b = mp.mpf(M) / mp.mpf(T)
                nlpt = mp.log1p((V - 1) * mp.e ** (-b))
                pt = mp.e ** (-nlpt)
                po = pt * mp.e ** (-b)
                H = pt * nlpt + (V - 1) * po * (b + nlpt)
                assert rel(o["entropy"][0], H) < 1e-13 + 2.3e-16 * V, (V, T, M, o["entropy"][0], H)
                assert o["argmax"][0] == t
                d = oracle.ce_grad_rows(z, lab, np.array([2.0]), T, lib=lib, threads=1)[0]
                w = 2.0 / T
                q = (V - 1) * mp.e ** (-b) / (1 + (V - 1) * mp.e ** (-b))
                assert rel(d[t], -w * q) < 1e-12, (V, T, M)
                other = 0 if t != 0 else 1
                assert rel(d[other], w * po) < 1e-12, (V, T, M)


def check_two_class(lib=None):
    """V = 2: log p_t = -softplus(x_o - x_t), the logistic."""
    rng = np.random.default_rng(11)
    for _ in range(40):
        z = (rng.standard_normal((1, 2)) * 30).astype(np.float32)
        t = int(rng.integers(0, 2))
        for T in (1.0, 0.7):
            o = oracle.ce_rows(z, np.array([t]), T, lib=lib, threads=1)
            d = (mp.mpf(float(z[0, 1 - t])) - mp.mpf(float(z[0, t]))) / mp.mpf(T)
            assert rel(o["logp"][0], -mp.log1p(mp.e ** d)) < 1e-13


def check_single_class(lib=None):
    """V = 1: log p = loss = H = 0, argmax 0, dl = 0; log p is -0.0, never +."""
    z = np.array([[1.75]], dtype=np.float32)
    o = oracle.ce_rows(z, np.array([0]), 0.9, lib=lib, threads=1)
    assert o["logp"][0] == 0 and math.copysign(1, o["logp"][0]) == -1
    assert o["loss"][0] == 0 and o["entropy"][0] == 0 and o["argmax"][0] == 0
    d = oracle.ce_grad_rows(z, np.array([0]), np.array([1.0]), 0.9, lib=lib, threads=1)
    assert d[0, 0] == 0


# ------------------------------------------------------------------------ P5
def _brute_rows(seed):
    """Small rows: random (fp32 and bf16 values), and peaked rows up to margin 80."""
    rng = np.random.default_rng(seed)
    rows = []
    for V in (5, 17, 64):
        z = (rng.standard_normal(V) * 3).astype(np.float32)
        rows.append(("f32", z))
        rows.append(("bf16", bf16_bits(z)))
        for M in (17.0, 50.0, 80.0):
            zp = rng.standard_normal(V).astype(np.float32)
            t = int(rng.integers(0, V))
            zp[t] = -np.inf
            zp[t] = np.float32(zp.max() + M)
            rows.append(("f32p%d" % t, zp))
    return rows


def check_bruteforce(lib=None):
    """Oracle vs 120-digit brute force: log p, loss, H, every dl_j, top-K, argmax."""
    for kind, z in _brute_rows(5):
        V = z.shape[0]
        stored = bf16_to_f32(z) if z.dtype == np.uint16 else z
        if kind.startswith("f32p"):
            t = int(kind[4:])
        else:
            t = (3 * V) // 5
        for T in (1.0, 0.9, 0.7):
            ref = mp_row(stored, t, T, g=1.25)
            o = oracle.ce_rows(z[None, :], np.array([t]), T, lib=lib, threads=1)
            assert rel(o["logp"][0], ref["logp"]) < 1e-13, (kind, V, T)
            assert rel(o["loss"][0], ref["loss"]) < 1e-13, (kind, V, T)
            assert rel(o["entropy"][0], ref["entropy"]) < 1e-12, (kind, V, T)
            assert o["argmax"][0] == int(np.argmax(stored))
            d = oracle.ce_grad_rows(z[None, :], np.array([t]), np.array([1.25]), T, lib=lib,
                                    threads=1)[0]
            for j in range(V):
                assert rel(d[j], ref["dl"][j]) < 1e-12, (kind, V, T, j, d[j], ref["dl"][j])
            idx = np.array([[t, 0, V - 1, V // 2]], dtype=np.int64)
            lp, _ = oracle.topk_rows(z[None, :], idx, T, lib=lib, threads=1)
            for k in range(idx.shape[1]):
                assert rel(lp[0, k], ref["logp_all"][idx[0, k]]) < 1e-13, (kind, V, T, k)


def check_central_difference(lib=None):
    """dl_j against mpmath central differences of the loss (g = 1)."""
    rng = np.random.default_rng(9)
    for V in (4, 9):
        z = (rng.standard_normal(V) * 2).astype(np.float32)
        t = 1
        T = 0.9
        d = oracle.ce_grad_rows(z[None, :], np.array([t]), np.array([1.0]), T, lib=lib,
                                threads=1)[0]
        for j in range(V):
            def f(h, j=j):
                zz = [mp.mpf(float(v)) for v in z]
                zz[j] += h
                return mp_loss_of(zz, t, T)
            num = mp.diff(f, 0)
            assert rel(d[j], num) < 1e-12, (V, j, d[j], num)


# ------------------------------------------------------------------------ P6
def _grid_row(rng, V):
    # Values on a 2^-10 grid within +-64: adding 5 or doubling stays exact in fp32.
    return (np.round(rng.standard_normal(V) * 3 * 1024) / 1024).astype(np.float32)


def check_invariants(lib=None):
    rng = np.random.default_rng(21)
    V = 1000
    z = np.stack([_grid_row(rng, V) for _ in range(6)])
    lab = rng.integers(0, V, 6).astype(np.int64)
    g = rng.standard_normal(6)
    base = oracle.ce_rows(z, lab, 0.9, lib=lib, threads=1)
    # log p <= 0, loss = -log p
    assert np.all(np.signbit(base["logp"]) | (base["logp"] == 0))
    assert np.all(base["loss"] == -base["logp"])
    assert np.all(base["entropy"] >= 0) and np.all(base["entropy"] <= math.log(V) + 1e-12)
    # gradient rows sum to zero
    d = oracle.ce_grad_rows(z, lab, g, 0.9, lib=lib, threads=1)
    assert np.all(np.abs(d.sum(1)) <= 1e-14 * np.abs(d).sum(1) * V ** 0.5 + 1e-300)
    # shift invariance (exact shift)
    sh = oracle.ce_rows(z + np.float32(5.0), lab, 0.9, lib=lib, threads=1)
    for k in ("logp", "entropy"):
        assert np.max(np.abs(sh[k] - base[k]) / np.abs(base[k])) < 1e-12, k
    assert np.array_equal(sh["argmax"], base["argmax"])
    # column permutation equivariance
    perm = rng.permutation(V)
    inv = np.argsort(perm)
    zp = np.ascontiguousarray(z[:, perm])
    lp = inv[lab]
    pp = oracle.ce_rows(zp, lp, 0.9, lib=lib, threads=1)
    for k in ("logp", "entropy"):
        assert np.max(np.abs(pp[k] - base[k]) / np.abs(base[k])) < 1e-12, k
    dp = oracle.ce_grad_rows(zp, lp, g, 0.9, lib=lib, threads=1)
    assert np.max(np.abs(dp[:, inv] - d) / np.abs(d)) < 1e-12
    # temperature scaling: T = 0.5 on z equals T = 1 on 2z (both exact)
    a = oracle.ce_rows(z, lab, 0.5, lib=lib, threads=1)
    b = oracle.ce_rows(z * np.float32(2.0), lab, 1.0, lib=lib, threads=1)
    for k in ("logp", "entropy"):
        assert np.array_equal(a[k], b[k]), k
    # top-K at index = label equals the single-target log p
    idx = np.stack([lab, (lab + 1) % V], axis=1)
    tk, _ = oracle.topk_rows(z, idx, 0.9, lib=lib, threads=1)
    assert np.max(np.abs(tk[:, 0] - base["logp"]) / np.abs(base["logp"])) < 1e-14


# ------------------------------------------------------------------------ P7
def check_library_routines(lib=None):
    rng = np.random.default_rng(33)
    V = 300
    z = bf16_bits((rng.standard_normal((40, V)) * 0.5).astype(np.float32))  # many ties
    stored = bf16_to_f32(z)
    # force explicit ties of the maximum in a few rows
    for r in range(0, 40, 5):
        c = rng.choice(V, 3, replace=False)
        z[r, c] = bf16_bits(np.array([9.0], dtype=np.float32))[0]
    stored = bf16_to_f32(z)
    lab = rng.integers(0, V, 40).astype(np.int64)
    o = oracle.ce_rows(z, lab, 1.0, lib=lib, threads=1)
    assert np.array_equal(o["argmax"], np.argmax(stored, axis=1))
    lab[rng.permutation(40)[:9]] = -100
    mask = (rng.random(40) > 0.2).astype(np.uint8)
    vr, st = oracle.valid_rows(lab, mask, V, lib=lib)
    assert np.array_equal(vr, np.flatnonzero((lab != -100) & (mask != 0)))
    assert st == 0
    lab[3] = V + 4
    vr, st = oracle.valid_rows(lab, None, V, lib=lib)
    assert st == oracle.BAD_LABEL and 3 not in vr


def check_strided(lib=None):
    """A padded row stride reads the same rows as the dense copy."""
    rng = np.random.default_rng(44)
    big = (rng.standard_normal((7, 150)) * 2).astype(np.float32)
    view = big[:, :101]
    dense = np.ascontiguousarray(view)
    lab = rng.integers(0, 101, 7).astype(np.int64)
    a = oracle.ce_rows(view, lab, 0.8, lib=lib, threads=1)
    b = oracle.ce_rows(dense, lab, 0.8, lib=lib, threads=1)
    for k in ("logp", "entropy", "argmax"):
        assert np.array_equal(a[k], b[k]), k
    g = rng.standard_normal(7)
    assert np.array_equal(oracle.ce_grad_rows(view, lab, g, 0.8, lib=lib, threads=1),
                          oracle.ce_grad_rows(dense, lab, g, 0.8, lib=lib, threads=1))
    # and each row of the dense copy equals the brute force of that row
    for r in range(7):
        ref = mp_row(dense[r], int(lab[r]), 0.8)
        assert rel(a["logp"][r], ref["logp"]) < 1e-13


def mp_smoothed(z, t, T, eps, g=1.0):
    """120-digit label-smoothed loss (1-eps)(-log p_t) + (eps/V) sum_j (-log p_j)
    and its gradient (g/T)(p_j - (1-eps)[j = t] - eps/V), unshifted."""
    ref = mp_row(z, t, T, g)
    V = len(z)
    e = mp.mpf(eps)
    loss = (1 - e) * ref["loss"] + e * mp.fsum(-lp for lp in ref["logp_all"]) / V
    w = mp.mpf(g) / mp.mpf(T)
    p = [mp.e ** lp for lp in ref["logp_all"]]
    dl = [w * (p[j] - (1 - e) * (1 if j == t else 0) - e / V) for j in range(V)]
    return loss, dl


def check_label_smoothing(lib=None):
    """Smoothed loss and gradient: 120-digit brute force on random and peaked
    rows, the uniform-row closed form (loss = log V for any eps), zero row
    sums, and central differences of the smoothed loss."""
    for kind, z in _brute_rows(17):
        V = z.shape[0]
        stored = bf16_to_f32(z) if z.dtype == np.uint16 else z
        t = int(kind[4:]) if kind.startswith("f32p") else V // 3
        for T, eps in ((1.0, 0.1), (0.7, 0.3)):
            loss, dl = mp_smoothed(stored, t, T, eps, g=0.75)
            o = oracle.ce_rows(z[None, :], np.array([t]), T, lib=lib, threads=1,
                               label_smoothing=eps)
            assert rel(o["loss"][0], loss) < 1e-13, (kind, T, eps)
            ref = mp_row(stored, t, T)
            assert rel(o["logp"][0], ref["logp"]) < 1e-13   # log p is not smoothed
            d = oracle.ce_grad_rows(z[None, :], np.array([t]), np.array([0.75]), T, lib=lib,
                                    threads=1, label_smoothing=eps)[0]
            for j in range(V):
                assert abs(d[j] - float(dl[j])) <= 1e-12 * (abs(float(dl[j])) + eps / V), \
                    (kind, T, eps, j)
            assert abs(d.sum()) <= 1e-13 * np.abs(d).sum()
    for V in (5, 1000):
        z = np.full((1, V), -2.5, dtype=np.float32)
        o = oracle.ce_rows(z, np.array([1]), 0.9, lib=lib, threads=1, label_smoothing=0.2)
        assert rel(o["loss"][0], math.log(V)) < 1e-13
    rng = np.random.default_rng(3)
    z = (rng.standard_normal(7) * 2).astype(np.float32)
    d = oracle.ce_grad_rows(z[None, :], np.array([2]), np.array([1.0]), 0.8, lib=lib, threads=1,
                            label_smoothing=0.25)[0]
    for j in range(7):
        def f(h, j=j):
            zz = [mp.mpf(float(v)) for v in z]
            zz[j] += h
            x = [v / mp.mpf(0.8) for v in zz]
            lse = mp.log(mp.fsum(mp.e ** xi for xi in x))
            return mp.mpf(0.75) * (lse - x[2]) + mp.mpf(0.25) * mp.fsum(lse - xi for xi in x) / 7
        assert rel(d[j], mp.diff(f, 0)) < 1e-12, j


def mp_topk_grad(z, idx, gk, T):
    """Gradient of sum_k g_k log p_{i_k} at 120 digits: (1/T) sum_k g_k([j = i_k] - p_j)."""
    ref = mp_row(z, 0, T)
    p = [mp.e ** lp for lp in ref["logp_all"]]
    V = len(z)
    out = [mp.mpf(0)] * V
    for i, g in zip(idx, gk):
        for j in range(V):
            out[j] += mp.mpf(g) * ((1 if j == i else 0) - p[j]) / mp.mpf(T)
    return out, ref


def check_topk_grad(lib=None):
    """Top-K gradient and q = 1 - p at gathered columns: 120-digit brute force
    on random and peaked rows with duplicate and ignored entries, and central
    differences of sum_k g_k log p_{i_k}."""
    rng = np.random.default_rng(29)
    for kind, z in _brute_rows(23):
        V = z.shape[0]
        stored = bf16_to_f32(z) if z.dtype == np.uint16 else z
        top = int(np.argmax(stored))
        idx = np.array([[top, (top + 1) % V, top, -100, (top + 3) % V]], dtype=np.int64)
        gk = rng.standard_normal((1, 5))
        for T in (1.0, 0.7):
            want, ref = mp_topk_grad(stored, [i for i in idx[0] if i != -100],
                                     [g for i, g in zip(idx[0], gk[0]) if i != -100], T)
            d = oracle.topk_grad_rows(z[None, :], idx, gk, T, lib=lib, threads=1)[0]
            for j in range(V):
                assert abs(d[j] - float(want[j])) <= 1e-12 * max(abs(float(want[j])), 1e-300), \
                    (kind, T, j, d[j], want[j])
            lp, q, _ = oracle.topk_rows(z[None, :], idx, T, lib=lib, threads=1, want_q=True)
            for k in range(5):
                if idx[0, k] == -100:
                    assert q[0, k] == 0 and lp[0, k] == 0
                else:
                    pk = mp.e ** ref["logp_all"][idx[0, k]]
                    assert rel(q[0, k], 1 - pk) < 1e-13, (kind, k)
    z = (rng.standard_normal(6) * 2).astype(np.float32)
    idx = np.array([[1, 4, 1]], dtype=np.int64)
    gk = np.array([[0.5, -1.25, 2.0]])
    d = oracle.topk_grad_rows(z[None, :], idx, gk, 0.9, lib=lib, threads=1)[0]
    for j in range(6):
        def f(h, j=j):
            zz = [mp.mpf(float(v)) for v in z]
            zz[j] += h
            x = [v / mp.mpf(0.9) for v in zz]
            lse = mp.log(mp.fsum(mp.e ** xi for xi in x))
            return sum(mp.mpf(g) * (x[i] - lse) for i, g in zip(idx[0], gk[0]))
        assert rel(d[j], mp.diff(f, 0)) < 1e-12, j


ALL_CHECKS = [check_label_smoothing, check_topk_grad, check_strided, check_uniform, check_peaked_closed_form, check_two_class, check_single_class,
              check_bruteforce, check_central_difference, check_invariants,
              check_library_routines]


# ------------------------------------------------ linear head (hidden x head^T)
def _bf16_identity(n, perm=None):
    """bf16 bit patterns of a permutation matrix: row j has 1.0 at column perm[j]."""
    w = np.zeros((n, n), dtype=np.uint16)
    cols = np.arange(n) if perm is None else perm
    w[np.arange(n), cols] = 0x3F80
    return w


def check_linear_identity(lib=None, orc=None):
    """A permutation head: logits_j = h_{perm[j]}, so the linear CE equals the
    (separately pinned) CE on the permuted hidden state, and the hidden
    gradient is that CE's gradient moved back: dh[:, perm] = dlogits."""
    orc = orc or oracle
    rng = np.random.default_rng(31)
    n = 37
    h = bf16_bits((rng.standard_normal((5, n)) * 3).astype(np.float32))
    labels = np.array([3, 36, -100, 0, 17], dtype=np.int64)
    g = np.array([1.0, -0.5, 2.0, 0.25, 1.5])
    for perm in (None, rng.permutation(n)):
        w = _bf16_identity(n, perm)
        z = h if perm is None else np.ascontiguousarray(h[:, perm])
        for T, eps in ((1.0, 0.0), (0.8, 0.1)):
            got = orc.linear_ce_rows(h, w, labels, T, label_smoothing=eps, lib=lib)
            ref = orc.ce_rows(z, labels, T, label_smoothing=eps, lib=lib)
            for k in ("logp", "loss", "entropy", "argmax"):
                assert np.array_equal(got[k], ref[k]), (k, T, eps)
            d = orc.linear_ce_grads(h, w, labels, g, T, label_smoothing=eps, lib=lib)
            dl = orc.ce_grad_rows(z, labels, g, T, label_smoothing=eps, lib=lib)
            p = np.arange(n) if perm is None else perm
            assert np.array_equal(d["dhidden"][:, p], dl), (T, eps)


def check_linear_scale(lib=None, orc=None):
    """(2^3 h, 2^-3 head) gives bit-identical logits and losses; the hidden
    gradient scales by 2^-3 and the head gradient by 2^3, exactly."""
    orc = orc or oracle
    rng = np.random.default_rng(32)
    h = (rng.standard_normal((4, 6)) * 2).astype(np.float32)
    w = (rng.standard_normal((11, 6)) * 0.5).astype(np.float32)
    labels = np.array([0, 10, 5, -100], dtype=np.int64)
    g = np.array([1.0, 2.0, -1.0, 1.0])
    a = orc.linear_ce_rows(h, w, labels, 0.9, lib=lib)
    b = orc.linear_ce_rows(h * np.float32(8), w / np.float32(8), labels, 0.9, lib=lib)
    for k in ("logp", "loss", "entropy", "argmax"):
        assert np.array_equal(a[k], b[k]), k
    da = orc.linear_ce_grads(h, w, labels, g, 0.9, lib=lib)
    db = orc.linear_ce_grads(h * np.float32(8), w / np.float32(8), labels, g, 0.9, lib=lib)
    assert np.array_equal(da["dhidden"] / 8, db["dhidden"])
    assert np.array_equal(da["dweight"] * 8, db["dweight"])


def check_linear_rows_list(lib=None, orc=None):
    """A row subset gives the same per-row results as the full call."""
    orc = orc or oracle
    rng = np.random.default_rng(33)
    h = bf16_bits((rng.standard_normal((6, 8)) * 2).astype(np.float32))
    w = bf16_bits((rng.standard_normal((13, 8)) * 0.7).astype(np.float32))
    labels = np.array([1, 12, -100, 4, 0, 7], dtype=np.int64)
    mask = np.array([1, 1, 1, 0, 1, 1], dtype=np.uint8)
    g = rng.standard_normal(6)
    full = orc.linear_ce_rows(h, w, labels, 1.1, row_mask=mask, lib=lib)
    rows = np.array([5, 0, 3], dtype=np.int64)
    sub = orc.linear_ce_rows(h, w, labels, 1.1, row_mask=mask, rows_list=rows, lib=lib)
    for k in ("logp", "loss", "argmax"):
        assert np.array_equal(sub[k][rows], full[k][rows]), k
    dfull = orc.linear_ce_grads(h, w, labels, g, 1.1, row_mask=mask, lib=lib)
    dsub = orc.linear_ce_grads(h, w, labels, g, 1.1, row_mask=mask, rows_list=rows, lib=lib)
    assert np.array_equal(dsub["dhidden"], dfull["dhidden"][rows])


def _mp_linear(h, w, labels, g, T, eps=0.0):
    """Brute force at the working precision of mpmath, straight from the
    definitions: z = h w^T, per-row CE with smoothing, dz, dh = dz w, dW = dz^T h."""
    R, H = h.shape
    V = w.shape[0]
    hm = [[mp.mpf(float(h[r, k])) for k in range(H)] for r in range(R)]
    wm = [[mp.mpf(float(w[j, k])) for k in range(H)] for j in range(V)]
    loss, dz = [], []
    for r in range(R):
        z = [mp.fsum(hm[r][k] * wm[j][k] for k in range(H)) for j in range(V)]
        x = [zj / mp.mpf(T) for zj in z]
        lse = mp.log(mp.fsum(mp.e ** xi for xi in x))
        t = int(labels[r])
        nll = lse - x[t]
        smooth = mp.fsum(lse - xi for xi in x) / V
        loss.append((1 - mp.mpf(eps)) * nll + mp.mpf(eps) * smooth)
        c = mp.mpf(float(g[r])) / mp.mpf(T)
        dz.append([c * (mp.e ** (xi - lse) - (1 - mp.mpf(eps)) * (1 if j == t else 0)
                        - mp.mpf(eps) / V) for j, xi in enumerate(x)])
    dh = [[mp.fsum(dz[r][j] * wm[j][k] for j in range(V)) for k in range(H)] for r in range(R)]
    dw = [[mp.fsum(dz[r][j] * hm[r][k] for r in range(R)) for k in range(H)] for j in range(V)]
    return loss, dh, dw


def check_linear_bruteforce(lib=None, orc=None):
    """Loss, hidden and head gradients of a tiny linear CE against mpmath."""
    orc = orc or oracle
    rng = np.random.default_rng(34)
    for T, eps in ((1.0, 0.0), (0.7, 0.3)):
        h = bf16_bits((rng.standard_normal((2, 3)) * 2).astype(np.float32))
        w = bf16_bits((rng.standard_normal((5, 3)) * 2).astype(np.float32))
        labels = np.array([4, 1], dtype=np.int64)
        g = np.array([1.0, -0.75])
        loss, dh, dw = _mp_linear(bf16_to_f32(h), bf16_to_f32(w), labels, g, T, eps)
        got = orc.linear_ce_rows(h, w, labels, T, label_smoothing=eps, lib=lib)
        d = orc.linear_ce_grads(h, w, labels, g, T, label_smoothing=eps, lib=lib)
        for r in range(2):
            assert rel(got["loss"][r], loss[r]) < 1e-12, (T, eps, r)
            for k in range(3):
                assert rel(d["dhidden"][r, k], dh[r][k]) < 1e-11, (T, eps, r, k)
        for j in range(5):
            for k in range(3):
                assert rel(d["dweight"][j, k], dw[j][k]) < 1e-11, (T, eps, j, k)


def check_linear_central_difference(lib=None, orc=None):
    """dh and dW against central differences of sum_r g_r loss_r (fp64 inputs,
    a non-square head, smoothing on, one ignored and one masked row)."""
    orc = orc or oracle
    rng = np.random.default_rng(35)
    R, H, V = 4, 5, 7
    h = rng.standard_normal((R, H))
    w = rng.standard_normal((V, H)) * 0.8
    labels = np.array([2, -100, 6, 0], dtype=np.int64)
    mask = np.array([1, 1, 1, 0], dtype=np.uint8)
    g = np.array([1.0, 3.0, -0.5, 2.0])
    T, eps, step = 0.7, 0.2, 1e-5

    def objective(hh, ww):
        o = orc.linear_ce_rows(hh, ww, labels, T, row_mask=mask, label_smoothing=eps, lib=lib)
        return float(np.sum(g * o["loss"]))

    d = orc.linear_ce_grads(h, w, labels, g, T, row_mask=mask, label_smoothing=eps, lib=lib)
    for arr, grad in ((h, d["dhidden"]), (w, d["dweight"])):
        for idx in np.ndindex(arr.shape):
            up = arr.copy()
            dn = arr.copy()
            up[idx] += step
            dn[idx] -= step
            num = (objective(up, w) - objective(dn, w)) if arr is h else \
                (objective(h, up) - objective(h, dn))
            num /= 2 * step
            assert abs(grad[idx] - num) <= 1e-7 * max(1.0, abs(num)), (idx, grad[idx], num)


LINEAR_CHECKS = [check_linear_identity, check_linear_scale, check_linear_rows_list,
                 check_linear_bruteforce, check_linear_central_difference]


# ------------------------------------------------------------ generalized JSD
# The references below come from the definitions of the generalized
# Jensen-Shannon divergence between P_t = softmax(z_teacher / T) and
# P_s = softmax(z_student / T) (beta = 0: KL(P_t || P_s); beta = 1:
# KL(P_s || P_t); in between beta KL(P_t || M) + (1 - beta) KL(P_s || M),
# M = beta P_t + (1 - beta) P_s), evaluated by mpmath at 120 digits or by
# scipy's own relative-entropy and Jensen-Shannon routines.

def _jsd_orc(orc):
    if orc is None:
        import oracle.jsd as j
        return j
    return orc


def _mp_jsd(zs, zt, T, beta):
    """Loss by brute force from the definitions, unshifted, at 120 digits."""
    def lsm(z):
        x = [mp.mpf(float(v)) / mp.mpf(T) for v in z]
        lse = mp.log(mp.fsum(mp.e ** xi for xi in x))
        return [xi - lse for xi in x]
    ls, lt = lsm(zs), lsm(zt)
    ps = [mp.e ** v for v in ls]
    pt = [mp.e ** v for v in lt]
    b = mp.mpf(beta)
    if beta == 0.0:
        return mp.fsum(p * (a - c) for p, a, c in zip(pt, lt, ls))
    if beta == 1.0:
        return mp.fsum(p * (a - c) for p, a, c in zip(ps, ls, lt))
    m = [b * q + (1 - b) * p for q, p in zip(pt, ps)]
    lm = [mp.log(v) for v in m]
    return (b * mp.fsum(q * (a - c) for q, a, c in zip(pt, lt, lm)) +
            (1 - b) * mp.fsum(p * (a - c) for p, a, c in zip(ps, ls, lm)))


def _jsd_cases():
    rng = np.random.default_rng(77)
    cases = []
    for V in (2, 5, 9):
        zs = (2.0 * rng.standard_normal(V)).astype(np.float32)
        zt = (2.0 * rng.standard_normal(V)).astype(np.float32)
        cases.append((zs, zt))
    # peaked rows past the fp64 collapse point (36.7): same and different argmax
    base = rng.standard_normal(6).astype(np.float32)
    for ms, mt, at in ((50.0, 45.0, 2), (120.0, 80.0, 2), (60.0, 70.0, 4)):
        zs = base.copy()
        zs[2] = np.float32(base.max() + ms)
        zt = (base + np.float32(0.5) * rng.standard_normal(6).astype(np.float32)).astype(np.float32)
        zt[at] = np.float32(zt.max() + mt)
        cases.append((zs, zt))
    return cases


def check_jsd_identical(orc=None):
    """Identical student and teacher rows: every divergence and gradient is 0."""
    j = _jsd_orc(orc)
    z = (3.0 * np.random.default_rng(71).standard_normal((4, 50))).astype(np.float32)
    z[2, 7] += 60.0
    for beta in (0.0, 0.25, 0.5, 1.0):
        loss = j.jsd_rows(z, z, 0.8, beta)
        assert np.all(np.abs(loss) <= 1e-15), (beta, loss)
        d = j.jsd_grad_rows(z, z, np.ones(4), 0.8, beta)
        assert np.all(np.abs(d) <= 1e-15), (beta, np.abs(d).max())


def check_jsd_scipy(orc=None):
    """beta = 0 and 1 against scipy.special.rel_entr on scipy.special.softmax;
    beta = 0.5 against scipy.spatial.distance.jensenshannon (natural log)
    squared."""
    from scipy.spatial.distance import jensenshannon
    from scipy.special import rel_entr, softmax
    j = _jsd_orc(orc)
    rng = np.random.default_rng(72)
    for T in (1.0, 0.7):
        zs = (2.0 * rng.standard_normal((3, 300))).astype(np.float32)
        zt = (2.0 * rng.standard_normal((3, 300))).astype(np.float32)
        ps = softmax(zs.astype(np.float64) / T, axis=1)
        pt = softmax(zt.astype(np.float64) / T, axis=1)
        fwd = j.jsd_rows(zs, zt, T, 0.0)
        rev = j.jsd_rows(zs, zt, T, 1.0)
        mid = j.jsd_rows(zs, zt, T, 0.5)
        for r in range(3):
            assert rel(fwd[r], rel_entr(pt[r], ps[r]).sum()) < 1e-12, ("forward KL", r)
            assert rel(rev[r], rel_entr(ps[r], pt[r]).sum()) < 1e-12, ("reverse KL", r)
            assert rel(mid[r], jensenshannon(pt[r], ps[r]) ** 2) < 1e-10, ("JSD", r)


def check_jsd_disjoint_limit(orc=None):
    """Rows peaked on different columns by 300: the two distributions have
    (numerically) disjoint supports, where the generalized JSD reaches its
    maximum, the binary entropy -beta log beta - (1 - beta) log(1 - beta)."""
    j = _jsd_orc(orc)
    zs = np.zeros((1, 40), np.float32)
    zt = np.zeros((1, 40), np.float32)
    zs[0, 3] = 300.0
    zt[0, 30] = 300.0
    for beta in (0.1, 0.5, 0.8):
        h = -beta * math.log(beta) - (1 - beta) * math.log(1 - beta)
        assert rel(j.jsd_rows(zs, zt, 1.0, beta)[0], h) < 1e-12, beta


def check_jsd_bruteforce(orc=None):
    """Loss against the 120-digit definition and every gradient entry against
    mpmath central differences of that loss, on random and peaked rows
    (margins 45 to 120, same and different argmax), beta in {0, 0.3, 0.5, 1}."""
    j = _jsd_orc(orc)
    for zs, zt in _jsd_cases():
        for beta in (0.0, 0.3, 0.5, 1.0):
            for T in (1.0, 0.7):
              # a row peaked by 120 / 0.7 has entries near e^-171 and a loss
              # near e^-120: a central difference of step 1e-80 needs 250 digits
              with mp.workdps(250):
                ref = _mp_jsd(zs, zt, T, beta)
                got = j.jsd_rows(zs[None], zt[None], T, beta)[0]
                assert abs(got - float(ref)) <= 1e-12 * abs(float(ref)) + 1e-300, \
                    ("loss", beta, T, got, float(ref))
                d = j.jsd_grad_rows(zs[None], zt[None], np.array([0.75]), T, beta)[0]
                mag = _mp_grad_terms(zs, zt, T, beta)
                # the student's argmax entry is minus the sum of the others, so
                # it errs like them, not like its own near-1 terms
                a = int(np.argmax(zs))
                mag[a] = sum(m for i, m in enumerate(mag) if i != a)
                h = mp.mpf("1e-80")
                for k in range(zs.size):
                    def shifted(s):
                        z = [mp.mpf(float(v)) for v in zs]
                        z[k] += s
                        return z
                    # the definition with z_k moved by +-h (unrounded)
                    def f(z):
                        return _mp_jsd_exact(z, zt, T, beta)
                    fd = (f(shifted(h)) - f(shifted(-h))) / (2 * h) * mp.mpf("0.75")
                    # an entry that is the difference of two nearly equal terms
                    # (rows peaked at different columns) is only as accurate
                    # as fp64 makes those terms: 1e-15 of their size
                    bound = 1e-10 * abs(float(fd)) + 1e-15 * 0.75 * mag[k] + 1e-300
                    assert abs(d[k] - float(fd)) <= bound, ("grad", beta, T, k, d[k], float(fd))


def _mp_grad_terms(zs, zt, T, beta):
    """Per column, the size of the two terms whose difference the gradient
    entry is: (ps + pt) / T at beta = 0; ps (|ls - lt| + loss) / T at beta = 1;
    (1 - beta) ps (|ls - lm| + |K|) / T in between (120+ digits, as floats)."""
    def lsm(z):
        x = [mp.mpf(float(v)) / mp.mpf(T) for v in z]
        lse = mp.log(mp.fsum(mp.e ** xi for xi in x))
        return [xi - lse for xi in x]
    ls, lt = lsm(zs), lsm(zt)
    ps = [mp.e ** v for v in ls]
    pt = [mp.e ** v for v in lt]
    b = mp.mpf(beta)
    if beta == 0.0:
        return [float((p + q) / T) for p, q in zip(ps, pt)]
    if beta == 1.0:
        L = mp.fsum(p * (a - c) for p, a, c in zip(ps, ls, lt))
        return [float(p * (abs(a - c) + abs(L)) / T) for p, a, c in zip(ps, ls, lt)]
    r = [a - mp.log(b * q + (1 - b) * p) for a, p, q in zip(ls, ps, pt)]
    K = mp.fsum(p * v for p, v in zip(ps, r))
    return [float((1 - b) * p * (abs(v) + abs(K)) / T) for p, v in zip(ps, r)]


def _mp_jsd_exact(zs_mp, zt, T, beta):
    """_mp_jsd with the student row already as mpmath numbers."""
    x = [v / mp.mpf(T) for v in zs_mp]
    lse = mp.log(mp.fsum(mp.e ** xi for xi in x))
    ls = [xi - lse for xi in x]
    y = [mp.mpf(float(v)) / mp.mpf(T) for v in zt]
    lse_t = mp.log(mp.fsum(mp.e ** yi for yi in y))
    lt = [yi - lse_t for yi in y]
    ps = [mp.e ** v for v in ls]
    pt = [mp.e ** v for v in lt]
    b = mp.mpf(beta)
    if beta == 0.0:
        return mp.fsum(p * (a - c) for p, a, c in zip(pt, lt, ls))
    if beta == 1.0:
        return mp.fsum(p * (a - c) for p, a, c in zip(ps, ls, lt))
    lm = [mp.log(b * q + (1 - b) * p) for q, p in zip(pt, ps)]
    return (b * mp.fsum(q * (a - c) for q, a, c in zip(pt, lt, lm)) +
            (1 - b) * mp.fsum(p * (a - c) for p, a, c in zip(ps, ls, lm)))


def check_jsd_invariants(orc=None):
    """Adding a constant to either row changes nothing (up to rounding);
    every gradient row sums to zero; masked and ignored rows are zero."""
    j = _jsd_orc(orc)
    rng = np.random.default_rng(73)
    zs = (2.0 * rng.standard_normal((4, 200))).astype(np.float64)
    zt = (2.0 * rng.standard_normal((4, 200))).astype(np.float64)
    g = rng.standard_normal(4)
    for beta in (0.0, 0.4, 1.0):
        a = j.jsd_rows(zs, zt, 1.3, beta)
        b = j.jsd_rows(zs + 5.0, zt - 3.0, 1.3, beta)
        assert np.all(np.abs(a - b) <= 1e-12 * np.abs(a)), beta
        da = j.jsd_grad_rows(zs, zt, g, 1.3, beta)
        db = j.jsd_grad_rows(zs + 5.0, zt - 3.0, g, 1.3, beta)
        assert np.all(np.abs(da - db) <= 1e-12 * np.abs(da).max()), beta
        assert np.all(np.abs(da.sum(1)) <= 1e-15 * np.abs(da).sum(1)), beta
        labels = np.array([1, -100, 3, 4])
        mask = np.array([1, 1, 0, 1], np.uint8)
        lm = j.jsd_rows(zs, zt, 1.3, beta, labels=labels, row_mask=mask)
        dm = j.jsd_grad_rows(zs, zt, g, 1.3, beta, labels=labels, row_mask=mask)
        assert lm[1] == 0 and lm[2] == 0 and lm[0] == a[0] and lm[3] == a[3]
        assert np.all(dm[[1, 2]] == 0) and np.array_equal(dm[[0, 3]], da[[0, 3]])


JSD_CHECKS = [check_jsd_identical, check_jsd_scipy, check_jsd_disjoint_limit,
              check_jsd_bruteforce, check_jsd_invariants]
