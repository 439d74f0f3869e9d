"""Element-by-element comparison of the HIP path's outputs with the fp64 oracle.

Bars (float32 logits / bfloat16 logits):
  log p, loss, top-K log p   |d| <= 2e-6 |ref|        / 2e-6 |ref|
  entropy                    |d| <= 1e-5 |ref|        / 1e-5 |ref|
  dlogits (each element)     |d| <= 2e-5 |ref| + 2^-126 / 4e-3 |ref| + 2^-126
  dlogits row sum            |sum| <= tol * sum|dl| + V 2^-126
  argmax, valid_rows, n_valid  bit-exact
The required bars are 2e-6 on fp32 log p and loss and 4e-3 on every output
for bf16 logits.  Only dlogits is rounded to bf16, so only dlogits needs the
4e-3 bar: log p, loss, entropy and top-K log p are fp32 outputs formed in
fp32 / fp64 from the exactly widened bf16 values, and are held to the fp32
bars whatever the input dtype (tighter than required).  The entropy and fp32
dlogits bounds follow from fp32 accumulation (about 1e-6 relative) plus one
fp32 rounding of each output, and the 2^-126 floor admits fp32 subnormal
outputs that the hardware exp flushes to zero.  A bf16 dlogit is one
round-to-nearest step (<= 2^-8 relative) from an fp32 value accurate to
~1e-6, inside 4e-3.
"""
from __future__ import annotations

import numpy as np

FLOOR = 2.0 ** -126
# Spacing of fp32 subnormals: an fp32 output below 2^-126 is exact only to
# half of this, so a per-row output that small is compared with this floor.
SUBNORMAL = 2.0 ** -149

RTOL = {
    "f32": dict(logp=2e-6, loss=2e-6, topk=2e-6, entropy=1e-5, dlogits=2e-5),
    "bf16": dict(logp=2e-6, loss=2e-6, topk=2e-6, entropy=1e-5, dlogits=4e-3),
}


def assert_close(name, got, ref, rtol, atol=0.0):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    err = np.abs(got - ref)
    bound = rtol * np.abs(ref) + atol
    bad = ~(err <= bound)
    if np.any(bad):
        i = np.unravel_index(np.argmax(np.where(bad, err - bound, -np.inf)), err.shape)
        raise AssertionError(
            f"{name}: {int(bad.sum())} of {bad.size} outside |d| <= {rtol:g}|ref| + {atol:g}; "
            f"worst at {i}: got {got[i]!r} ref {ref[i]!r}")
    # report the worst relative error where the relative bound governs (the
    # absolute floor covers the rest, e.g. flushed fp32 subnormals)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(ref != 0, err / np.abs(ref), np.where(err == 0, 0.0, np.inf))
    governed = rtol * np.abs(ref) >= atol
    rel = rel[governed] if atol > 0 else rel
    return float(np.max(rel)) if rel.size else 0.0


def assert_nonpositive(name, logp, valid=None):
    """Every log p is <= 0; on valid rows the sign bit is set (so an exact zero
    is -0.0, never +0.0)."""
    logp = np.asarray(logp)
    assert np.all(~(logp > 0)), f"{name}: positive log p {logp[logp > 0][:5]}"
    if valid is not None:
        assert np.all(np.signbit(logp[valid])), f"{name}: valid-row log p without sign bit"


def assert_row_sums(name, dl, rtol):
    dl = np.asarray(dl, dtype=np.float64)
    s = np.abs(dl.sum(axis=1))
    bound = rtol * np.abs(dl).sum(axis=1) + dl.shape[1] * FLOOR
    bad = s > bound
    assert not np.any(bad), f"{name}: row sums {s[bad][:5]} above {bound[bad][:5]}"
