"""fp64 oracle for the collapse-safe generalized Jensen-Shannon divergence
between a student and a teacher logit row (KL at the two ends).

TEST INFRASTRUCTURE ONLY (see the package docstring): the tests, smoke() and
bench.py's cpu_baseline are the only callers; the product path never
imports it.

Definitions (unsloth-zoo #2079 Summary, quoted on the Liger-Kernel PR #1555
page: logits divided by T, log-softmax of both rows, beta = 0 the forward KL,
beta = 1 the reverse KL, the log-sum-exp mixture in between; rows whose label
is the ignore index are masked), per valid row with x = z_student / T and
y = z_teacher / T:

  ls = log_softmax(x),  lt = log_softmax(y),  ps = e^ls,  pt = e^lt
  beta = 0:     loss = sum_j pt_j (lt_j - ls_j)                 KL(P_t || P_s)
  beta = 1:     loss = sum_j ps_j (ls_j - lt_j)                 KL(P_s || P_t)
  0 < beta < 1: lm = log(beta pt + (1 - beta) ps)
                loss = beta sum pt (lt - lm) + (1 - beta) sum ps (ls - lm)

and the gradient of g * loss with respect to the student logits z (the
teacher is never differentiated):

  beta = 0:     d_j = g (ps_j - pt_j) / T
  beta = 1:     d_j = g ps_j (ls_j - lt_j - loss) / T
  0 < beta < 1: d_j = g (1 - beta) ps_j (ls_j - lm_j - K) / T,
                K = sum_j ps_j (ls_j - lm_j)

(the chain rule through log_softmax; each sums to zero over j).  Every
quantity is evaluated so that it keeps its relative accuracy on rows peaked by
far more than the 16.6 (fp32) and 36.7 (fp64) at which a plain log-softmax
collapses (Liger-Kernel PR #1555, Summary and Details):

* log_softmax is based at the row's first argmax a:
  ls_j = (x_j - x_a) - log1p(S), S = sum_{j != a} e^(x_j - x_a), so ls_a is
  -log1p(S), never x_a - lse rounded to 0.
* The mixture enters only through ls - lm and lt - lm, written as
  functions of delta = lt - ls alone:
    ls - lm = -log1p(beta expm1(delta))                       (delta <= 0)
            = -delta - log1p((1 - beta) expm1(-delta))         (delta > 0)
    lt - lm = delta + (ls - lm), evaluated the mirrored way
  (the exponent is never positive), so they keep their relative accuracy
  where ls and lm are both large and nearly equal; the gradient factor
  (ls_j - lm_j) - K then only loses what its own cancellation costs.
* The gradient at the student's argmax is minus the sum of the other
  entries of the row (the argmax rule of the Liger-Kernel PR #1555 Summary,
  "fused KL / JSD" bullet), which is the same value up to rounding and keeps
  the row summing to zero.

Parity status: pinned (tests/pinlib.py JSD_CHECKS): identical rows give
0; beta = 0 and 1 against scipy's relative entropy on the softmax; beta = 0.5
against scipy's Jensen-Shannon distance squared; 120-digit mpmath brute
force of the loss and every gradient entry, peaked rows included; mpmath
central differences of the loss; invariance to shifting either row.
"""
from __future__ import annotations

import numpy as np


def _widen(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def log_softmax_safe(x):
    """ls_j = x_j - log sum_k e^(x_k), based at the first argmax a; returns
    (ls, a, S) with S the sum over the other columns of e^(x_j - x_a)."""
    x = np.asarray(x, dtype=np.float64)
    a = int(np.argmax(x))
    d = x - x[a]
    e = np.exp(d)
    e[a] = 0.0
    S = float(np.sum(e))
    ls = d - np.log1p(S)
    ls[a] = -np.log1p(S)
    return ls, a, S


def _mixture_gaps(ls, lt, beta):
    """(ls - lm, lt - lm) with lm = log(beta e^lt + (1 - beta) e^ls), from
    delta = lt - ls: beta e^lt + (1 - beta) e^ls = e^ls (1 + beta expm1(delta))
    = e^lt (1 + (1 - beta) expm1(-delta))."""
    delta = lt - ls
    neg = delta <= 0
    dn = np.where(neg, delta, 0.0)
    dp = np.where(neg, 0.0, delta)
    a = -np.log1p(beta * np.expm1(dn))            # ls - lm where delta <= 0
    b = -np.log1p((1.0 - beta) * np.expm1(-dp))   # lt - lm where delta > 0
    r = np.where(neg, a, b - dp)                  # ls - lm
    q = np.where(neg, a + dn, b)                  # lt - lm
    return r, q


def _row_valid(labels, row_mask, r, ignore_index):
    if row_mask is not None and row_mask[r] == 0:
        return False
    if labels is not None and labels[r] == ignore_index:
        return False
    return True


def jsd_row(zs, zt, temperature, beta):
    """(loss, K, ls, lt, r) for one valid row; K is the beta-specific
    constant of the gradient (the loss at beta = 1, sum ps (ls - lm) in
    between, 0 at beta = 0) and r = ls - lm in between (None otherwise)."""
    T = float(temperature)
    ls, a_s, _ = log_softmax_safe(_widen(zs) / T)
    lt, a_t, _ = log_softmax_safe(_widen(zt) / T)
    if beta == 0.0:
        pt = np.exp(lt)
        return float(np.sum(pt * (lt - ls))), 0.0, ls, lt, None
    if beta == 1.0:
        ps = np.exp(ls)
        loss = float(np.sum(ps * (ls - lt)))
        return loss, loss, ls, lt, None
    r, q = _mixture_gaps(ls, lt, beta)
    ps, pt = np.exp(ls), np.exp(lt)
    K = float(np.sum(ps * r))
    loss = beta * float(np.sum(pt * q)) + (1.0 - beta) * K
    return loss, K, ls, lt, r


def jsd_rows(student, teacher, temperature=1.0, beta=0.5, labels=None, row_mask=None,
             ignore_index=-100, rows_list=None):
    """Per-row loss (float64 [rows]); 0 for masked rows.  Rows outside
    rows_list (if given) are NaN."""
    R = student.shape[0]
    out = np.full(R, np.nan) if rows_list is not None else np.zeros(R)
    rows = range(R) if rows_list is None else rows_list
    for r in rows:
        r = int(r)
        if not _row_valid(labels, row_mask, r, ignore_index):
            out[r] = 0.0
            continue
        out[r] = jsd_row(student[r], teacher[r], temperature, beta)[0]
    return out


def jsd_grad_row(zs, zt, g, temperature, beta):
    """float64 gradient of g * loss with respect to one valid student row."""
    T = float(temperature)
    loss, K, ls, lt, r = jsd_row(zs, zt, temperature, beta)
    ps = np.exp(ls)
    if beta == 0.0:
        d = (ps - np.exp(lt)) / T
    elif beta == 1.0:
        d = ps * ((ls - lt) - loss) / T
    else:
        d = (1.0 - beta) * ps * (r - K) / T
    a = int(np.argmax(_widen(zs)))
    d[a] = 0.0
    d[a] = -np.sum(d)
    return g * d


def jsd_grad_rows(student, teacher, g, temperature=1.0, beta=0.5, labels=None, row_mask=None,
                  ignore_index=-100, rows_list=None):
    """float64 gradients [len(rows), vocab] for rows_list (all rows if None);
    masked rows are zero."""
    R, V = student.shape
    rows = list(range(R)) if rows_list is None else [int(r) for r in rows_list]
    out = np.zeros((len(rows), V))
    for i, r in enumerate(rows):
        if _row_valid(labels, row_mask, r, ignore_index):
            out[i] = jsd_grad_row(student[r], teacher[r], float(g[r]), temperature, beta)
    return out
