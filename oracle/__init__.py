"""fp64 CPU oracle for collapse-safe selective log-softmax / cross-entropy.

TEST INFRASTRUCTURE ONLY.  The test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The product path
(``cross_entropy_vocab_amd`` and its HIP library) never imports this package,
and this package imports nothing from it: the two share no code.

The arithmetic lives in ``oracle_cev.c`` (plain C, double precision, one row
and one column at a time).  This module only builds that file with gcc, loads
it with ctypes and spreads row ranges over host threads (ctypes releases the
GIL for the duration of each foreign call, so the threads run in parallel).

Every function here returns float64 results computed from the *stored* input
values: fp32 logits are passed as float32 arrays, bf16 logits as their uint16
bit patterns, and the C side widens both exactly.

Parity status of each function (what pins it is listed in the tests):
  valid_rows, ce_rows (with label smoothing), ce_grad_rows (with label
  smoothing), topk_rows (with q), topk_grad_rows -- pinned by closed forms,
  invariants, 120-digit brute force and library routines (tests/test_oracle_pins.py).
  linear_logits, linear_ce_rows, linear_ce_grads (the linear head in front
  of the cross-entropy) -- pinned by the identity head, exact rescaling, a
  50-digit brute force and central differences of the loss in both the
  hidden state and the head.
  jsd.jsd_rows, jsd.jsd_grad_rows (generalized JSD / KL between a student and
  a teacher row, numpy fp64 in oracle/jsd.py) -- pinned by identical rows,
  scipy's relative entropy and Jensen-Shannon distance, the disjoint-support
  maximum, 250-digit brute force with central differences, and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_cev.c")
_LIB = os.path.join(_HERE, "liboracle_cev.so")

BAD_LABEL = 1
BAD_INDEX = 2

F32 = 0
BF16 = 1
F64 = 2

_default = None


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile oracle_cev.c into liboracle_cev.so next to it (gcc, -O2, IEEE:
    no -ffast-math, no FMA contraction, so each operation rounds as written)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
            "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, src, "-lm",
        ])
        os.replace(tmp, out)
    return out


_SAN_LIB = os.path.join(_HERE, "liboracle_cev_san.so")
_CLANG = "/opt/rocm/lib/llvm/bin/clang"


def build_sanitized(src: str = _SRC, out: str = _SAN_LIB) -> str:
    """liboracle_cev_san.so: the oracle under ASan + UBSan (clang, the same IEEE
    flags; load it with clang's ASan runtime preloaded).  Used when the
    environment sets CEV_ORACLE_SANITIZE=1."""
    tmp = out + ".tmp"
    subprocess.check_call([
        _CLANG, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
        "-fno-fast-math", "-Wall", "-Wextra", "-fsanitize=address,undefined",
        "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-shared-libsan",
        "-o", tmp, src, "-lm",
    ])
    os.replace(tmp, out)
    return out


def load_library(path: str):
    """Load an oracle library built from oracle_cev.c (or a test's mutant of it)."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_valid_rows.argtypes = [P, P, I64, I64, I64, P, P]
    lib.oracle_valid_rows.restype = I64
    lib.oracle_ce_rows.argtypes = [P, I64, I64, I64, ctypes.c_int, P, I64, ctypes.c_double,
                                   ctypes.c_double, P, I64, I64, P, P, P, P, P]
    lib.oracle_ce_rows.restype = ctypes.c_int
    lib.oracle_ce_grad_rows.argtypes = [P, I64, I64, I64, ctypes.c_int, P, I64, ctypes.c_double,
                                        ctypes.c_double, P, P, I64, I64, P]
    lib.oracle_ce_grad_rows.restype = ctypes.c_int
    lib.oracle_topk_rows.argtypes = [P, I64, I64, I64, ctypes.c_int, P, I64, I64, I64,
                                     ctypes.c_double, P, I64, I64, P, P]
    lib.oracle_topk_rows.restype = ctypes.c_int
    lib.oracle_topk_grad_rows.argtypes = [P, I64, I64, I64, ctypes.c_int, P, I64, I64, I64,
                                          ctypes.c_double, P, P, I64, I64, P]
    lib.oracle_topk_grad_rows.restype = ctypes.c_int
    return lib


def _load(lib=None):
    global _default
    if lib is not None:
        return lib
    if _default is None:
        if os.environ.get("CEV_ORACLE_SANITIZE") == "1":
            if not os.path.exists(_SAN_LIB) or os.path.getmtime(_SAN_LIB) < os.path.getmtime(_SRC):
                build_sanitized()
            _default = load_library(_SAN_LIB)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            _default = load_library(_LIB)
    return _default


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype_code(logits: np.ndarray) -> int:
    if logits.dtype == np.float32:
        return F32
    if logits.dtype == np.uint16:
        return BF16
    if logits.dtype == np.float64:
        return F64
    raise TypeError("oracle logits must be float32, float64 or uint16 (bf16 bit patterns)")


def _check_2d(logits):
    if logits.ndim != 2 or logits.strides[1] != logits.itemsize:
        raise ValueError("logits must be 2-D with unit column stride")
    if logits.strides[0] % logits.itemsize:
        raise ValueError("row stride must be a whole number of elements")
    return logits.strides[0] // logits.itemsize


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ranges(rows, rows_list, threads):
    """Split either [0, rows) or an explicit row list into work items."""
    if rows_list is not None:
        rl = np.asarray(rows_list, dtype=np.int64)
        return [(int(r), int(r) + 1) for r in rl]
    n = max(1, min(threads, rows))
    step = (rows + n - 1) // n
    return [(a, min(rows, a + step)) for a in range(0, rows, step)]


def _labels(labels, rows):
    lab = np.ascontiguousarray(labels, dtype=np.int64)
    if lab.shape != (rows,):
        raise ValueError("labels must have shape [rows]")
    return lab


def _mask(row_mask, rows):
    if row_mask is None:
        return None
    m = np.ascontiguousarray(row_mask, dtype=np.uint8)
    if m.shape != (rows,):
        raise ValueError("row_mask must have shape [rows]")
    return m


def valid_rows(labels, row_mask=None, vocab=None, ignore_index=-100, lib=None):
    """Ascending list of valid rows (int64) and the status bits."""
    lab = np.ascontiguousarray(labels, dtype=np.int64)
    rows = lab.shape[0]
    m = _mask(row_mask, rows)
    out = np.empty(rows, dtype=np.int64)
    st = ctypes.c_int32(0)
    n = _load(lib).oracle_valid_rows(_ptr(lab), _ptr(m), rows, int(vocab), int(ignore_index),
                                  _ptr(out), ctypes.addressof(st))
    return out[:n].copy(), int(st.value)


def ce_rows(logits, labels, temperature=1.0, row_mask=None, ignore_index=-100, rows_list=None,
            threads=None, want_entropy=True, want_argmax=True, lib=None, label_smoothing=0.0):
    """Per-row forward.  Returns dict of float64/int64 arrays over all rows
    (rows not in rows_list, if given, are left as NaN / -2) and the status."""
    lib = _load(lib)
    dt = _dtype_code(logits)
    stride = _check_2d(logits)
    rows, vocab = logits.shape
    lab = _labels(labels, rows)
    m = _mask(row_mask, rows)
    out = {
        "logp": np.full(rows, np.nan),
        "loss": np.full(rows, np.nan),
        "q": np.full(rows, np.nan),
        "entropy": np.full(rows, np.nan) if want_entropy else None,
        "argmax": np.full(rows, -2, dtype=np.int64) if want_argmax else None,
    }
    threads = threads or default_threads()

    def work(rng):
        return lib.oracle_ce_rows(_ptr(logits), rows, vocab, stride, dt, _ptr(lab),
                                  int(ignore_index), float(temperature), float(label_smoothing),
                                  _ptr(m), rng[0], rng[1],
                                  _ptr(out["logp"]), _ptr(out["loss"]), _ptr(out["entropy"]),
                                  _ptr(out["argmax"]), _ptr(out["q"]))

    st = 0
    with ThreadPoolExecutor(threads) as ex:
        for s in ex.map(work, _ranges(rows, rows_list, threads)):
            st |= s
    out["status"] = st
    return out


def ce_grad_rows(logits, labels, g, temperature=1.0, row_mask=None, ignore_index=-100, r0=0,
                 r1=None, threads=None, lib=None, label_smoothing=0.0):
    """float64 dlogits for rows [r0, r1) as an array of shape [r1 - r0, vocab]."""
    lib = _load(lib)
    dt = _dtype_code(logits)
    stride = _check_2d(logits)
    rows, vocab = logits.shape
    r1 = rows if r1 is None else r1
    lab = _labels(labels, rows)
    m = _mask(row_mask, rows)
    gg = np.ascontiguousarray(g, dtype=np.float64)
    out = np.empty((r1 - r0, vocab), dtype=np.float64)
    threads = threads or default_threads()
    n = r1 - r0
    parts = _ranges(n, None, threads) if n > 0 else []

    def work(rng):
        a, b = rng
        return lib.oracle_ce_grad_rows(_ptr(logits), rows, vocab, stride, dt, _ptr(lab),
                                       int(ignore_index), float(temperature),
                                       float(label_smoothing), _ptr(m), _ptr(gg),
                                       r0 + a, r0 + b, out[a:].ctypes.data)

    st = 0
    with ThreadPoolExecutor(threads) as ex:
        for s in ex.map(work, parts):
            st |= s
    return out


def topk_rows(logits, indices, temperature=1.0, row_mask=None, ignore_index=-100, rows_list=None,
              threads=None, lib=None, want_q=False):
    """float64 log p at K gathered indices per row: [rows, K] (rows outside
    rows_list, if given, are NaN) and the status; with want_q also
    q = 1 - p at each gathered index (0 for ignored entries and masked rows)."""
    lib = _load(lib)
    dt = _dtype_code(logits)
    stride = _check_2d(logits)
    rows, vocab = logits.shape
    idx = np.asarray(indices, dtype=np.int64)
    if idx.ndim != 2 or idx.shape[0] != rows or idx.strides[1] != 8:
        raise ValueError("indices must be [rows, K] int64 with unit column stride")
    K = idx.shape[1]
    m = _mask(row_mask, rows)
    out = np.full((rows, K), np.nan)
    q = np.full((rows, K), np.nan) if want_q else None
    threads = threads or default_threads()

    def work(rng):
        return lib.oracle_topk_rows(_ptr(logits), rows, vocab, stride, dt, _ptr(idx), K,
                                    idx.strides[0] // 8, int(ignore_index), float(temperature),
                                    _ptr(m), rng[0], rng[1], _ptr(out), _ptr(q))

    st = 0
    with ThreadPoolExecutor(threads) as ex:
        for s in ex.map(work, _ranges(rows, rows_list, threads)):
            st |= s
    if want_q:
        return out, q, st
    return out, st


def topk_grad_rows(logits, indices, g, temperature=1.0, row_mask=None, ignore_index=-100, r0=0,
                   r1=None, threads=None, lib=None):
    """float64 gradient of sum_k g[r, k] log p_{i_k} for rows [r0, r1):
    an array of shape [r1 - r0, vocab]."""
    lib = _load(lib)
    dt = _dtype_code(logits)
    stride = _check_2d(logits)
    rows, vocab = logits.shape
    r1 = rows if r1 is None else r1
    idx = np.asarray(indices, dtype=np.int64)
    if idx.ndim != 2 or idx.shape[0] != rows or idx.strides[1] != 8:
        raise ValueError("indices must be [rows, K] int64 with unit column stride")
    K = idx.shape[1]
    gg = np.ascontiguousarray(g, dtype=np.float64)
    if gg.shape != (rows, K):
        raise ValueError("g must be [rows, K]")
    m = _mask(row_mask, rows)
    out = np.empty((r1 - r0, vocab), dtype=np.float64)
    threads = threads or default_threads()
    n = r1 - r0
    parts = _ranges(n, None, threads) if n > 0 else []

    def work(rng):
        a, b = rng
        return lib.oracle_topk_grad_rows(_ptr(logits), rows, vocab, stride, dt, _ptr(idx), K,
                                         idx.strides[0] // 8, int(ignore_index),
                                         float(temperature), _ptr(m), _ptr(gg), r0 + a, r0 + b,
                                         out[a:].ctypes.data)

    st = 0
    with ThreadPoolExecutor(threads) as ex:
        for s in ex.map(work, parts):
            st |= s
    return out


# ---------------------------------------------------------------------------
# Linear head in front of the cross-entropy (the fused linear CE / log-prob
# setting of the unsloth-zoo #2080 Summary quoted on the Liger-Kernel PR #1555
# page: logits = hidden x head^T, never stored in full by the fused kernels).

def _widen(a: np.ndarray) -> np.ndarray:
    """Stored values as float64: bf16 bit patterns (uint16), fp32 or fp64."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError("hidden / head must be uint16 (bf16 bits), float32 or float64")


def linear_logits(hidden, weight, rows=None, vchunk=16384):
    """logits[r, j] = sum_k hidden[r, k] * weight[j, k] in float64 (a library
    matmul of the widened stored values; every product of two bf16 values is
    exact in float64).  hidden [R, H], weight [V, H]; rows selects rows."""
    h = _widen(hidden if rows is None else hidden[np.asarray(rows, dtype=np.int64)])
    V = weight.shape[0]
    out = np.empty((h.shape[0], V), dtype=np.float64)
    for j0 in range(0, V, vchunk):
        j1 = min(V, j0 + vchunk)
        out[:, j0:j1] = h @ _widen(weight[j0:j1]).T
    return out


def linear_ce_rows(hidden, weight, labels, temperature=1.0, row_mask=None, ignore_index=-100,
                   rows_list=None, label_smoothing=0.0, want_entropy=True, lib=None):
    """ce_rows on the float64 logits hidden x weight^T.  Rows outside
    rows_list (if given) are NaN / -2, as in ce_rows."""
    R = hidden.shape[0]
    rl = np.arange(R, dtype=np.int64) if rows_list is None else np.asarray(rows_list, np.int64)
    lab = np.asarray(labels, dtype=np.int64)
    z = linear_logits(hidden, weight, rl)
    sub_mask = None if row_mask is None else np.ascontiguousarray(np.asarray(row_mask)[rl])
    sub = ce_rows(z, np.ascontiguousarray(lab[rl]), temperature, row_mask=sub_mask,
                  ignore_index=ignore_index, label_smoothing=label_smoothing,
                  want_entropy=want_entropy, lib=lib)
    out = {}
    for k, v in sub.items():
        if k == "status":
            out[k] = v
        elif v is None:
            out[k] = None
        else:
            full = np.full(R, -2 if v.dtype == np.int64 else np.nan, dtype=v.dtype)
            full[rl] = v
            out[k] = full
    return out


def linear_ce_grads(hidden, weight, labels, g, temperature=1.0, row_mask=None, ignore_index=-100,
                    rows_list=None, label_smoothing=0.0, want_weight=True, lib=None):
    """Gradients of sum_r g[r] loss[r] through logits = hidden x weight^T:
    dlogits = ce_grad_rows(logits), dhidden = dlogits x weight,
    dweight = dlogits^T x hidden (the chain rule through the product).
    With rows_list, dhidden holds those rows only and dweight is None (it sums
    over every row)."""
    R = hidden.shape[0]
    rl = np.arange(R, dtype=np.int64) if rows_list is None else np.asarray(rows_list, np.int64)
    lab = np.asarray(labels, dtype=np.int64)
    gg = np.asarray(g, dtype=np.float64)
    z = linear_logits(hidden, weight, rl)
    sub_mask = None if row_mask is None else np.ascontiguousarray(np.asarray(row_mask)[rl])
    dl = ce_grad_rows(z, np.ascontiguousarray(lab[rl]), np.ascontiguousarray(gg[rl]),
                      temperature, row_mask=sub_mask, ignore_index=ignore_index,
                      label_smoothing=label_smoothing, lib=lib)
    w64 = _widen(weight)
    out = {"dhidden": dl @ w64, "dweight": None}
    if want_weight and rows_list is None:
        out["dweight"] = dl.T @ _widen(hidden)
    return out
