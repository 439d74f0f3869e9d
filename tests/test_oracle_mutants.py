"""Plant plausible mistakes in a copy of the oracle's C source (on the CPU) and
show that the pins catch every one of them: a dropped term, a wrong sign, a
wrong index, a transposed operand, a missing 1/T."""
import os
import shutil
import subprocess

import pytest

import oracle
import pinlib

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle_cev.c")

# (name, text in oracle_cev.c, replacement)
MUTANTS = [
    ("softplus_drops_one", "log1p(exp(-fabs(u)))", "log(exp(-fabs(u)))"),
    ("softplus_sign", "fmax(u, 0.0) + log1p", "fmax(-u, 0.0) + log1p"),
    ("sigmoid_neg_branch", "return e / (1.0 + e);", "return 1.0 / (1.0 + e);"),
    ("sum_includes_target", "        if (j != excl)\n            s += exp",
     "        if (1)\n            s += exp"),
    ("lse_drops_shift", "return m + log(s);", "return log(s);"),
    ("u_sign", "double u = lse_excluding(row, dtype, vocab, T, t) - xt;\n        double l = softplus",
     "double u = xt - lse_excluding(row, dtype, vocab, T, t);\n        double l = softplus"),
    ("target_not_scaled", "double xt = load_z(row, dtype, t) / T;\n        double u = lse_excluding(row, dtype, vocab, T, t) - xt;\n        double l = softplus",
     "double xt = load_z(row, dtype, t);\n        double u = lse_excluding(row, dtype, vocab, T, t) - xt;\n        double l = softplus"),
    ("entropy_drops_target_term", "double h = exp(-l) * l;", "double h = 0.0;"),
    ("entropy_sign", "h += exp(x - lse) * (lse - x);", "h += exp(x - lse) * (x - lse);"),
    ("argmax_last_tie", "if (z > best) {", "if (z >= best) {"),
    ("grad_target_sign", "w * (-sigmoid(u) + eps - ev)", "w * (sigmoid(u) + eps - ev)"),
    ("grad_drops_chain_rule", "double w = g[r] / T;", "double w = g[r];"),
    ("grad_other_index", "w * (exp(load_z(row, dtype, j) / T - lse) - ev)",
     "w * (exp(load_z(row, dtype, vocab - 1 - j) / T - lse) - ev)"),
    ("bf16_widen_shift", "<< 16;", "<< 15;"),
    ("row_stride_ignored", "(size_t)r * (size_t)row_stride * esz", "(size_t)r * (size_t)1 * esz"),
    ("topk_no_exclusion", "double u = lse_excluding(row, dtype, vocab, T, i) - xi;\n                v",
     "double u = lse_excluding(row, dtype, vocab, T, -1) - xi;\n                v"),
    ("smoothing_scale", "loss[r] = (1.0 - eps) * l + eps * ls;", "loss[r] = (1.0 - eps) * l + ls;"),
    ("smoothing_term_sign", "ls += lse - load_z(row, dtype, j) / T;", "ls += load_z(row, dtype, j) / T - lse;"),
    ("smoothing_grad_target", "w * (-sigmoid(u) + eps - ev)", "w * (-sigmoid(u) + eps)"),
    ("smoothing_grad_other", "/ T - lse) - ev)", "/ T - lse))"),
    ("topk_q_sign", "qk = sigmoid(u);", "qk = sigmoid(-u);"),
    ("topk_grad_gathered", "o[i] = (gj * qj - pj * (gs - gj)) / T;", "o[i] = (gj * qj - pj * gs) / T;"),
    ("topk_grad_other_sign", "o[j] = -(gs / T) * exp(", "o[j] = (gs / T) * exp("),
    ("topk_grad_dup", "for (int64_t k2 = k; k2 < K; ++k2)", "for (int64_t k2 = k; k2 < k + 1; ++k2)"),
    ("topk_row_index", "int64_t i = idx[r * idx_stride + k];\n            double v = 0.0, qk",
     "int64_t i = idx[k * idx_stride + r % 1];\n            double v = 0.0, qk"),
    ("mask_inverted", "if (row_mask && row_mask[r] == 0)\n        return 0;",
     "if (row_mask && row_mask[r] != 0)\n        return 0;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not unique or missing"
    src = tmp_path / "oracle_cev.c"
    src.write_text(text.replace(old, new))
    lib_path = str(tmp_path / "liboracle_mut.so")
    oracle.build(force=True, src=str(src), out=lib_path)
    lib = oracle.load_library(lib_path)
    caught = []
    for check in pinlib.ALL_CHECKS:
        try:
            check(lib=lib)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(check.__name__)
            break
    assert caught, f"no pin caught mutant {name}"


def test_unmutated_source_passes_all_pins(tmp_path):
    src = tmp_path / "oracle_cev.c"
    shutil.copy(SRC, src)
    lib_path = str(tmp_path / "liboracle_copy.so")
    oracle.build(force=True, src=str(src), out=lib_path)
    lib = oracle.load_library(lib_path)
    for check in pinlib.ALL_CHECKS:
        check(lib=lib)


# Mistakes planted in the Python half of the oracle (the linear head in front
# of the cross-entropy): a missing transpose, a gradient through the wrong
# operand layout, rows out of step, labels not following a row subset.
PKG = os.path.dirname(oracle.__file__)
PY_MUTANTS = [
    ("logits_untransposed_head", "out[:, j0:j1] = h @ _widen(weight[j0:j1]).T",
     "out[:, j0:j1] = h @ _widen(weight[j0:j1])"),
    ("dhidden_transposed_head", '"dhidden": dl @ w64', '"dhidden": dl @ w64.T'),
    ("dweight_rows_shifted", 'out["dweight"] = dl.T @ _widen(hidden)',
     'out["dweight"] = dl.T @ np.roll(_widen(hidden), 1, axis=0)'),
    ("subset_labels_not_followed", "sub = ce_rows(z, np.ascontiguousarray(lab[rl]), temperature",
     "sub = ce_rows(z, np.ascontiguousarray(lab[:rl.size]), temperature"),
]


def _load_mutant_package(tmp_path, old, new):
    import importlib.util
    import sys
    d = tmp_path / "oracle_mut"
    d.mkdir()
    text = open(os.path.join(PKG, "__init__.py")).read()
    assert text.count(old) == 1, "mutation site not unique or missing"
    (d / "__init__.py").write_text(text.replace(old, new))
    shutil.copy(SRC, d / "oracle_cev.c")
    name = f"oracle_mut_{abs(hash((old, new)))}"
    spec = importlib.util.spec_from_file_location(name, d / "__init__.py",
                                                  submodule_search_locations=[str(d)])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,old,new", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_linear_pins_catch_python_mutant(tmp_path, name, old, new):
    mod = _load_mutant_package(tmp_path, old, new)
    caught = []
    for check in pinlib.LINEAR_CHECKS:
        try:
            check(orc=mod)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
            break
    assert caught, f"no pin caught mutant {name}"


def test_unmutated_python_oracle_passes_linear_pins(tmp_path):
    mod = _load_mutant_package(tmp_path, "F64 = 2\n", "F64 = 2\n\n")
    for check in pinlib.LINEAR_CHECKS:
        check(orc=mod)


# Mistakes planted in the generalized-JSD oracle (oracle/jsd.py, a plain
# numpy module): each must be caught by one of the JSD pins.
JSD_MUTANTS = [
    ("mixture_weights_swapped", "a = -np.log1p(beta * np.expm1(dn))",
     "a = -np.log1p((1.0 - beta) * np.expm1(dn))"),
    ("naive_log_softmax_at_argmax", "ls[a] = -np.log1p(S)",
     "ls[a] = x[a] - np.log(np.sum(np.exp(x)))"),
    ("reverse_kl_grad_without_loss", "d = ps * ((ls - lt) - loss) / T", "d = ps * (ls - lt) / T"),
    ("argmax_rule_dropped", "    d[a] = 0.0\n    d[a] = -np.sum(d)\n", "    pass\n"),
    ("teacher_not_tempered", "lt, a_t, _ = log_softmax_safe(_widen(zt) / T)",
     "lt, a_t, _ = log_softmax_safe(_widen(zt))"),
    ("forward_kl_reversed", "return float(np.sum(pt * (lt - ls))), 0.0, ls, lt, None",
     "return float(np.sum(pt * (ls - lt))), 0.0, ls, lt, None"),
    ("mixed_grad_without_K", "d = (1.0 - beta) * ps * (r - K) / T", "d = (1.0 - beta) * ps * r / T"),
]


def _load_jsd_mutant(tmp_path, old, new):
    import importlib.util
    text = open(os.path.join(PKG, "jsd.py")).read()
    assert text.count(old) == 1, "mutation site not unique or missing"
    f = tmp_path / "jsd_mut.py"
    f.write_text(text.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"jsd_mut_{abs(hash((old, new)))}", f)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,old,new", JSD_MUTANTS, ids=[m[0] for m in JSD_MUTANTS])
def test_jsd_pins_catch_mutant(tmp_path, name, old, new):
    import warnings
    mod = _load_jsd_mutant(tmp_path, old, new)
    caught = []
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        for check in pinlib.JSD_CHECKS:
            try:
                check(orc=mod)
            except (AssertionError, ValueError, IndexError, FloatingPointError):
                caught.append(check.__name__)
                break
    assert caught, f"no pin caught mutant {name}"


def test_unmutated_jsd_oracle_passes_pins(tmp_path):
    mod = _load_jsd_mutant(tmp_path, "import numpy as np\n", "import numpy as np\n\n")
    for check in pinlib.JSD_CHECKS:
        check(orc=mod)
