"""CPU-side checks of the C ABI: the library loads, exports every function that
include/cevocab.h declares, and rejects bad arguments on the host before any
launch (these calls never reach the GPU, so they run without one)."""
import ctypes
import os
import re

import pytest

import cross_entropy_vocab_amd as cev
from cross_entropy_vocab_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cevocab.h")

E = dict(OK=0, NULL=-1, SHAPE=-2, STRIDE=-3, ALIGN=-4, DTYPE=-5, TEMP=-6, WORKSPACE=-7,
         ALIAS=-8, LAUNCH=-9, SMOOTH=-10, BETA=-11)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from cross_entropy_vocab_amd import build
        build.build()
    return _lib.get()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^(?:int|size_t|const char \*)\s*(\w+)\(", text, flags=re.M)


def test_header_declares_the_boundary():
    names = set(declared_functions())
    assert {"sls_forward", "sls_topk_forward", "sls_topk_backward", "ce_forward", "ce_backward",
            "ce_fused", "ce_vocab_shard_forward", "ce_vocab_merge", "ce_vocab_shard_backward",
            "lce_forward", "lce_backward", "lce_workspace_size",
            "cev_workspace_size", "cev_status_string", "cev_version"} <= names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, name


def test_codes_match_header():
    text = open(HEADER).read()
    for key, val in E.items():
        if key == "OK":
            continue
        m = re.search(r"CEV_E%s\s*=\s*(-?\d+)" % key, text)
        assert m and int(m.group(1)) == val, key
    assert re.search(r"CEV_STATUS_BAD_LABEL\s+1u", text)
    assert re.search(r"CEV_STATUS_BAD_INDEX\s+2u", text)
    assert re.search(r"CEV_STATUS_BAD_PARTS\s+4u", text)
    assert re.search(r"CEV_PART_ENTROPY\s+1u", text) and re.search(r"CEV_PART_VALUE_SUM\s+2u", text)
    assert cev.STATUS_BAD_LABEL == 1 and cev.STATUS_BAD_INDEX == 2 and cev.STATUS_BAD_PARTS == 4
    assert cev.PART_ENTROPY == 1 and cev.PART_VALUE_SUM == 2 and cev.PARTIAL_BYTES == 48


def test_version_and_strings(lib):
    assert lib.cev_version() == 210
    for code in E.values():
        assert lib.cev_status_string(code)
    assert lib.cev_workspace_size(10, 100, 0) == 88          # list + count only
    assert lib.cev_workspace_size(8192, 152064, 1) == 8193 * 8  # enough rows: no split
    # few long rows split over workgroups: 40-byte partial records (max, its
    # column, sum, entropy term, value sum) follow the 32-byte aligned list
    assert lib.cev_workspace_size(12, 152064, 1) == 128 + 12 * 9 * 40
    assert lib.cev_workspace_size(64, 152064, 1) == 65 * 8     # 64 rows: whole rows
    assert lib.cev_workspace_size(-1, 100, 0) == 0
    assert lib.cev_workspace_size(10, 100, 5) == 0


# fake, never-dereferenced device addresses (validation fails before any launch)
A = 0x10000
B = 0x900000


def sls(lib, **kw):
    a = dict(logits=A, rows=4, vocab=100, stride=100, dtype=0, labels=A, ig=-100, T=1.0,
             mask=None, logp=A, ent=None, arg=None, status=None, stream=None)
    a.update(kw)
    return lib.sls_forward(a["logits"], a["rows"], a["vocab"], a["stride"], a["dtype"],
                           a["labels"], a["ig"], a["T"], a["mask"], a["logp"], a["ent"], a["arg"],
                           a["status"], a["stream"])


def test_sls_forward_validation(lib):
    assert sls(lib, dtype=7) == E["DTYPE"]
    assert sls(lib, T=0.0) == E["TEMP"]
    assert sls(lib, T=-1.0) == E["TEMP"]
    assert sls(lib, T=float("nan")) == E["TEMP"]
    assert sls(lib, T=float("inf")) == E["TEMP"]
    assert sls(lib, T=1e-40) == E["TEMP"]
    assert sls(lib, rows=-1) == E["SHAPE"]
    assert sls(lib, vocab=0) == E["SHAPE"]
    assert sls(lib, rows=2 ** 31) == E["SHAPE"]
    assert sls(lib, rows=2 ** 22 + 1) == E["SHAPE"]
    assert sls(lib, stride=99) == E["STRIDE"]
    assert sls(lib, logits=None) == E["NULL"]
    assert sls(lib, labels=None) == E["NULL"]
    assert sls(lib, logp=None) == E["NULL"]
    assert sls(lib, logits=A + 1) == E["ALIGN"]
    assert sls(lib, logits=A + 1, dtype=1) == E["ALIGN"]
    assert sls(lib, labels=A + 4) == E["ALIGN"]
    assert sls(lib, logp=A + 2) == E["ALIGN"]
    assert sls(lib, arg=A + 4) == E["ALIGN"]
    assert sls(lib, status=A + 2) == E["ALIGN"]
    # rows == 0 is a no-op that succeeds without touching any pointer
    assert sls(lib, rows=0, logits=None, labels=None, logp=None) == E["OK"]


def test_topk_validation(lib):
    def call(**kw):
        a = dict(logits=A, rows=4, vocab=100, stride=100, dtype=1, idx=A, K=8, istride=8,
                 ig=-100, T=0.7, mask=None, logp=A, q=None, saved=None, status=None)
        a.update(kw)
        return lib.sls_topk_forward(a["logits"], a["rows"], a["vocab"], a["stride"], a["dtype"],
                                    a["idx"], a["K"], a["istride"], a["ig"], a["T"], a["mask"],
                                    a["logp"], a["q"], a["saved"], a["status"], None)
    assert call(K=0) == E["SHAPE"]
    assert call(K=1025) == E["SHAPE"]
    assert call(istride=7) == E["STRIDE"]
    assert call(idx=None) == E["NULL"]
    assert call(idx=A + 4) == E["ALIGN"]
    assert call(q=A + 2) == E["ALIGN"]
    assert call(saved=A + 8) == E["ALIGN"]
    assert call(T=0.0) == E["TEMP"]
    assert call(rows=0) == E["OK"]


def test_topk_backward_validation(lib):
    def call(**kw):
        a = dict(logits=A, rows=4, vocab=100, stride=100, dtype=1, idx=A, K=8, istride=8,
                 ig=-100, T=0.7, mask=None, g=A, saved=A, q=A, dl=B, dstride=100, status=None)
        a.update(kw)
        return lib.sls_topk_backward(a["logits"], a["rows"], a["vocab"], a["stride"], a["dtype"],
                                     a["idx"], a["K"], a["istride"], a["ig"], a["T"], a["mask"],
                                     a["g"], a["saved"], a["q"], a["dl"], a["dstride"],
                                     a["status"], None)
    assert call(K=0) == E["SHAPE"]
    assert call(K=1025) == E["SHAPE"]
    assert call(istride=7) == E["STRIDE"]
    assert call(dstride=99) == E["STRIDE"]
    for k in ("idx", "g", "saved", "q", "dl"):
        assert call(**{k: None}) == E["NULL"], k
    assert call(saved=A + 8) == E["ALIGN"]
    assert call(q=A + 2) == E["ALIGN"]
    assert call(dl=B + 1) == E["ALIGN"]
    assert call(dl=A) == E["ALIAS"]
    assert call(T=float("inf")) == E["TEMP"]
    assert call(dtype=2) == E["DTYPE"]
    assert call(rows=0) == E["OK"]


def test_ce_forward_validation(lib):
    def call(**kw):
        a = dict(logits=A, rows=4, vocab=100, stride=100, dtype=0, labels=A, ig=-100, T=1.0,
                 eps=0.0, mask=None, loss=A, saved=A, logp=None, ent=None, arg=None, vr=None,
                 nv=None, ws=None, wsb=0, status=None)
        a.update(kw)
        return lib.ce_forward(a["logits"], a["rows"], a["vocab"], a["stride"], a["dtype"],
                              a["labels"], a["ig"], a["T"], a["eps"], a["mask"], a["loss"],
                              a["saved"],
                              a["logp"], a["ent"], a["arg"], a["vr"], a["nv"], a["ws"], a["wsb"],
                              a["status"], None)
    # A list output asked for without the other and without a workspace (both
    # absent with no workspace is accepted: every row is swept in place).
    assert call(vr=A) == E["NULL"]
    assert call(nv=A) == E["NULL"]
    assert call(ws=A, wsb=39) == E["WORKSPACE"]      # needs (4 + 1) * 8 = 40 bytes
    assert call(ws=A + 4, wsb=40) == E["ALIGN"]
    assert call(vr=A, nv=A, saved=A + 8) == E["ALIGN"]  # saved records are 16-byte aligned
    assert call(vr=A, nv=A, loss=None) == E["NULL"]
    assert call(vr=A, nv=A, saved=None) == E["NULL"]
    assert call(vr=A, nv=A, dtype=3) == E["DTYPE"]
    for eps in (-0.1, 1.5, float("nan"), float("inf")):
        assert call(vr=A, nv=A, eps=eps) == E["SMOOTH"]
        assert call(rows=0, eps=eps) == E["SMOOTH"]
    assert call(rows=0) == E["OK"]


def test_ce_backward_validation(lib):
    def call(**kw):
        a = dict(logits=A, rows=4, vocab=100, stride=100, dtype=1, labels=A, ig=-100, T=1.0,
                 eps=0.0, mask=None, g=A, saved=A, dl=B, dstride=100, status=None)
        a.update(kw)
        return lib.ce_backward(a["logits"], a["rows"], a["vocab"], a["stride"], a["dtype"],
                               a["labels"], a["ig"], a["T"], a["eps"], a["mask"], a["g"],
                               a["saved"],
                               a["dl"], a["dstride"], a["status"], None)
    assert call(dl=A) == E["ALIAS"]
    assert call(dl=A + 2 * 350) == E["ALIAS"]                 # overlaps the last row
    assert call(dstride=50) == E["STRIDE"]
    assert call(g=None) == E["NULL"]
    assert call(saved=None) == E["NULL"]
    assert call(dl=None) == E["NULL"]
    assert call(saved=A + 8) == E["ALIGN"]
    assert call(dl=B + 1) == E["ALIGN"]
    assert call(T=float("nan")) == E["TEMP"]
    assert call(eps=-1e-9) == E["SMOOTH"]
    assert call(rows=0) == E["OK"]


def test_ce_fused_validation(lib):
    def call(**kw):
        a = dict(logits=A, rows=4, vocab=100, stride=100, dtype=1, labels=A, ig=-100, T=1.0,
                 eps=0.0, mask=None, g=A, loss=A, saved=A, logp=None, ent=None, arg=None, dl=B,
                 dstride=100, vr=None, nv=None, ws=None, wsb=0, status=None)
        a.update(kw)
        return lib.ce_fused(a["logits"], a["rows"], a["vocab"], a["stride"], a["dtype"],
                            a["labels"], a["ig"], a["T"], a["eps"], a["mask"], a["g"], a["loss"],
                            a["saved"], a["logp"], a["ent"], a["arg"], a["dl"], a["dstride"],
                            a["vr"], a["nv"], a["ws"], a["wsb"], a["status"], None)
    assert call(dl=A) == E["ALIAS"]
    assert call(g=None) == E["NULL"]
    assert call(saved=None) == E["NULL"]
    assert call(loss=None) == E["NULL"]
    assert call(dl=None) == E["NULL"]
    assert call(saved=A + 8) == E["ALIGN"]
    assert call(dstride=99) == E["STRIDE"]
    assert call(vr=A) == E["NULL"]                    # count missing and no workspace
    assert call(vr=A, ws=A, wsb=39) == E["WORKSPACE"]
    assert call(T=0.0) == E["TEMP"]
    assert call(dtype=9) == E["DTYPE"]
    assert call(eps=1.0 + 1e-12) == E["SMOOTH"]
    assert call(rows=0) == E["OK"]


def test_vocab_shard_forward_validation(lib):
    def call(**kw):
        a = dict(logits=A, rows=4, sv=100, stride=100, dtype=1, off=200, V=1000, labels=A,
                 ig=-100, T=1.0, mask=None, what=0, parts=A, status=None)
        a.update(kw)
        return lib.ce_vocab_shard_forward(a["logits"], a["rows"], a["sv"], a["stride"],
                                          a["dtype"], a["off"], a["V"], a["labels"], a["ig"],
                                          a["T"], a["mask"], a["what"], a["parts"], a["status"],
                                          None)
    assert call(off=-1) == E["SHAPE"]
    assert call(off=901) == E["SHAPE"]            # shard past the vocabulary
    assert call(V=99) == E["SHAPE"]
    assert call(sv=0) == E["SHAPE"]
    assert call(stride=99) == E["STRIDE"]
    assert call(labels=None) == E["NULL"]
    assert call(parts=None) == E["NULL"]
    assert call(parts=A + 4) == E["ALIGN"]
    assert call(T=0.0) == E["TEMP"]
    assert call(dtype=5) == E["DTYPE"]
    assert call(rows=0, off=-1) == E["SHAPE"]
    assert call(rows=0) == E["OK"]


def test_vocab_merge_validation(lib):
    def call(**kw):
        a = dict(parts=A, P=8, rows=4, V=1000, labels=A, ig=-100, T=1.0, eps=0.0, mask=None,
                 loss=A, saved=A, logp=None, ent=None, arg=None, status=None)
        a.update(kw)
        return lib.ce_vocab_merge(a["parts"], a["P"], a["rows"], a["V"], a["labels"], a["ig"],
                                  a["T"], a["eps"], a["mask"], a["loss"], a["saved"], a["logp"],
                                  a["ent"], a["arg"], a["status"], None)
    assert call(P=0) == E["SHAPE"]
    assert call(P=4097) == E["SHAPE"]
    assert call(V=0) == E["SHAPE"]
    assert call(rows=-1) == E["SHAPE"]
    assert call(parts=None) == E["NULL"]
    assert call(loss=None) == E["NULL"]
    assert call(saved=None) == E["NULL"]
    assert call(parts=A + 4) == E["ALIGN"]
    assert call(saved=A + 8) == E["ALIGN"]
    assert call(T=-1.0) == E["TEMP"]
    assert call(eps=2.0) == E["SMOOTH"]
    assert call(rows=0, parts=None) == E["OK"]


def test_vocab_shard_backward_validation(lib):
    def call(**kw):
        a = dict(logits=A, rows=4, sv=100, stride=100, dtype=1, off=0, V=400, labels=A,
                 ig=-100, T=1.0, eps=0.0, mask=None, g=A, saved=A, dl=B, dstride=100,
                 status=None)
        a.update(kw)
        return lib.ce_vocab_shard_backward(a["logits"], a["rows"], a["sv"], a["stride"],
                                           a["dtype"], a["off"], a["V"], a["labels"], a["ig"],
                                           a["T"], a["eps"], a["mask"], a["g"], a["saved"],
                                           a["dl"], a["dstride"], a["status"], None)
    assert call(off=301) == E["SHAPE"]
    assert call(dstride=99) == E["STRIDE"]
    assert call(g=None) == E["NULL"]
    assert call(saved=A + 4) == E["ALIGN"]
    assert call(dl=A + 2) == E["ALIAS"]
    assert call(eps=-0.5) == E["SMOOTH"]
    assert call(rows=0) == E["OK"]


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(_lib.LibraryMissing):
        cev.version()


def test_product_never_imports_the_oracle():
    """The package and its sources do not reference the oracle."""
    pkg = os.path.join(ROOT, "cross_entropy_vocab_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "oracle_" not in text, f


def test_lce_validation(lib):
    def fwd(**kw):
        a = dict(h=A, rows=4, hd=128, hs=128, w=B, V=1000, ws=128, labels=A, ig=-100, T=1.0,
                 eps=0.0, mask=None, loss=A, saved=A, logp=None, ent=None, arg=None, lg=None,
                 lgs=0, wk=A, wkb=1 << 30, status=None)
        a.update(kw)
        return lib.lce_forward(a["h"], a["rows"], a["hd"], a["hs"], a["w"], a["V"], a["ws"],
                               a["labels"], a["ig"], a["T"], a["eps"], a["mask"], a["loss"],
                               a["saved"], a["logp"], a["ent"], a["arg"], a["lg"], a["lgs"],
                               a["wk"], a["wkb"], a["status"], None)
    assert fwd(hd=100, hs=104) == E["SHAPE"]          # hidden size not a multiple of 64
    assert fwd(hd=0) == E["SHAPE"]
    assert fwd(hs=120) == E["STRIDE"]
    assert fwd(hs=132) == E["STRIDE"]                 # stride not a multiple of 8
    assert fwd(ws=64) == E["STRIDE"]
    assert fwd(h=A + 8) == E["ALIGN"]                 # 16-byte alignment
    assert fwd(w=B + 8) == E["ALIGN"]
    assert fwd(wk=None) == E["NULL"]
    assert fwd(saved=None) == E["NULL"]
    assert fwd(wkb=lib.lce_workspace_size(4, 128, 1000) - 1) == E["WORKSPACE"]
    assert fwd(T=0.0) == E["TEMP"]
    assert fwd(eps=-1.0) == E["SMOOTH"]
    assert fwd(V=0) == E["SHAPE"]
    assert fwd(rows=0, h=None, w=None) == E["OK"]
    # stored logits: row stride at least the vocab and a multiple of 4, 16-byte aligned
    assert fwd(lg=A, lgs=996) == E["STRIDE"]
    assert fwd(lg=A, lgs=1002) == E["STRIDE"]
    assert fwd(lg=A + 4, lgs=1000) == E["ALIGN"]
    assert fwd(lg=None, lgs=7, wkb=0) == E["WORKSPACE"]   # stride ignored without logits
    # the stored logits (4 rows x 1000 fp32 = 16000 bytes) overlapping hidden,
    # the head or the workspace (each case clear of the other two)
    W2 = 0x80000000
    assert fwd(lg=A + 512, lgs=1000, wk=W2) == E["ALIAS"]
    assert fwd(lg=B + 4096, lgs=1000, wk=W2) == E["ALIAS"]
    assert fwd(lg=0x40000000, lgs=1000, wk=0x40000000 + 16000 - 16) == E["ALIAS"]
    assert fwd(lg=0x40000000, lgs=1000, wk=0x40000000 + 16000, wkb=0) == E["WORKSPACE"]
    # dlogits [R64, V64] (bf16) and up to 8 split-K partial products of dhidden (fp32)
    assert lib.lce_workspace_size(8192, 2560, 151936) == 2 * 8192 * 151936 + 8 * 8192 * 2560 * 4
    assert lib.lce_workspace_size(8, 100, 10) == 0

    def bwd(**kw):
        a = dict(h=A, rows=4, hd=128, hs=128, w=B, V=1000, ws=128, labels=A, ig=-100, T=1.0,
                 eps=0.0, mask=None, g=A, saved=A, lg=None, lgs=0, dh=A, dhs=128, dw=None,
                 dws=0, wk=A, wkb=1 << 30, status=None)
        a.update(kw)
        return lib.lce_backward(a["h"], a["rows"], a["hd"], a["hs"], a["w"], a["V"], a["ws"],
                                a["labels"], a["ig"], a["T"], a["eps"], a["mask"], a["g"],
                                a["saved"], a["lg"], a["lgs"], a["dh"], a["dhs"], a["dw"],
                                a["dws"], a["wk"], a["wkb"], a["status"], None)
    assert bwd(dhs=64) == E["STRIDE"]
    assert bwd(dw=B, dws=100) == E["STRIDE"]
    assert bwd(dh=None) == E["NULL"]
    assert bwd(g=None) == E["NULL"]
    assert bwd(saved=A + 4) == E["ALIGN"]
    assert bwd(wkb=16) == E["WORKSPACE"]
    assert bwd(lg=A, lgs=999) == E["STRIDE"]
    assert bwd(lg=A + 8, lgs=1000) == E["ALIGN"]
    W2 = 0x80000000
    assert bwd(lg=A + 1024, lgs=1000, wk=W2) == E["ALIAS"]    # overlaps dhidden
    assert bwd(lg=0x40000000, lgs=1000, dw=0x40000000 + 4096, dws=128, wk=W2) == E["ALIAS"]
    assert bwd(lg=0x40000000, lgs=1000, wk=0x40000000 + 15984) == E["ALIAS"]
    assert bwd(lg=0x40000000, lgs=1000, wk=W2, wkb=16) == E["WORKSPACE"]   # clear of all
    assert bwd(rows=0) == E["OK"]


def test_jsd_validation(lib):
    """Every argument error of the JSD entry points is returned before any
    launch (host-side only; the pointers are never dereferenced)."""
    def fwd(**kw):
        a = dict(s=A, t=B, rows=4, V=1000, ss=1000, ts=1000, dtype=0, labels=None, ig=-100,
                 T=1.0, beta=0.5, mask=None, loss=A, saved=A, status=None)
        a.update(kw)
        return lib.jsd_forward(a["s"], a["t"], a["rows"], a["V"], a["ss"], a["ts"], a["dtype"],
                               a["labels"], a["ig"], a["T"], a["beta"], a["mask"], a["loss"],
                               a["saved"], a["status"], None)
    assert fwd(beta=-0.1) == E["BETA"]
    assert fwd(beta=1.5) == E["BETA"]
    assert fwd(beta=float("nan")) == E["BETA"]
    assert fwd(T=0.0) == E["TEMP"]
    assert fwd(dtype=3) == E["DTYPE"]
    assert fwd(V=0) == E["SHAPE"]
    assert fwd(ss=999) == E["STRIDE"]
    assert fwd(ts=999) == E["STRIDE"]
    assert fwd(t=None) == E["NULL"]
    assert fwd(loss=None) == E["NULL"]
    assert fwd(saved=None) == E["NULL"]
    assert fwd(s=A + 2) == E["ALIGN"]                  # element alignment
    assert fwd(t=B + 2) == E["ALIGN"]
    assert fwd(dtype=1, t=B + 1) == E["ALIGN"]
    assert fwd(saved=A + 8) == E["ALIGN"]
    assert fwd(rows=0, s=None, t=None) == E["OK"]
    for beta in (0.0, 1.0):
        assert fwd(beta=beta, t=None) == E["NULL"]     # the ends of [0, 1] are accepted

    def bwd(**kw):
        a = dict(s=A, t=B, rows=4, V=1000, ss=1000, ts=1000, dtype=0, labels=None, ig=-100,
                 T=1.0, beta=0.5, mask=None, g=A, saved=A, d=A + (1 << 24), ds=1000, status=None)
        a.update(kw)
        return lib.jsd_backward(a["s"], a["t"], a["rows"], a["V"], a["ss"], a["ts"], a["dtype"],
                                a["labels"], a["ig"], a["T"], a["beta"], a["mask"], a["g"],
                                a["saved"], a["d"], a["ds"], a["status"], None)
    assert bwd(beta=2.0) == E["BETA"]
    assert bwd(ds=999) == E["STRIDE"]
    assert bwd(g=None) == E["NULL"]
    assert bwd(d=None) == E["NULL"]
    assert bwd(d=A + (1 << 24) + 2) == E["ALIGN"]
    assert bwd(d=A + 64) == E["ALIAS"]                  # overlaps the student
    assert bwd(d=B + 64) == E["ALIAS"]                  # overlaps the teacher
    assert bwd(rows=0) == E["OK"]
