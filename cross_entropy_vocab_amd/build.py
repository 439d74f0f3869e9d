"""Build libcevocab.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m cross_entropy_vocab_amd.build [--sanitize]

Objects go to cross_entropy_vocab_amd/_build/, the library next to this file.
--sanitize builds _build/libcevocab_san.so, the same library with its host code
(the C ABI's argument checks) under ASan and UBSan.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcevocab.so")
SOURCES = ["sweep.hip", "backward.hip", "compact.hip", "fused.hip", "shard.hip", "lce.hip", "jsd.hip",
           "noalloc.hip", "api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
        "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC,
        # packed fp32 VALU forms are kept out of generated code on purpose
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # leading scalar kernel arguments arrive in SGPRs at wave start (gfx950
        # kernel-argument preloading; kernels taking one struct are unaffected)
        "-mllvm", "-amdgpu-kernarg-preload-count=14",
    ]


# Host-side sanitizers for the C ABI's argument checks: ASan and UBSan on the
# host code of api.cpp and noalloc.hip only (each flag after -Xarch_host, so no
# device code is instrumented), linked with the regular device objects.
SANITIZED_SOURCES = ["api.cpp", "noalloc.hip"]
SAN_LIB = os.path.join(BUILD, "libcevocab_san.so")


def san_flags() -> list:
    out = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-g",
              "-fno-omit-frame-pointer"):
        out += ["-Xarch_host", f]
    return out


def build_sanitized(verbose: bool = False) -> str:
    """libcevocab_san.so: the library with its host code under ASan + UBSan
    (load it with the compiler's ASan runtime preloaded)."""
    if not all(os.path.exists(os.path.join(BUILD, os.path.splitext(s)[0] + ".o")) for s in SOURCES):
        build(verbose)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        base = os.path.splitext(src)[0]
        if src not in SANITIZED_SOURCES:
            objs.append(os.path.join(BUILD, base + ".o"))
            continue
        obj = os.path.join(BUILD, base + "_san.o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        r = subprocess.run([cc, *compile_flags(), *san_flags(), *lang, "-c", os.path.join(CSRC, src),
                            "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}{r.stderr}")
        objs.append(obj)
    link_san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-shared-libsan"):
        link_san += ["-Xarch_host", f]
    subprocess.check_call([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_san, "-o", SAN_LIB,
                           *objs])
    return SAN_LIB


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *compile_flags(), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for cmd, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the packed-fp32 feature name; harmless
        text = "\n".join(l for l in text.splitlines() if "not a recognized feature" not in l)
        if verbose and text.strip():
            print(text)
        if p.returncode != 0:
            failed.append((cmd, text))
    if failed:
        msg = "\n\n".join(" ".join(c) + "\n" + t for c, t in failed)
        raise RuntimeError("hipcc failed:\n" + msg)
    tmp = LIB + ".tmp"
    subprocess.check_call([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
