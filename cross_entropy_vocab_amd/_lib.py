"""ctypes view of libcevocab.so: symbol declarations only.

The library is built in-tree by ``python -m cross_entropy_vocab_amd.build``.
Every compute entry point of this package goes through it; there is no other
implementation to fall back on, so a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os

# CEV_LIBRARY names another build of the same library (the host-sanitized one).
LIB_PATH = os.environ.get("CEV_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                          "libcevocab.so")

P = ctypes.c_void_p
I64 = ctypes.c_int64
I32 = ctypes.c_int
D = ctypes.c_double
SZ = ctypes.c_size_t
U32 = ctypes.c_uint

# name -> (restype, argtypes), mirroring include/cevocab.h
SIGNATURES = {
    "sls_forward": (I32, [P, I64, I64, I64, I32, P, I64, D, P, P, P, P, P, P]),
    "sls_topk_forward": (I32, [P, I64, I64, I64, I32, P, I64, I64, I64, D, P, P, P, P, P, P]),
    "sls_topk_backward": (I32, [P, I64, I64, I64, I32, P, I64, I64, I64, D, P, P, P, P, P, I64,
                                P, P]),
    "ce_forward": (I32, [P, I64, I64, I64, I32, P, I64, D, D, P, P, P, P, P, P, P, P, P, SZ, P,
                         P]),
    "ce_forward_noalloc": (I32, [P, I64, I64, I64, I32, P, I64, D, D, P, P, P, P, P, P, P, P, P,
                                 P]),
    "cev_noalloc_scratch_bytes": (SZ, []),
    "ce_backward": (I32, [P, I64, I64, I64, I32, P, I64, D, D, P, P, P, P, I64, P, P]),
    "ce_fused": (I32, [P, I64, I64, I64, I32, P, I64, D, D, P, P, P, P, P, P, P, P, I64, P, P, P,
                       SZ, P, P]),
    "ce_vocab_shard_forward": (I32, [P, I64, I64, I64, I32, I64, I64, P, I64, D, P, U32, P, P,
                                     P]),
    "ce_vocab_merge": (I32, [P, I64, I64, I64, P, I64, D, D, P, P, P, P, P, P, P, P]),
    "ce_vocab_shard_backward": (I32, [P, I64, I64, I64, I32, I64, I64, P, I64, D, D, P, P, P, P,
                                      I64, P, P]),
    "lce_forward": (I32, [P, I64, I64, I64, P, I64, I64, P, I64, D, D, P, P, P, P, P, P, P, I64,
                          P, SZ, P, P]),
    "lce_backward": (I32, [P, I64, I64, I64, P, I64, I64, P, I64, D, D, P, P, P, P, I64, P, I64,
                           P, I64, P, SZ, P, P]),
    "lce_workspace_size": (SZ, [I64, I64, I64]),
    "jsd_forward": (I32, [P, P, I64, I64, I64, I64, I32, P, I64, D, D, P, P, P, P, P]),
    "jsd_backward": (I32, [P, P, I64, I64, I64, I64, I32, P, I64, D, D, P, P, P, P, I64, P, P]),
    "cev_workspace_size": (SZ, [I64, I64, I32]),
    "cev_status_string": (ctypes.c_char_p, [I32]),
    "cev_version": (I32, []),
}

_lib = None


class LibraryMissing(RuntimeError):
    pass


def get():
    """The loaded library; raises LibraryMissing if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(
            f"{LIB_PATH} is missing: build the HIP library with "
            "`python -m cross_entropy_vocab_amd.build` (there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
