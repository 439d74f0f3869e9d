"""Host <-> device plumbing for the GPU tests: numpy workloads in, numpy
outputs of the HIP path out.  Every computation goes through the C ABI via
cross_entropy_vocab_amd; nothing here computes a log-softmax."""
from __future__ import annotations

import sys

import numpy as np
import torch

import cross_entropy_vocab_amd as cev
from workloads import bf16_to_f32

DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return bf16_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy()


def strided_dev(a: np.ndarray, stride: int) -> torch.Tensor:
    """Device logits with a padded row stride (columns past V hold NaN/garbage
    canaries that must never influence a result)."""
    rows, V = a.shape
    if a.dtype == np.uint16:
        pad = np.full((rows, stride), 0x7FC1, dtype=np.uint16)  # bf16 NaN
        pad[:, :V] = a
        return to_dev(pad)[:, :V]
    pad = np.full((rows, stride), np.nan, dtype=np.float32)
    pad[:, :V] = a
    return to_dev(pad)[:, :V]


def run_ce(w, entropy=True, argmax=True, logits_dev=None, label_smoothing=0.0):
    """ce_forward + ce_backward on a workload dict; returns numpy outputs."""
    logits = logits_dev if logits_dev is not None else to_dev(w["logits"])
    labels = to_dev(w["labels"])
    mask = None if w.get("row_mask") is None else to_dev(w["row_mask"])
    g = to_dev(np.asarray(w["g"], dtype=np.float32))
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    T = w["temperature"]
    out = cev.ce_forward(logits, labels, T, row_mask=mask, entropy=entropy, argmax=argmax,
                         status=status, label_smoothing=label_smoothing)
    dl = cev.ce_backward(logits, labels, g, out["saved"], T, row_mask=mask, status=status,
                         label_smoothing=label_smoothing)
    torch.cuda.synchronize()
    res = {k: (None if v is None else to_host(v)) for k, v in out.items() if k != "workspace"}
    res["dlogits"] = to_host(dl)
    res["status"] = int(status.item())
    return res


def run_sls(w, entropy=True, argmax=True):
    logits = to_dev(w["logits"])
    labels = to_dev(w["labels"])
    mask = None if w.get("row_mask") is None else to_dev(w["row_mask"])
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = cev.sls_forward(logits, labels, w["temperature"], row_mask=mask, entropy=entropy,
                          argmax=argmax, status=status)
    torch.cuda.synchronize()
    res = {k: (None if v is None else to_host(v)) for k, v in out.items()}
    res["status"] = int(status.item())
    return res


def run_topk(w, indices=None):
    logits = to_dev(w["logits"])
    idx = to_dev(w["indices"] if indices is None else indices)
    mask = None if w.get("row_mask") is None else to_dev(w["row_mask"])
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    lp = cev.sls_topk_forward(logits, idx, w["temperature"], row_mask=mask, status=status)
    torch.cuda.synchronize()
    return to_host(lp), int(status.item())


def run_topk_fb(w, indices, g, logits_dev=None, dl_stride=None):
    """sls_topk_forward (with q and the saved record) then sls_topk_backward;
    returns numpy logp, q, dlogits and the status word."""
    logits = logits_dev if logits_dev is not None else to_dev(w["logits"])
    idx = to_dev(np.ascontiguousarray(indices))
    mask = None if w.get("row_mask") is None else to_dev(w["row_mask"])
    gk = to_dev(np.ascontiguousarray(g, dtype=np.float32))
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    T = w["temperature"]
    lp, q, saved = cev.sls_topk_forward(logits, idx, T, row_mask=mask, status=status, saved=True)
    R, V = logits.shape
    dl = None
    if dl_stride is not None:
        dl = torch.zeros((R, dl_stride), dtype=logits.dtype, device=DEV)[:, :V]
    dl = cev.sls_topk_backward(logits, idx, gk, saved, q, T, row_mask=mask, dlogits=dl,
                               status=status)
    torch.cuda.synchronize()
    return dict(logp=to_host(lp), q=to_host(q), dlogits=to_host(dl), status=int(status.item()))
