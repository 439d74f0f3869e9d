"""cross_entropy_vocab_amd -- collapse-safe selective log-softmax and
cross-entropy over a [rows, vocab] logit matrix on AMD MI355X (gfx950).

Thin binding over libcevocab.so (see include/cevocab.h).  The functions below
check tensor metadata, allocate outputs with PyTorch when the caller does not
pass them, and hand device pointers plus the current HIP stream to the C ABI.
Every step of the computation runs in the library's HIP kernels; PyTorch is
used for device memory and streams only.

    out = ce_forward(logits, labels, temperature=1.0, row_mask=mask)
    dlogits = ce_backward(logits, labels, g, out["saved"], temperature=1.0, row_mask=mask)
"""
from __future__ import annotations

import torch

from . import _lib

__all__ = ["sls_forward", "sls_topk_forward", "sls_topk_backward", "ce_forward",
           "ce_forward_noalloc", "noalloc_scratch_bytes", "ce_backward", "ce_fused", "ce_vocab_shard_forward", "ce_vocab_merge",
           "ce_vocab_shard_backward", "lce_forward", "lce_backward", "lce_workspace_size",
           "jsd_forward", "jsd_backward", "workspace_size", "JSD_SAVED_BYTES",
           "status_string", "version", "CEV_F32", "CEV_BF16", "STATUS_BAD_LABEL",
           "STATUS_BAD_INDEX", "STATUS_BAD_PARTS", "SAVED_BYTES", "PARTIAL_BYTES", "CevError"]

CEV_F32 = 0
CEV_BF16 = 1
STATUS_BAD_LABEL = 1
STATUS_BAD_INDEX = 2
STATUS_BAD_PARTS = 4
SAVED_BYTES = 16
JSD_SAVED_BYTES = 48
PARTIAL_BYTES = 48
PART_ENTROPY = 1
PART_VALUE_SUM = 2


class CevError(RuntimeError):
    """A non-zero return code from libcevocab.so."""

    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn}: {status_string(code)} (code {code})")


def status_string(code: int) -> str:
    return _lib.get().cev_status_string(int(code)).decode()


def version() -> int:
    return int(_lib.get().cev_version())


def workspace_size(rows: int, vocab: int, dtype: int) -> int:
    return int(_lib.get().cev_workspace_size(int(rows), int(vocab), int(dtype)))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CEV_F32
    if t.dtype == torch.bfloat16:
        return CEV_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _check_logits(logits: torch.Tensor):
    if not logits.is_cuda:
        raise ValueError("logits must be a GPU tensor")
    if logits.dim() != 2:
        raise ValueError("logits must be 2-D [rows, vocab] (flatten leading dimensions)")
    if logits.shape[0] > 0 and logits.shape[1] > 1 and logits.stride(1) != 1:
        raise ValueError("logits must have unit column stride")
    rows, vocab = logits.shape
    stride = logits.stride(0) if rows > 1 else max(vocab, logits.stride(0))
    return rows, vocab, max(stride, vocab)


def _dev(t, name, dtype, shape, device):
    if t is None:
        return None
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _mask(row_mask, rows, device):
    if row_mask is None:
        return None
    if row_mask.dtype == torch.bool:
        row_mask = row_mask.view(torch.uint8)
    return _dev(row_mask, "row_mask", torch.uint8, (rows,), device)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _check(fn, rc):
    if rc != 0:
        raise CevError(fn, rc)


def sls_forward(logits, labels, temperature=1.0, row_mask=None, ignore_index=-100,
                entropy=False, argmax=False, status=None):
    """log p at the label per row (fp32 [rows]), plus optional entropy and
    argmax.  Returns a dict with keys logp, entropy, argmax."""
    rows, vocab, stride = _check_logits(logits)
    dev = logits.device
    _dev(labels, "labels", torch.int64, (rows,), dev)
    m = _mask(row_mask, rows, dev)
    _dev(status, "status", torch.int32, (1,), dev)
    out = {
        "logp": torch.empty(rows, dtype=torch.float32, device=dev),
        "entropy": torch.empty(rows, dtype=torch.float32, device=dev) if entropy else None,
        "argmax": torch.empty(rows, dtype=torch.int64, device=dev) if argmax else None,
    }
    rc = _lib.get().sls_forward(_ptr(logits), rows, vocab, stride, _dtype_code(logits),
                                _ptr(labels), int(ignore_index), float(temperature), _ptr(m),
                                _ptr(out["logp"]), _ptr(out["entropy"]), _ptr(out["argmax"]),
                                _ptr(status), _stream(dev))
    _check("sls_forward", rc)
    return out


def _indices(indices, rows, dev):
    if indices.dim() != 2 or indices.shape[0] != rows or indices.dtype != torch.int64:
        raise ValueError("indices must be int64 [rows, K]")
    if not indices.is_cuda or indices.device != dev:
        raise ValueError(f"indices must be on {dev}")
    K = indices.shape[1]
    if rows > 1 and K > 1 and indices.stride(1) != 1:
        raise ValueError("indices must have unit column stride")
    istride = indices.stride(0) if rows > 1 else K
    return K, max(istride, K)


def sls_topk_forward(logits, indices, temperature=1.0, row_mask=None, ignore_index=-100,
                     status=None, saved=False):
    """log p at K gathered indices per row: fp32 [rows, K].  With saved=True
    returns (logp, q, saved): q = 1 - p at each index [rows, K] and the per-row
    record [rows, 16] that sls_topk_backward takes."""
    rows, vocab, stride = _check_logits(logits)
    dev = logits.device
    K, istride = _indices(indices, rows, dev)
    m = _mask(row_mask, rows, dev)
    _dev(status, "status", torch.int32, (1,), dev)
    logp = torch.empty((rows, K), dtype=torch.float32, device=dev)
    q = torch.empty((rows, K), dtype=torch.float32, device=dev) if saved else None
    sv = torch.empty((rows, SAVED_BYTES), dtype=torch.uint8, device=dev) if saved else None
    rc = _lib.get().sls_topk_forward(_ptr(logits), rows, vocab, stride, _dtype_code(logits),
                                     _ptr(indices), K, istride, int(ignore_index),
                                     float(temperature), _ptr(m), _ptr(logp), _ptr(q), _ptr(sv),
                                     _ptr(status), _stream(dev))
    _check("sls_topk_forward", rc)
    return (logp, q, sv) if saved else logp


def sls_topk_backward(logits, indices, g, saved, q, temperature=1.0, row_mask=None,
                      ignore_index=-100, dlogits=None, status=None):
    """Gradient of sum_k g[r, k] logp[r, k] with respect to logits, in the
    logits dtype; `saved` and `q` come from sls_topk_forward(saved=True)."""
    rows, vocab, stride = _check_logits(logits)
    dev = logits.device
    K, istride = _indices(indices, rows, dev)
    _dev(g, "g", torch.float32, (rows, K), dev)
    _dev(q, "q", torch.float32, (rows, K), dev)
    _dev(saved, "saved", torch.uint8, (rows, SAVED_BYTES), dev)
    m = _mask(row_mask, rows, dev)
    _dev(status, "status", torch.int32, (1,), dev)
    dlogits, dstride = _dlogits(dlogits, logits, rows, vocab, dev)
    rc = _lib.get().sls_topk_backward(_ptr(logits), rows, vocab, stride, _dtype_code(logits),
                                      _ptr(indices), K, istride, int(ignore_index),
                                      float(temperature), _ptr(m), _ptr(g), _ptr(saved), _ptr(q),
                                      _ptr(dlogits), dstride, _ptr(status), _stream(dev))
    _check("sls_topk_backward", rc)
    return dlogits


def _dlogits(dlogits, logits, rows, vocab, dev):
    if dlogits is None:
        dlogits = torch.empty((rows, vocab), dtype=logits.dtype, device=dev)
    else:
        if dlogits.dtype != logits.dtype or tuple(dlogits.shape) != (rows, vocab):
            raise ValueError("dlogits must match logits in dtype and shape")
        if not dlogits.is_cuda or dlogits.device != dev:
            raise ValueError(f"dlogits must be on {dev}")
        if rows > 0 and vocab > 1 and dlogits.stride(1) != 1:
            raise ValueError("dlogits must have unit column stride")
    return dlogits, max(dlogits.stride(0) if rows > 1 else vocab, vocab)


def ce_forward(logits, labels, temperature=1.0, row_mask=None, ignore_index=-100, logp=True,
               entropy=False, argmax=False, valid_rows=True, status=None, out=None,
               label_smoothing=0.0):
    """Per-row cross-entropy forward with device-side compaction of the valid
    rows.  Returns a dict: loss [rows] fp32, saved [rows, 16] uint8 (for
    ce_backward), and optionally logp, entropy, argmax, valid_rows [rows] int64
    (first n_valid entries meaningful) and n_valid [1] int64.

    `out` may hold preallocated tensors under the same keys (plus "workspace")
    so that repeated calls allocate nothing."""
    rows, vocab, stride = _check_logits(logits)
    dev = logits.device
    _dev(labels, "labels", torch.int64, (rows,), dev)
    m = _mask(row_mask, rows, dev)
    _dev(status, "status", torch.int32, (1,), dev)
    o = dict(out) if out else {}

    def want(key, flag, dtype, shape):
        if not flag:
            o[key] = None
        elif o.get(key) is None:
            o[key] = torch.empty(shape, dtype=dtype, device=dev)
        else:
            _dev(o[key], key, dtype, shape, dev)

    want("loss", True, torch.float32, (rows,))
    want("saved", True, torch.uint8, (rows, SAVED_BYTES))
    want("logp", logp, torch.float32, (rows,))
    want("entropy", entropy, torch.float32, (rows,))
    want("argmax", argmax, torch.int64, (rows,))
    want("valid_rows", valid_rows, torch.int64, (rows,))
    want("n_valid", valid_rows, torch.int64, (1,))
    ws_bytes = workspace_size(rows, vocab, _dtype_code(logits))
    ws = o.get("workspace")
    if ws is None or ws.numel() < ws_bytes:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    o["workspace"] = ws
    rc = _lib.get().ce_forward(_ptr(logits), rows, vocab, stride, _dtype_code(logits),
                               _ptr(labels), int(ignore_index), float(temperature),
                               float(label_smoothing), _ptr(m),
                               _ptr(o["loss"]), _ptr(o["saved"]), _ptr(o["logp"]),
                               _ptr(o["entropy"]), _ptr(o["argmax"]), _ptr(o["valid_rows"]),
                               _ptr(o["n_valid"]), _ptr(ws), ws_bytes, _ptr(status),
                               _stream(dev))
    _check("ce_forward", rc)
    return o


def noalloc_scratch_bytes() -> int:
    return int(_lib.get().cev_noalloc_scratch_bytes())


def ce_forward_noalloc(logits, labels, temperature=1.0, row_mask=None, ignore_index=-100,
                       status=None, label_smoothing=0.0, *, loss, saved, logp=None, entropy=None,
                       argmax=None, valid_rows=None, n_valid=None):
    """ce_forward into caller-provided outputs, with the library's static
    per-GPU scratch in place of a workspace: no device memory is allocated
    here or in the library.  Outputs as in ce_forward (loss and saved
    required, the others optional); calls that overlap on one GPU race."""
    rows, vocab, stride = _check_logits(logits)
    dev = logits.device
    _dev(labels, "labels", torch.int64, (rows,), dev)
    m = _mask(row_mask, rows, dev)
    _dev(status, "status", torch.int32, (1,), dev)
    _dev(loss, "loss", torch.float32, (rows,), dev)
    _dev(saved, "saved", torch.uint8, (rows, SAVED_BYTES), dev)
    for t, name, dt, shape in ((logp, "logp", torch.float32, (rows,)),
                               (entropy, "entropy", torch.float32, (rows,)),
                               (argmax, "argmax", torch.int64, (rows,)),
                               (valid_rows, "valid_rows", torch.int64, (rows,)),
                               (n_valid, "n_valid", torch.int64, (1,))):
        if t is not None:
            _dev(t, name, dt, shape, dev)
    rc = _lib.get().ce_forward_noalloc(_ptr(logits), rows, vocab, stride, _dtype_code(logits),
                                       _ptr(labels), int(ignore_index), float(temperature),
                                       float(label_smoothing), _ptr(m), _ptr(loss), _ptr(saved),
                                       _ptr(logp), _ptr(entropy), _ptr(argmax), _ptr(valid_rows),
                                       _ptr(n_valid), _ptr(status), _stream(dev))
    _check("ce_forward_noalloc", rc)


def ce_backward(logits, labels, g, saved, temperature=1.0, row_mask=None, ignore_index=-100,
                dlogits=None, status=None, label_smoothing=0.0):
    """dlogits = (g/T)(softmax(logits/T) - onehot(labels)) per valid row (with
    label smoothing eps: minus (g/T) eps (1/V - onehot)), zero rows elsewhere,
    in the logits dtype."""
    rows, vocab, stride = _check_logits(logits)
    dev = logits.device
    _dev(labels, "labels", torch.int64, (rows,), dev)
    _dev(g, "g", torch.float32, (rows,), dev)
    _dev(saved, "saved", torch.uint8, (rows, SAVED_BYTES), dev)
    m = _mask(row_mask, rows, dev)
    _dev(status, "status", torch.int32, (1,), dev)
    dlogits, dstride = _dlogits(dlogits, logits, rows, vocab, dev)
    rc = _lib.get().ce_backward(_ptr(logits), rows, vocab, stride, _dtype_code(logits),
                                _ptr(labels), int(ignore_index), float(temperature),
                                float(label_smoothing), _ptr(m),
                                _ptr(g), _ptr(saved), _ptr(dlogits), dstride, _ptr(status),
                                _stream(dev))
    _check("ce_backward", rc)
    return dlogits


def ce_fused(logits, labels, g, temperature=1.0, row_mask=None, ignore_index=-100, logp=True,
             entropy=False, argmax=False, valid_rows=False, dlogits=None, status=None, out=None,
             label_smoothing=0.0):
    """ce_forward and ce_backward in one call for a g known up front (part of
    each row held on chip between the sweep and the gradient pass, the rest
    read again).  Returns the ce_forward dict plus "dlogits"."""
    rows, vocab, stride = _check_logits(logits)
    dev = logits.device
    _dev(labels, "labels", torch.int64, (rows,), dev)
    _dev(g, "g", torch.float32, (rows,), dev)
    m = _mask(row_mask, rows, dev)
    _dev(status, "status", torch.int32, (1,), dev)
    o = dict(out) if out else {}

    def want(key, flag, dtype, shape):
        if not flag:
            o[key] = None
        elif o.get(key) is None:
            o[key] = torch.empty(shape, dtype=dtype, device=dev)
        else:
            _dev(o[key], key, dtype, shape, dev)

    want("loss", True, torch.float32, (rows,))
    want("saved", True, torch.uint8, (rows, SAVED_BYTES))
    want("logp", logp, torch.float32, (rows,))
    want("entropy", entropy, torch.float32, (rows,))
    want("argmax", argmax, torch.int64, (rows,))
    want("valid_rows", valid_rows, torch.int64, (rows,))
    want("n_valid", valid_rows, torch.int64, (1,))
    if dlogits is None:
        dlogits = o.get("dlogits")
    dlogits, dstride = _dlogits(dlogits, logits, rows, vocab, dev)
    o["dlogits"] = dlogits
    ws_bytes = workspace_size(rows, vocab, _dtype_code(logits))
    ws = o.get("workspace")
    if ws is None or ws.numel() < ws_bytes:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    o["workspace"] = ws
    rc = _lib.get().ce_fused(_ptr(logits), rows, vocab, stride, _dtype_code(logits),
                             _ptr(labels), int(ignore_index), float(temperature),
                             float(label_smoothing), _ptr(m), _ptr(g),
                             _ptr(o["loss"]), _ptr(o["saved"]), _ptr(o["logp"]),
                             _ptr(o["entropy"]), _ptr(o["argmax"]), _ptr(dlogits), dstride,
                             _ptr(o["valid_rows"]), _ptr(o["n_valid"]), _ptr(ws), ws_bytes,
                             _ptr(status), _stream(dev))
    _check("ce_fused", rc)
    return o


def ce_vocab_shard_forward(logits, labels, col_offset, vocab, temperature=1.0, row_mask=None,
                           ignore_index=-100, entropy=False, value_sum=False, partials=None,
                           status=None):
    """Partial records [rows, 48] uint8 of one vocab shard: `logits` holds
    global columns [col_offset, col_offset + logits.shape[1]) of each row."""
    rows, sv, stride = _check_logits(logits)
    dev = logits.device
    _dev(labels, "labels", torch.int64, (rows,), dev)
    m = _mask(row_mask, rows, dev)
    _dev(status, "status", torch.int32, (1,), dev)
    if partials is None:
        partials = torch.empty((rows, PARTIAL_BYTES), dtype=torch.uint8, device=dev)
    else:
        _dev(partials, "partials", torch.uint8, (rows, PARTIAL_BYTES), dev)
    what = (PART_ENTROPY if entropy else 0) | (PART_VALUE_SUM if value_sum else 0)
    rc = _lib.get().ce_vocab_shard_forward(_ptr(logits), rows, sv, stride, _dtype_code(logits),
                                           int(col_offset), int(vocab), _ptr(labels),
                                           int(ignore_index), float(temperature), _ptr(m), what,
                                           _ptr(partials), _ptr(status), _stream(dev))
    _check("ce_vocab_shard_forward", rc)
    return partials


def ce_vocab_merge(partials, labels, vocab, temperature=1.0, row_mask=None, ignore_index=-100,
                   label_smoothing=0.0, logp=True, entropy=False, argmax=False, status=None):
    """Merge [parts, rows, 48] partial records (shard order = ascending column
    ranges) into the ce_forward outputs of the whole rows: a dict with loss,
    saved and optionally logp, entropy, argmax."""
    if partials.dim() != 3 or partials.shape[2] != PARTIAL_BYTES:
        raise ValueError("partials must be [parts, rows, 48] uint8")
    parts, rows = partials.shape[0], partials.shape[1]
    dev = partials.device
    _dev(partials, "partials", torch.uint8, (parts, rows, PARTIAL_BYTES), dev)
    _dev(labels, "labels", torch.int64, (rows,), dev)
    m = _mask(row_mask, rows, dev)
    _dev(status, "status", torch.int32, (1,), dev)
    o = {
        "loss": torch.empty(rows, dtype=torch.float32, device=dev),
        "saved": torch.empty((rows, SAVED_BYTES), dtype=torch.uint8, device=dev),
        "logp": torch.empty(rows, dtype=torch.float32, device=dev) if logp else None,
        "entropy": torch.empty(rows, dtype=torch.float32, device=dev) if entropy else None,
        "argmax": torch.empty(rows, dtype=torch.int64, device=dev) if argmax else None,
    }
    rc = _lib.get().ce_vocab_merge(_ptr(partials), parts, rows, int(vocab), _ptr(labels),
                                   int(ignore_index), float(temperature), float(label_smoothing),
                                   _ptr(m), _ptr(o["loss"]), _ptr(o["saved"]), _ptr(o["logp"]),
                                   _ptr(o["entropy"]), _ptr(o["argmax"]), _ptr(status),
                                   _stream(dev))
    _check("ce_vocab_merge", rc)
    return o


def ce_vocab_shard_backward(logits, labels, g, saved, col_offset, vocab, temperature=1.0,
                            row_mask=None, ignore_index=-100, label_smoothing=0.0, dlogits=None,
                            status=None):
    """ce_backward over one vocab shard's columns, from the merged record."""
    rows, sv, stride = _check_logits(logits)
    dev = logits.device
    _dev(labels, "labels", torch.int64, (rows,), dev)
    _dev(g, "g", torch.float32, (rows,), dev)
    _dev(saved, "saved", torch.uint8, (rows, SAVED_BYTES), dev)
    m = _mask(row_mask, rows, dev)
    _dev(status, "status", torch.int32, (1,), dev)
    dlogits, dstride = _dlogits(dlogits, logits, rows, sv, dev)
    rc = _lib.get().ce_vocab_shard_backward(_ptr(logits), rows, sv, stride, _dtype_code(logits),
                                            int(col_offset), int(vocab), _ptr(labels),
                                            int(ignore_index), float(temperature),
                                            float(label_smoothing), _ptr(m), _ptr(g),
                                            _ptr(saved), _ptr(dlogits), dstride, _ptr(status),
                                            _stream(dev))
    _check("ce_vocab_shard_backward", rc)
    return dlogits


def _jsd_pair(student, teacher):
    rows, vocab, sstride = _check_logits(student)
    if teacher.dtype != student.dtype or tuple(teacher.shape) != (rows, vocab):
        raise ValueError("teacher must match student in dtype and shape")
    if teacher.device != student.device:
        raise ValueError("teacher must be on the student's device")
    _, _, tstride = _check_logits(teacher)
    return rows, vocab, sstride, tstride


def jsd_forward(student, teacher, temperature=1.0, beta=0.5, labels=None, row_mask=None,
                ignore_index=-100, status=None, out=None):
    """Generalized JSD per row between softmax(student / T) and
    softmax(teacher / T) (beta = 0: KL(teacher || student), beta = 1:
    KL(student || teacher)).  Returns a dict: loss [rows] fp32 and saved
    [rows, 48] uint8 (for jsd_backward)."""
    rows, vocab, ss, ts = _jsd_pair(student, teacher)
    dev = student.device
    _dev(labels, "labels", torch.int64, (rows,), dev)
    m = _mask(row_mask, rows, dev)
    _dev(status, "status", torch.int32, (1,), dev)
    o = dict(out) if out else {}
    if o.get("loss") is None:
        o["loss"] = torch.empty(rows, dtype=torch.float32, device=dev)
    if o.get("saved") is None:
        o["saved"] = torch.empty((rows, JSD_SAVED_BYTES), dtype=torch.uint8, device=dev)
    _dev(o["loss"], "loss", torch.float32, (rows,), dev)
    _dev(o["saved"], "saved", torch.uint8, (rows, JSD_SAVED_BYTES), dev)
    rc = _lib.get().jsd_forward(_ptr(student), _ptr(teacher), rows, vocab, ss, ts,
                                _dtype_code(student), _ptr(labels), int(ignore_index),
                                float(temperature), float(beta), _ptr(m), _ptr(o["loss"]),
                                _ptr(o["saved"]), _ptr(status), _stream(dev))
    _check("jsd_forward", rc)
    return o


def jsd_backward(student, teacher, g, saved, temperature=1.0, beta=0.5, labels=None,
                 row_mask=None, ignore_index=-100, dstudent=None, status=None):
    """g[r] times the gradient of row r's jsd_forward loss with respect to the
    student logits (dtype and shape of student)."""
    rows, vocab, ss, ts = _jsd_pair(student, teacher)
    dev = student.device
    _dev(labels, "labels", torch.int64, (rows,), dev)
    _dev(g, "g", torch.float32, (rows,), dev)
    _dev(saved, "saved", torch.uint8, (rows, JSD_SAVED_BYTES), dev)
    m = _mask(row_mask, rows, dev)
    _dev(status, "status", torch.int32, (1,), dev)
    dstudent, dstride = _dlogits(dstudent, student, rows, vocab, dev)
    rc = _lib.get().jsd_backward(_ptr(student), _ptr(teacher), rows, vocab, ss, ts,
                                 _dtype_code(student), _ptr(labels), int(ignore_index),
                                 float(temperature), float(beta), _ptr(m), _ptr(g), _ptr(saved),
                                 _ptr(dstudent), dstride, _ptr(status), _stream(dev))
    _check("jsd_backward", rc)
    return dstudent


def lce_workspace_size(rows: int, hidden_dim: int, vocab: int) -> int:
    return int(_lib.get().lce_workspace_size(int(rows), int(hidden_dim), int(vocab)))


def _check_bf16_2d(t, name, dev=None):
    if not t.is_cuda or (dev is not None and t.device != dev):
        raise ValueError(f"{name} must be a GPU tensor on the same device")
    if t.dtype != torch.bfloat16 or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D bfloat16 tensor")
    if t.shape[0] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return max(t.stride(0) if t.shape[0] > 1 else t.shape[1], t.shape[1])


def _lce_workspace(o, rows, H, V, dev):
    need = lce_workspace_size(rows, H, V)
    ws = o.get("workspace")
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    return ws, need


def _lce_logits(logits, rows, V, dev, allocate):
    """(tensor, row stride) of a stored-logits buffer: None, True (allocate
    [rows, V] fp32, rows padded to 16 bytes) or an fp32 [rows, V] view with
    unit column stride, 16-byte aligned rows and a row stride a multiple of 4."""
    if logits is None or logits is False:
        return None, 0
    if logits is True:
        if not allocate:
            raise ValueError("logits must be the tensor lce_forward stored them in")
        # rows padded to a multiple of 4 floats (16-byte aligned rows)
        logits = torch.empty((rows, V + (-V) % 4), dtype=torch.float32, device=dev)[:, :V]
    if not logits.is_cuda or logits.device != dev or logits.dtype != torch.float32 \
            or tuple(logits.shape) != (rows, V) or (V > 1 and logits.stride(1) != 1):
        raise ValueError("logits must be a float32 [rows, vocab] GPU tensor on the same device")
    stride = logits.stride(0) if rows > 1 else V + (-V) % 4
    return logits, stride


def lce_forward(hidden, weight, labels, temperature=1.0, row_mask=None, ignore_index=-100,
                label_smoothing=0.0, logp=True, entropy=False, argmax=False, status=None,
                out=None, logits=None):
    """Linear cross-entropy forward: logits = hidden x weight^T (bf16 in, fp32
    accumulate), then the collapse-safe per-row CE.  The logits are never
    stored unless `logits` is True (a new fp32 [rows, vocab] tensor) or such a
    tensor: then lce_backward can read them back instead of recomputing them.
    Returns a dict with loss, saved (for lce_backward) and optionally logp,
    entropy, argmax, logits, plus the workspace it used."""
    rows, H = hidden.shape
    dev = hidden.device
    hs = _check_bf16_2d(hidden, "hidden")
    ws_ = _check_bf16_2d(weight, "weight", dev)
    V = weight.shape[0]
    if weight.shape[1] != H:
        raise ValueError("weight must be [vocab, hidden_dim]")
    _dev(labels, "labels", torch.int64, (rows,), dev)
    m = _mask(row_mask, rows, dev)
    _dev(status, "status", torch.int32, (1,), dev)
    o = dict(out) if out else {}

    def want(key, flag, dtype, shape):
        if not flag:
            o[key] = None
        elif o.get(key) is None:
            o[key] = torch.empty(shape, dtype=dtype, device=dev)
        else:
            _dev(o[key], key, dtype, shape, dev)

    want("loss", True, torch.float32, (rows,))
    want("saved", True, torch.uint8, (rows, SAVED_BYTES))
    want("logp", logp, torch.float32, (rows,))
    want("entropy", entropy, torch.float32, (rows,))
    want("argmax", argmax, torch.int64, (rows,))
    ws, need = _lce_workspace(o, rows, H, V, dev)
    o["workspace"] = ws
    lg, ldl = _lce_logits(logits, rows, V, dev, allocate=True)
    o["logits"] = lg
    rc = _lib.get().lce_forward(_ptr(hidden), rows, H, hs, _ptr(weight), V, ws_, _ptr(labels),
                                int(ignore_index), float(temperature), float(label_smoothing),
                                _ptr(m), _ptr(o["loss"]), _ptr(o["saved"]), _ptr(o["logp"]),
                                _ptr(o["entropy"]), _ptr(o["argmax"]), _ptr(lg), ldl, _ptr(ws),
                                need, _ptr(status), _stream(dev))
    _check("lce_forward", rc)
    return o


def lce_backward(hidden, weight, labels, g, saved, temperature=1.0, row_mask=None,
                 ignore_index=-100, label_smoothing=0.0, dweight=False, status=None,
                 workspace=None, dhidden=None, logits=None):
    """Gradients of sum_r g[r] loss[r] through logits = hidden x weight^T:
    dhidden [rows, hidden_dim] fp32, and dweight [vocab, hidden_dim] fp32 when
    dweight is True or such a tensor to fill (else None, a frozen head).  `logits`: the tensor lce_forward
    stored the logits in, read instead of recomputing them."""
    rows, H = hidden.shape
    dev = hidden.device
    hs = _check_bf16_2d(hidden, "hidden")
    ws_ = _check_bf16_2d(weight, "weight", dev)
    V = weight.shape[0]
    _dev(labels, "labels", torch.int64, (rows,), dev)
    _dev(g, "g", torch.float32, (rows,), dev)
    _dev(saved, "saved", torch.uint8, (rows, SAVED_BYTES), dev)
    m = _mask(row_mask, rows, dev)
    _dev(status, "status", torch.int32, (1,), dev)
    ws, need = _lce_workspace({"workspace": workspace}, rows, H, V, dev)
    if dhidden is None:
        dhidden = torch.empty((rows, H), dtype=torch.float32, device=dev)
    else:
        _dev(dhidden, "dhidden", torch.float32, (rows, H), dev)
    if isinstance(dweight, torch.Tensor):
        _dev(dweight, "dweight", torch.float32, (V, H), dev)
        dw = dweight
    else:
        dw = torch.empty((V, H), dtype=torch.float32, device=dev) if dweight else None
    lg, ldl = _lce_logits(logits, rows, V, dev, allocate=False)
    rc = _lib.get().lce_backward(_ptr(hidden), rows, H, hs, _ptr(weight), V, ws_, _ptr(labels),
                                 int(ignore_index), float(temperature), float(label_smoothing),
                                 _ptr(m), _ptr(g), _ptr(saved), _ptr(lg), ldl, _ptr(dhidden), H,
                                 _ptr(dw), H, _ptr(ws), need, _ptr(status), _stream(dev))
    _check("lce_backward", rc)
    return dhidden, dw
