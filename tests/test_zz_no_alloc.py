"""ce_forward_noalloc (the static-scratch variant of ce_forward) against
ce_forward with a caller workspace, both called through the C ABI: two calls
in a row on one GPU, the second with a smaller input, every output compared
bit for bit.  The first call keeps its compacted list in the scratch (no
valid_rows / n_valid outputs); the second splits its few long rows over
several workgroups, whose partial records also live in the scratch, over the
first call's leftovers."""
import ctypes

import numpy as np
import pytest
import torch

import cross_entropy_vocab_amd as cev
from cross_entropy_vocab_amd import _lib
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
CEV_ESCRATCH = -12


def _dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _p(t):
    return None if t is None else t.data_ptr()


def _outputs(rows, lists):
    o = {"loss": torch.full((rows,), np.nan, dtype=torch.float32, device=DEV),
         "saved": torch.full((rows, 16), 0xAB, dtype=torch.uint8, device=DEV),
         "logp": torch.full((rows,), np.nan, dtype=torch.float32, device=DEV),
         "entropy": torch.full((rows,), np.nan, dtype=torch.float32, device=DEV),
         "argmax": torch.full((rows,), -7, dtype=torch.int64, device=DEV),
         "status": torch.zeros(1, dtype=torch.int32, device=DEV)}
    if lists:
        o["valid_rows"] = torch.full((rows,), -7, dtype=torch.int64, device=DEV)
        o["n_valid"] = torch.full((1,), -7, dtype=torch.int64, device=DEV)
    else:
        o["valid_rows"] = o["n_valid"] = None
    return o


def _call(noalloc, w, lists, T):
    lib = _lib.get()
    z = _dev(w["logits"])
    rows, vocab = z.shape
    dt = cev.CEV_BF16 if w["logits"].dtype == np.uint16 else cev.CEV_F32
    lab = _dev(w["labels"])
    mask = None if w.get("row_mask") is None else _dev(w["row_mask"])
    o = _outputs(rows, lists)
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    common = (_p(z), rows, vocab, vocab, dt, _p(lab), -100, T, 0.0, _p(mask), _p(o["loss"]),
              _p(o["saved"]), _p(o["logp"]), _p(o["entropy"]), _p(o["argmax"]),
              _p(o["valid_rows"]), _p(o["n_valid"]))
    if noalloc:
        rc = lib.ce_forward_noalloc(*common, _p(o["status"]), stream)
    else:
        ws_bytes = lib.cev_workspace_size(rows, vocab, dt)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
        rc = lib.ce_forward(*common, _p(ws), ws_bytes, _p(o["status"]), stream)
    assert rc == 0, (noalloc, rc)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in o.items()}


def _same(a, b, what):
    for k in a:
        if a[k] is None:
            assert b[k] is None, (what, k)
            continue
        assert a[k].dtype == b[k].dtype and a[k].shape == b[k].shape, (what, k)
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), (what, k)


def test_noalloc_matches_ce_forward_twice_then_smaller():
    assert cev.noalloc_scratch_bytes() == 4 << 20
    # call 1: 1922 x 4096 fp32, 256 supervised rows, list and count in the scratch
    w1 = workloads.sparse()
    print("[noalloc] call 1: sparse 1922x4096 f32, list in the scratch", flush=True)
    a1 = _call(True, w1, False, 1.0)
    b1 = _call(False, w1, False, 1.0)
    _same(a1, b1, "sparse")
    assert np.count_nonzero(a1["saved"][:, 12] & 1) == 256
    # call 2, smaller: 8 x 152064 bf16 with a mask; each row split over several
    # workgroups whose partial records go to the scratch as well
    w2 = workloads.grpo(rows=8, vocab=152064)
    assert w2["logits"].size < w1["logits"].size
    print("[noalloc] call 2: grpo 8x152064 bf16, split rows", flush=True)
    a2 = _call(True, w2, False, 1.0)
    b2 = _call(False, w2, False, 1.0)
    _same(a2, b2, "split")
    # and with the list taken as outputs (the scratch then holds only partials)
    a3 = _call(True, w2, True, 0.7)
    b3 = _call(False, w2, True, 0.7)
    _same(a3, b3, "split with list outputs")
    n = int(a3["n_valid"][0])
    vr = np.flatnonzero((w2["labels"] != -100) & (w2["row_mask"] != 0))
    assert n == vr.size and np.array_equal(a3["valid_rows"][:n], vr)


def test_noalloc_rejects_inputs_beyond_the_scratch():
    lib = _lib.get()
    rows = (cev.noalloc_scratch_bytes() // 8)      # (rows + 1) * 8 bytes > the scratch
    z = torch.zeros((1, 8), dtype=torch.float32, device=DEV)   # never read: rejected first
    lab = torch.zeros(1, dtype=torch.int64, device=DEV)
    loss = torch.zeros(1, dtype=torch.float32, device=DEV)
    saved = torch.zeros((1, 16), dtype=torch.uint8, device=DEV)
    rc = lib.ce_forward_noalloc(_p(z), rows, 8, 8, cev.CEV_F32, _p(lab), -100, 1.0, 0.0, None,
                                _p(loss), _p(saved), None, None, None, None, None, None, None)
    assert rc == CEV_ESCRATCH
    assert "scratch" in cev.status_string(rc)
