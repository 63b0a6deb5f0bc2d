"""The Python binding refuses tensors whose shape or dtype does not match what
q and k imply, before any pointer reaches the C ABI (which takes every size
from q and k alone). Host tensors are enough: the shape and dtype checks come
before the device checks, so every refusal here is the one under test."""
import pytest
import torch

import sliding_window_flash_amd as swa

T, HQ, HKV, D = 40, 4, 2, 64
KW = dict(max_seqlen_q=T, max_seqlen_k=T, window=16, causal=True)


def base(dtype=torch.bfloat16):
    q = torch.zeros((T, HQ, D), dtype=dtype)
    k = torch.zeros((T, HKV, D), dtype=dtype)
    v = torch.zeros_like(k)
    cu = torch.tensor([0, T], dtype=torch.int32)
    return dict(q=q, k=k, v=v, o=torch.zeros_like(q), lse=torch.zeros((HQ, T), dtype=torch.float32),
                do=torch.zeros_like(q), cu_q=cu, cu_k=cu.clone())


def call_fwd(x, **extra):
    return swa.fwd(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], **KW, **extra)


def call_bwd(x, **extra):
    return swa.bwd(x["q"], x["k"], x["v"], x["o"], x["lse"], x["do"], x["cu_q"], x["cu_k"], **KW, **extra)


@pytest.mark.parametrize("change,match", [
    (dict(cu_q=torch.tensor([0, T])), "cu_q has dtype torch.int64"),          # torch.tensor's default
    (dict(cu_k=torch.tensor([0, 10, T], dtype=torch.int32)), "batch \\+ 1"),
    (dict(v=torch.zeros((T - 1, HKV, D), dtype=torch.bfloat16)), "v has shape"),
    (dict(v=torch.zeros((T, HKV, D), dtype=torch.float32)), "v has dtype"),
    (dict(k=torch.zeros((T, HKV, 32), dtype=torch.bfloat16)), "head_dim"),
    (dict(k=torch.zeros((T, HKV, D), dtype=torch.float16)), "k has dtype"),
    (dict(q=torch.zeros((T, HQ * D), dtype=torch.bfloat16)), "q must be"),
])
def test_forward_refuses_mismatched_inputs(change, match):
    x = base()
    x.update(change)
    with pytest.raises(ValueError, match=match):
        call_fwd(x)


@pytest.mark.parametrize("which,bad,match", [
    ("out", torch.zeros((T - 8, HQ, D), dtype=torch.bfloat16), "o has shape"),
    ("out", torch.zeros((T, HQ, D), dtype=torch.float32), "o has dtype"),
    ("lse", torch.zeros((T, HQ), dtype=torch.float32), "lse has shape"),
    ("lse", torch.zeros((HQ, T), dtype=torch.bfloat16), "lse has dtype"),
    ("mask", torch.zeros((T - 1, 4), dtype=torch.int32), "mask must be"),
    ("mask", torch.zeros((T, 4), dtype=torch.int64), "mask must be"),
])
def test_forward_refuses_mismatched_outputs_and_mask(which, bad, match):
    with pytest.raises(ValueError, match=match):
        call_fwd(base(), **{which: bad})


@pytest.mark.parametrize("which,bad,match", [
    ("o", torch.zeros((T, HQ, D - 8), dtype=torch.bfloat16), "o has shape"),
    ("do", torch.zeros((T, HQ, D), dtype=torch.float32), "do has dtype"),
    ("lse", torch.zeros((HQ, T - 1), dtype=torch.float32), "lse has shape"),
])
def test_backward_refuses_mismatched_inputs(which, bad, match):
    x = base()
    x[which] = bad
    with pytest.raises(ValueError, match=match):
        call_bwd(x)


@pytest.mark.parametrize("which,bad,match", [
    ("dq", torch.zeros((T, HQ, D), dtype=torch.float16), "dq has dtype"),
    ("dk", torch.zeros((T, HQ, D), dtype=torch.bfloat16), "dk has shape"),
    ("dv", torch.zeros((T - 1, HKV, D), dtype=torch.bfloat16), "dv has shape"),
    ("mask", torch.zeros((T + 1, 4), dtype=torch.int32), "mask must be"),
    ("workspace", torch.zeros(8, dtype=torch.uint8), "workspace holds 8 bytes"),
])
def test_backward_refuses_mismatched_outputs(which, bad, match):
    with pytest.raises(ValueError, match=match):
        call_bwd(base(), **{which: bad})


def test_matching_host_tensors_reach_the_device_check():
    with pytest.raises(ValueError, match="contiguous device tensor"):
        call_fwd(base())
    with pytest.raises(ValueError, match="contiguous device tensor"):
        call_bwd(base())


N, V, HID = 16, 300, 256


def ce_base():
    return dict(h=torch.zeros((N, HID), dtype=torch.bfloat16), w=torch.zeros((V, HID), dtype=torch.bfloat16),
                targets=torch.zeros(N, dtype=torch.int32))


@pytest.mark.parametrize("change,match", [
    (dict(targets=torch.zeros(N, dtype=torch.int64)), "targets has dtype"),
    (dict(targets=torch.zeros(N - 1, dtype=torch.int32)), "targets has shape"),
    (dict(w=torch.zeros((V, HID + 256), dtype=torch.bfloat16)), "h must be"),
])
def test_ce_refuses_mismatched_inputs(change, match):
    x = ce_base()
    x.update(change)
    with pytest.raises(ValueError, match=match):
        swa.ce_fwd(x["h"], x["w"], x["targets"])


def test_ce_refuses_mismatched_outputs():
    x = ce_base()
    with pytest.raises(ValueError, match="nll has dtype"):
        swa.ce_fwd(x["h"], x["w"], x["targets"], nll=torch.zeros(N, dtype=torch.float64))
    lse = torch.zeros(N, dtype=torch.float32)
    with pytest.raises(ValueError, match="dnll has shape"):
        swa.ce_bwd(x["h"], x["w"], x["targets"], lse, torch.zeros(N + 1, dtype=torch.float32))
    with pytest.raises(ValueError, match="dh has dtype"):
        swa.ce_bwd(x["h"], x["w"], x["targets"], lse, lse.clone(), dh=torch.zeros((N, HID), dtype=torch.float16))
    with pytest.raises(ValueError, match="contiguous device tensor"):
        swa.ce_fwd(x["h"], x["w"], x["targets"])
