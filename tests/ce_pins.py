"""Pins for the fp64 linear cross-entropy oracle (``oracle.ce``).

Each ``pin_*`` takes a module exposing ``ce_reference`` (the real oracle or a
copy with a planted mistake) and raises AssertionError on disagreement with:

  * torch's own cross-entropy on the materialised logits (CPU, fp64) and its
    autograd gradient into the hidden states (a library routine for the
    special case the oracle's definition reduces to),
  * central finite differences of the oracle's own loss (the backward formula),
  * the independent per-token brute-force loop (``oracle.loop.ce_loop``),
  * closed forms: a one-word vocabulary (loss 0, no gradient); a head whose
    rows are all equal (loss log V, no gradient),
  * invariants: adding one vector c to every head row leaves the loss and the
    gradient unchanged and shifts LSE and the target logit by h . c; max z <=
    LSE <= max z + log V; the gradient is linear in the upstream gradient.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import loop
from sliding_window_flash_amd.workloads import CEWorkload, make_ce_inputs


def _case(n, vocab, hidden, seed):
    return make_ce_inputs(CEWorkload(f"ce_pin_{seed}", n, vocab, hidden, "f32", seed))


def _close(a, b, tol, what):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = float(np.max(np.abs(a - b), initial=0.0))
    assert err <= tol, f"{what}: max abs error {err} > {tol}"


def pin_torch_cross_entropy(ref):
    import torch
    x = _case(9, 13, 5, 1)
    out = ref.ce_reference(x["h"], x["w"], x["targets"], x["dnll"])
    h = torch.tensor(x["h"], dtype=torch.float64, requires_grad=True)
    z = h @ torch.tensor(x["w"], dtype=torch.float64).T
    t = torch.tensor(x["targets"], dtype=torch.int64)
    nll = torch.nn.functional.cross_entropy(z, t, reduction="none")
    (nll * torch.tensor(x["dnll"], dtype=torch.float64)).sum().backward()
    _close(out["nll"], nll.detach().numpy(), 1e-12, "torch cross_entropy nll")
    _close(out["lse"], torch.logsumexp(z, 1).detach().numpy(), 1e-12, "torch logsumexp")
    _close(out["dh"], h.grad.numpy(), 1e-12, "torch autograd dH")


def pin_finite_differences(ref):
    x = _case(4, 6, 3, 2)
    out = ref.ce_reference(x["h"], x["w"], x["targets"], x["dnll"])
    h = np.array(x["h"], dtype=np.float64)
    g = np.asarray(x["dnll"], np.float64)
    num = np.zeros_like(h)
    step = 1e-5
    for idx in np.ndindex(h.shape):
        keep = h[idx]
        h[idx] = keep + step
        up = float(np.sum(g * ref.ce_reference(h, x["w"], x["targets"])["nll"]))
        h[idx] = keep - step
        dn = float(np.sum(g * ref.ce_reference(h, x["w"], x["targets"])["nll"]))
        h[idx] = keep
        num[idx] = (up - dn) / (2 * step)
    _close(out["dh"], num, 1e-8, "finite differences dH")


def pin_loop(ref):
    for n, (tok, vocab, hid, seed) in enumerate([(5, 7, 3, 3), (3, 11, 4, 4), (6, 2, 5, 5)]):
        x = _case(tok, vocab, hid, seed)
        a = ref.ce_reference(x["h"], x["w"], x["targets"], x["dnll"])
        b = loop.ce_loop(x["h"], x["w"], x["targets"], x["dnll"])
        for key in ("nll", "lse", "tgt", "dh"):
            _close(a[key], b[key], 1e-12, f"loop {key} case {n}")


def pin_one_word_vocabulary(ref):
    x = _case(5, 1, 4, 6)
    out = ref.ce_reference(x["h"], x["w"], x["targets"], x["dnll"])
    _close(out["nll"], np.zeros(5), 1e-14, "V = 1: nll = 0")
    _close(out["lse"], out["tgt"], 1e-14, "V = 1: lse = target logit")
    _close(out["dh"], np.zeros((5, 4)), 1e-14, "V = 1: dH = 0")


def pin_equal_rows(ref):
    x = _case(5, 9, 4, 7)
    wq = np.repeat(x["w"][:1], 9, axis=0)
    out = ref.ce_reference(x["h"], wq, x["targets"], x["dnll"])
    _close(out["nll"], np.full(5, math.log(9)), 1e-13, "equal rows: nll = log V")
    _close(out["dh"], np.zeros((5, 4)), 1e-13, "equal rows: dH = 0")


def pin_shift_rows(ref):
    x = _case(6, 10, 4, 8)
    c = np.random.default_rng(0).standard_normal(4)
    a = ref.ce_reference(x["h"], x["w"], x["targets"], x["dnll"])
    b = ref.ce_reference(x["h"], np.asarray(x["w"], np.float64) + c, x["targets"], x["dnll"])
    hc = np.asarray(x["h"], np.float64) @ c
    _close(b["nll"], a["nll"], 1e-12, "row shift: nll")
    _close(b["dh"], a["dh"], 1e-12, "row shift: dH")
    _close(b["lse"], a["lse"] + hc, 1e-12, "row shift: lse")
    _close(b["tgt"], a["tgt"] + hc, 1e-12, "row shift: target logit")


def pin_bounds_and_linearity(ref):
    x = _case(7, 12, 5, 9)
    out = ref.ce_reference(x["h"], x["w"], x["targets"], x["dnll"])
    z = np.asarray(x["h"], np.float64) @ np.asarray(x["w"], np.float64).T
    assert np.all(z.max(1) <= out["lse"] + 1e-12) and np.all(out["lse"] <= z.max(1) + math.log(12) + 1e-12)
    two = ref.ce_reference(x["h"], x["w"], x["targets"], 2.0 * x["dnll"])
    _close(two["dh"], 2.0 * out["dh"], 1e-12, "dH linear in dnll")


ALL_PINS = [pin_torch_cross_entropy, pin_finite_differences, pin_loop, pin_one_word_vocabulary,
            pin_equal_rows, pin_shift_rows, pin_bounds_and_linearity]
