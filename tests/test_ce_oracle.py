"""The fp64 linear cross-entropy oracle against its pins; planted mistakes in
a copy of it must each fail at least one pin; row sampling matches the full
computation."""
import os
import types

import numpy as np
import pytest

import ce_pins as pins
from oracle import ce
from sliding_window_flash_amd.workloads import CEWorkload, make_ce_inputs

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "ce.py")


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(ce)


MUTANTS = {
    "log base 2 in LSE": ("lse = m + np.log(", "lse = m + np.log2("),
    "target logit of the row index": ("tgt = z[np.arange(rr.size), targets[rr]]", "tgt = z[np.arange(rr.size), np.arange(rr.size) % z.shape[1]]"),
    "gradient without the target term": ("(p @ w64 - w64[targets[rr]])", "(p @ w64)"),
    "gradient sign": ("(p @ w64 - w64[targets[rr]])", "(w64[targets[rr]] - p @ w64)"),
    "probabilities not normalised": ("p = np.exp(z - lse[:, None])", "p = np.exp(z - m[:, None])"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("ce_mutant")
    exec(compile(src.replace(old, new), "ce_mutant", "exec"), mod.__dict__)
    caught = False
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            caught = True
            break
    assert caught, f"no pin catches the planted mistake: {name}"


def test_row_sample_matches_full():
    x = make_ce_inputs(CEWorkload("t", 40, 300, 16, "bf16", 3))
    full = ce.ce_reference(x["h"], x["w"], x["targets"], x["dnll"], panel_rows=7)
    rows = np.array([0, 5, 39, 17])
    part = ce.ce_reference(x["h"], x["w"], x["targets"], x["dnll"][rows], rows=rows)
    for key in ("nll", "lse", "tgt", "dh"):
        np.testing.assert_allclose(part[key], full[key][rows], atol=1e-13)
