"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Each mutant is the text of oracle/dense.py with one plausible error (a wrong
comparison, index, sign, dropped term or swapped operand), executed as a
separate module on the CPU. The real oracle is never modified.
"""
import os
import types

import pytest

import oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "dense.py")

MUTANTS = {
    "window counts one extra key": ("pos - j[None, :] < window", "pos - j[None, :] <= window"),
    "queries aligned to the start": ("pos = (i + (lk - lq))[:, None]", "pos = (i + 0)[:, None]"),
    "D with the wrong sign": ("ds = p * (dp - dlt[:, None])", "ds = p * (dp + dlt[:, None])"),
    "D term dropped": ("ds = p * (dp - dlt[:, None])", "ds = p * dp"),
    "scale dropped from dQ": ("= scale * (ds @ kb)", "= (ds @ kb)"),
    "dV from dS instead of P": ('+= res["p"].T @ doh', '+= res["ds"].T @ doh'),
    "interleaved head groups": ("g = h // grp\n            kg", "g = h % hkv\n            kg"),
    "log base 2 in LSE": ("lse = np.where(has_key, m + np.log(zs)", "lse = np.where(has_key, m + np.log2(zs)"),
    "dK from dO instead of Q": ("scale * (ds.T @ qh)", "scale * (ds.T @ doh)"),
    "two-sided window one-sided": ("vis = np.abs(pos - j[None, :]) < window", "vis = (pos - j[None, :]) < window"),
    "two-sided window one key wider": ("vis = np.abs(pos - j[None, :]) < window",
                                       "vis = np.abs(pos - j[None, :]) <= window"),
    "two-sided window >= L_k taken as full attention": (
        "vis = np.abs(pos - j[None, :]) < window",
        "vis = (np.abs(pos - j[None, :]) < window) | (window >= lk)"),
    "mask ignored": ("vis = vis & np.asarray(allowed, dtype=bool)[:, c0:c1]", "vis = vis"),
    "mask rows not offset by the sequence start": ("mask[q0 + np.asarray(rows, dtype=np.int64)]",
                                                   "mask[np.asarray(rows, dtype=np.int64)]"),
    "mask complement applied": ("vis & np.asarray(allowed, dtype=bool)[:, c0:c1]",
                                "vis & ~np.asarray(allowed, dtype=bool)[:, c0:c1]"),
}


def _mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, old
    mod = types.ModuleType("dense_mutant")
    exec(compile(src.replace(old, new, 1), "dense_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
            break
    assert caught, f"no pin catches the planted mistake: {name}"


# Planted mistakes in the key band (the optional restriction of each row
# panel to the keys that can be visible): the band result must then differ
# from the full panels on the cases that pin the band.
BAND_MUTANTS = {
    "causal band one key short": ("c1 = min(lk, p1 + 1) if causal", "c1 = min(lk, p1) if causal"),
    "band starts one key late": ("c0 = max(0, p0 - window + 1)", "c0 = max(0, p0 - window + 2)"),
    "two-sided band one key short": ("else min(lk, p1 + window)", "else min(lk, p1 + window - 1)"),
    "band keys not offset into dK": ("dk[k0 + c0:k0 + c1, g, :]", "dk[k0:k0 + c1 - c0, g, :]"),
}


@pytest.mark.parametrize("name", sorted(BAND_MUTANTS))
def test_band_mutant_is_caught(name):
    import numpy as np

    from sliding_window_flash_amd.workloads import make_inputs, small_case
    mod = _mutant(*BAND_MUTANTS[name])
    differs = False
    for lq, lk, win, causal in (([300, 40], [320, 40], 64, True), ([200, 333], None, 65, False)):
        w = small_case(lq, lk, heads_q=2, heads_kv=1, head_dim=8, window=win, causal=causal, seed=63)
        x = make_inputs(w)
        args = (x["q"], x["k"], x["v"], x["do"], x["cu_q"], x["cu_k"], w.scale, w.window, w.causal)
        full = mod.sdpa_reference(*args, panel_rows=100)
        band = mod.sdpa_reference(*args, panel_rows=100, band=True)
        for key in ("o", "lse", "dq", "dk", "dv"):
            a, b = np.nan_to_num(band[key], neginf=-1e300), np.nan_to_num(full[key], neginf=-1e300)
            differs |= not np.allclose(a, b, rtol=0, atol=1e-9)
    assert differs, f"the band mutant matches the full panels: {name}"
