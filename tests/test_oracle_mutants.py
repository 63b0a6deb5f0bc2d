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
    "scale dropped from dQ": ("= scale * (ds @ kg)", "= (ds @ kg)"),
    "dV from dS instead of P": ('+= res["p"].T @ doh', '+= res["ds"].T @ doh'),
    "interleaved head groups": ("g = h // grp\n            kg", "g = h % hkv\n            kg"),
    "log base 2 in LSE": ("lse = np.where(has_key, m + np.log(zs)", "lse = np.where(has_key, m + np.log2(zs)"),
    "dK from dO instead of Q": ("scale * (ds.T @ qh)", "scale * (ds.T @ doh)"),
    "two-sided window one-sided": ("vis = np.abs(pos - j[None, :]) < window", "vis = (pos - j[None, :]) < window"),
    "two-sided window one key wider": ("vis = np.abs(pos - j[None, :]) < window",
                                       "vis = np.abs(pos - j[None, :]) <= window"),
    "mask ignored": ("vis = vis & np.asarray(allowed, dtype=bool)[:, :lk]", "vis = vis"),
    "mask rows not offset by the sequence start": ("mask[q0 + np.asarray(rows, dtype=np.int64)]",
                                                   "mask[np.asarray(rows, dtype=np.int64)]"),
    "mask complement applied": ("vis & np.asarray(allowed, dtype=bool)[:, :lk]",
                                "vis & ~np.asarray(allowed, dtype=bool)[:, :lk]"),
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
