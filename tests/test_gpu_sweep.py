"""Parity-sweep grid on the GPU: many small shapes against the fp64 oracle,
element by element (the lab record's gradient-parity entry sweeps dtypes,
head dims, grouped-query ratios, queries shorter than keys, windows from 1 up,
causal and not). The cases are a fixed, seeded draw from that grid plus its
corners; each case spans several tiles with ragged tails."""
import os
import zlib

import numpy as np
import pytest

import gpu_helpers as H
from sliding_window_flash_amd.workloads import INT32_MAX, make_inputs, small_case

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "bf16", "fp16")
RULE_MIN_WINDOW = 7
# half a unit in the last place at 1.0 of each I/O type: the largest relative
# error of rounding one exact output to it (2^-9 bf16, 2^-12 fp16, 2^-25 fp32)
HALF_ULP = {"bf16": 2.0 ** -9, "fp16": 2.0 ** -12, "f32": 2.0 ** -25}
WINDOWS = (1, 2, 7, 31, 64, 100, 128, 129, 300, 1000, INT32_MAX)
LONG_WINDOWS = (1000, 2000, 5000)


def _grid(n=60, seed=2024, longer_q=False):
    """The record's grid: head dims 64 to 512, windows 1 to 5,000 (and none),
    grouped-query ratios, queries shorter than keys, causal and not. One case
    in ten is a single long sequence (1,500 to 6,000 tokens) under a window of
    1,000 to 5,000, so that the long windows bite. ``longer_q``: the cases
    with unequal lengths get more queries than keys instead (down to no key),
    beyond the record's grid."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        dt = DTYPES[rng.integers(3)]
        if rng.random() < 0.1:
            d = int(rng.choice([64, 128]))
            lq = [int(rng.integers(1500, 6000))]
            lk = None
            hkv, g = 1, int(rng.choice([1, 2, 4]))
            causal = rng.random() < 0.7
            window = int(LONG_WINDOWS[rng.integers(len(LONG_WINDOWS))])
            cases.append((tuple(lq), lk, hkv * g, hkv, d, window, causal, dt))
            continue
        d = int(rng.choice([64, 128, 256, 512] if dt != "f32" else [64, 128]))
        hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 2, 3, 4, 5, 8]))   # odd groups: forward/dQ head chunks of 1, odd dK/dV step counts
        nseq = int(rng.integers(1, 4))
        lq = [int(x) for x in rng.integers(1, 400, nseq)]
        shorter = rng.random() < 0.35          # queries shorter than keys
        lk = [q + int(rng.integers(1, 200)) for q in lq] if shorter else None
        if shorter and longer_q:
            lk = [max(0, q - int(rng.integers(1, 200))) for q in lq]
        causal = rng.random() < 0.7
        window = int(WINDOWS[rng.integers(len(WINDOWS))])   # without causal: two-sided
        cases.append((tuple(lq), None if lk is None else tuple(lk), hkv * g, hkv, d, window, causal, dt))
    return cases


# SWA_SWEEP_CASES / SWA_SWEEP_SEED widen the draw for a longer run (3,000 cases
# take about two minutes on one GPU); the default is the fixed 60-case draw.
# SWA_SWEEP_LONGER_Q=1 draws more queries than keys where lengths differ.
CASES = _grid(int(os.environ.get("SWA_SWEEP_CASES", "60")), int(os.environ.get("SWA_SWEEP_SEED", "2024")),
              os.environ.get("SWA_SWEEP_LONGER_Q", "0") == "1")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_grid_covers_its_corners():
    seen = {(c[7], c[4]) for c in CASES}
    assert {("f32", 64), ("bf16", 128), ("fp16", 256)} <= seen
    assert any(c[4] == 512 for c in CASES) and any(c[5] == 5000 for c in CASES)
    assert any(c[5] == 1 for c in CASES) and any(not c[6] for c in CASES)
    assert any(c[1] is not None for c in CASES) and any(c[2] // c[3] == 4 for c in CASES)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[7]}-d{c[4]}-g{c[2] // c[3]}-w{c[5]}-{'c' if c[6] else 'nc'}-{len(c[0])}seq")
def test_sweep_case(case):
    lq, lk, hq, hkv, d, win, causal, dt = case
    # dO at 0.1 as in the bench workloads: at window 1 the exact dQ and dK are
    # zero and what remains is rounding of dP - D, which scales with |dO| |V|;
    # the zero-reference bars are set for that scale
    w = small_case(lq, lk, heads_q=hq, heads_kv=hkv, head_dim=d, window=win, causal=causal, dtype=dt,
                   do_scale=0.1, seed=zlib.crc32(repr(case).encode()) % 10000)
    H.say(f"sweep case {case}")
    x = make_inputs(w)
    dev = H.to_device(w, x)
    got = H.run_hip(w, dev)
    zero = ("dq", "dk") if win == 1 else ()
    stats = H.compare_full(w, x, got, zero=zero, scale_f32=True)
    # The record's acceptance rule: a windowed backward's error stays within
    # twice the plain backward's error at the same shape (the same inputs with
    # no window: causal attention for a causal window, full attention for a
    # two-sided one, which can hold up to twice as many cells), plus the
    # dtype's half unit of rounding of the outputs. Windows below 7 keep only
    # a handful of terms per row, where a relative error says little (window 1
    # has exact-zero dQ and dK).
    if RULE_MIN_WINDOW <= win < max(max(w.lengths_q), max(w.lengths_k)):
        plain_w = w.replace(window=INT32_MAX)
        base = H.compare_full(plain_w, x, H.run_hip(plain_w, dev), scale_f32=True)
        floor = HALF_ULP[dt]
        for key in ("dq", "dk", "dv"):
            assert stats[key]["rel_fro"] <= 2 * base[key]["rel_fro"] + floor, (
                f"{key}: windowed rel-Fro {stats[key]['rel_fro']:.3e} > 2 x unwindowed "
                f"{base[key]['rel_fro']:.3e} + {floor:.1e}")


# Query-major workgroups take 4, 2 or 1 heads of a KV group (the largest that
# divides the group size) and 32, 64 or 128 rows; with groups larger than that
# a group is split into several head chunks. These cases exercise every chunk
# layout: groups 8 and 12 (4 heads x 32 rows, 2 and 3 chunks), 6 (2 heads x 64
# rows, 3 chunks) and 5 (1 head x 128 rows, 5 chunks).
GROUP_CASES = [
    ((200, 57), None, 16, 2, 128, 64, True, "bf16"),
    ((130, 261), (260, 300), 24, 2, 64, 100, True, "f32"),
    ((97, 190), None, 12, 2, 128, 31, False, "bf16"),
    ((300,), (333,), 6, 1, 64, INT32_MAX, True, "fp16"),
    ((150, 33, 70), None, 10, 2, 128, 129, True, "bf16"),
]


@pytest.mark.parametrize("case", GROUP_CASES, ids=lambda c: f"{c[7]}-d{c[4]}-g{c[2] // c[3]}-w{c[5]}-{'c' if c[6] else 'nc'}")
def test_group_chunks(case):
    lq, lk, hq, hkv, d, win, causal, dt = case
    w = small_case(lq, lk, heads_q=hq, heads_kv=hkv, head_dim=d, window=win, causal=causal, dtype=dt,
                   do_scale=0.1, seed=zlib.crc32(repr(case).encode()) % 10000)
    H.say(f"group-chunk case {case}")
    x = make_inputs(w)
    got = H.run_hip(w, H.to_device(w, x))
    H.compare_full(w, x, got)
