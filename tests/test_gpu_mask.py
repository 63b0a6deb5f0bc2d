"""A boolean mask combined with the window, through attn_fwd_masked and
attn_bwd_masked, against the fp64 oracle element by element.

Reading ("Off NVIDIA, you fix the platform yourself", list of what is not
proved, and its backward-memory record entry): a cell is visible iff the window
shows it and the caller's boolean mask (one per packed batch, shared by every
head) allows it. Cases cover every dtype and head_dim, causal and two-sided
windows, queries shorter than keys, several tiles with ragged tails, masks
from nearly empty to nearly full, rows that allow no key at all, document
(block-diagonal) masks, and the 32K-token document workload on sampled rows.
"""
import os

import numpy as np
import pytest

import gpu_helpers as H
import sliding_window_flash_amd.workloads as W
from sliding_window_flash_amd.workloads import INT32_MAX, make_inputs, small_case

pytestmark = pytest.mark.gpu

# (lengths_q, lengths_k, heads_q, heads_kv, head_dim, window, causal, dtype, density, empty rows)
CASES = [
    ([300, 77], None, 4, 2, 128, 96, True, "bf16", 0.7, 3),
    ([260], [333], 4, 1, 64, 129, True, "f32", 0.5, 2),
    ([190, 64], None, 2, 2, 128, 50, False, "bf16", 0.85, 1),
    ([211], [300], 4, 2, 128, INT32_MAX, True, "fp16", 0.3, 0),
    ([150, 45], [160, 90], 2, 1, 256, 70, True, "bf16", 0.6, 2),
    ([129], None, 2, 1, 64, 40, False, "f32", 0.97, 1),
    ([257], None, 4, 4, 64, 300, True, "fp16", 0.15, 4),
    ([97, 200], [120, 230], 2, 1, 256, INT32_MAX, False, "fp16", 0.5, 1),
    ([150, 45], [160, 90], 3, 1, 256, 70, True, "bf16", 0.6, 2),  # odd group at 256
    # groups split into head chunks (forward / dQ workgroups take 4 or 2 heads)
    ([170, 90], None, 16, 2, 128, 80, True, "bf16", 0.6, 2),
    ([140], [200], 6, 1, 64, 60, False, "f32", 0.7, 1),
    # head_dim 512: 32-key forward / dQ tiles, one mask word per row and tile
    ([150, 45], [160, 90], 4, 2, 512, 70, True, "bf16", 0.6, 2),
    ([211], None, 2, 1, 512, 90, False, "fp16", 0.4, 1),
    # more queries than keys (negative positions)
    ([330, 60], [90, 100], 4, 2, 128, 50, True, "bf16", 0.6, 2),
    ([330, 60], [90, 100], 2, 1, 64, 120, False, "f32", 0.7, 1),
]


def _device_mask(m, max_lk):
    import torch
    bits = W.pack_mask(m, W.mask_row_words(max_lk))
    return torch.from_numpy(bits.view(np.int32)).cuda()


def _run_masked(case, seed, scale_f32=False):
    lq, lk, hq, hkv, d, win, causal, dt, dens, empty = case
    w = small_case(lq, lk, heads_q=hq, heads_kv=hkv, head_dim=d, window=win, causal=causal,
                   dtype=dt, do_scale=1.0 if dt == "f32" else 0.1, seed=seed)
    H.say(f"masked case {case}: {w}")
    x = make_inputs(w)
    m = W.random_mask(w, dens, seed=seed + 50, empty_rows=empty)
    dev = H.to_device(w, x)
    got = H.run_hip(w, dev, mask=_device_mask(m, max(w.lengths_k)))
    stats = H.compare_full(w, x, got, mask=m, scale_f32=scale_f32)
    H.say("   ", {k: {a: f"{b:.2e}" for a, b in v.items()} for k, v in stats.items()})
    # a row that allows no key: O = 0, LSE = -inf, dQ = 0
    dead = np.nonzero(~m.any(axis=1))[0]
    if dead.size:
        assert np.all(H.host64(got["o"])[dead] == 0)
        assert np.all(H.host64(got["lse"])[:, dead] == -np.inf)
        assert np.all(H.host64(got["dq"])[dead] == 0)


@pytest.mark.parametrize("n", range(len(CASES)))
def test_masked_small_full_oracle(n):
    _run_masked(CASES[n], 700 + n)


def _mask_grid(n, seed):
    """Seeded random draw over the same axes as CASES (every dtype and head_dim,
    KV groups 1 to 8, causal and two-sided windows, L_q < L_k, densities and
    rows that allow no key)."""
    rng = np.random.default_rng(seed)
    out = []
    windows = (1, 7, 33, 64, 100, 129, 300, INT32_MAX)
    while len(out) < n:
        dt = ("f32", "bf16", "fp16")[rng.integers(3)]
        d = int(rng.choice([64, 128, 256, 512] if dt != "f32" else [64, 128]))
        hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 2, 3, 4, 8]))
        lq = [int(x) for x in rng.integers(1, 300, int(rng.integers(1, 3)))]
        lk = [q + int(rng.integers(1, 150)) for q in lq] if rng.random() < 0.35 else None
        out.append((lq, lk, hkv * g, hkv, d, int(windows[rng.integers(len(windows))]), bool(rng.random() < 0.6), dt,
                    float(rng.uniform(0.1, 0.98)), int(rng.integers(0, 4))))
    return out


# SWA_MASK_SWEEP_CASES widens the draw for a longer run; the default is 16 cases
MASK_SWEEP = _mask_grid(int(os.environ.get("SWA_MASK_SWEEP_CASES", "16")), int(os.environ.get("SWA_MASK_SWEEP_SEED", "31")))


@pytest.mark.parametrize("n", range(len(MASK_SWEEP)))
def test_masked_sweep(n):
    _run_masked(MASK_SWEEP[n], 900 + n, scale_f32=True)


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f32", 64), ("fp16", 256)])
def test_documents_full_oracle(dt, d):
    """Block-diagonal masks: packed documents inside each sequence."""
    w = small_case([700, 333], [760, 333], heads_q=4, heads_kv=2, head_dim=d, window=200,
                   dtype=dt, do_scale=1.0 if dt == "f32" else 0.1, seed=33)
    x = make_inputs(w)
    docs = [[100, 300, 5, 355], [333]]
    bits = W.document_mask_bits(w, docs)
    m = W.unpack_rows(bits, range(w.total_q), max(w.lengths_k))
    import torch
    got = H.run_hip(w, H.to_device(w, x), mask=torch.from_numpy(bits.view(np.int32)).cuda())
    stats = H.compare_full(w, x, got, mask=m)
    H.say(f"documents {dt} d={d}:", {k: {a: f"{b:.2e}" for a, b in v.items()} for k, v in stats.items()})


@pytest.mark.parametrize("dt,d,causal", [("bf16", 128, True), ("fp16", 64, False), ("f32", 128, True),
                                         ("bf16", 256, True)])
def test_all_true_mask_is_bitwise_the_unmasked_path(dt, d, causal):
    """The masked kernels do the same arithmetic on the cells the window shows."""
    import torch
    w = small_case([517, 130], [600, 130], heads_q=4, heads_kv=2, head_dim=d, window=150,
                   causal=causal, dtype=dt, do_scale=0.1, seed=34)
    x = make_inputs(w)
    dev = H.to_device(w, x)
    a = H.run_hip(w, dev)
    ones = np.ones((w.total_q, 600), bool)
    b = H.run_hip(w, dev, mask=_device_mask(ones, 600))
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_document_workload_32k_sampled():
    """The bench workload's shape (bf16, 32,768 tokens, window 1,024, 32/8
    heads, d 128) with its tokens packed from corpus-like documents."""
    import torch
    w = W.SWA_32K
    x = make_inputs(w)
    docs = W.document_lengths(91, w.lengths_k[0])
    bits = W.document_mask_bits(w, [docs])
    H.say(f"32K document mask: {len(docs)} documents {docs}")
    got = H.run_hip(w, H.to_device(w, x), mask=torch.from_numpy(bits.view(np.int32)).cuda())
    view = W.PackedMaskRows(bits, w.lengths_k[0])
    stats = H.compare_sampled(w, x, got, n_q=5, n_k=3, seed=5, mask=view)
    H.say("   ", {k: {a: f"{b:.2e}" for a, b in v.items()} for k, v in stats.items()})
    # the first token of every document sees only itself
    starts = np.cumsum([0] + docs[:-1])
    for t in starts[:4]:
        h = 0
        np.testing.assert_allclose(H.host64(got["o"][int(t), h]), x["v"][int(t), 0].astype(np.float64),
                                   atol=H.BF16_MAX_ABS)
