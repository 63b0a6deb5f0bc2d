"""The oracle against what the pages and the mathematics fix (no GPU)."""
import numpy as np

import sliding_window_flash_amd.workloads as W
import pytest

import oracle_pins as pins
from oracle import dense
from sliding_window_flash_amd.workloads import INT32_MAX, make_inputs, random_mask, small_case


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(dense)


def test_sampled_rows_match_full_reference():
    w = small_case([150, 90, 0, 70], [180, 90, 5, 70], heads_q=4, heads_kv=2, head_dim=16,
                   window=40, seed=21)
    x = make_inputs(w)
    args = (x["q"], x["k"], x["v"], x["do"], x["cu_q"], x["cu_k"], w.scale, w.window, w.causal)
    full = dense.sdpa_reference(*args, panel_rows=37)
    rng = np.random.default_rng(0)
    toks = rng.integers(0, w.total_q, 25)
    heads = rng.integers(0, w.heads_q, 25)
    rows = dense.sdpa_query_rows(*args, toks, heads)
    np.testing.assert_allclose(rows["o"], full["o"][toks, heads], atol=1e-13)
    np.testing.assert_allclose(rows["lse"], full["lse"][heads, toks], atol=1e-13)
    np.testing.assert_allclose(rows["delta"], full["delta"][heads, toks], atol=1e-13)
    np.testing.assert_allclose(rows["dq"], full["dq"][toks, heads], atol=1e-13)
    ktoks = np.concatenate([rng.integers(0, w.total_k, 20), [0, 179, 180, 275]])
    kh = rng.integers(0, w.heads_kv, ktoks.size)
    keys = dense.sdpa_key_rows(*args, ktoks, kh, panel_rows=11)
    np.testing.assert_allclose(keys["dk"], full["dk"][ktoks, kh], atol=1e-13)
    np.testing.assert_allclose(keys["dv"], full["dv"][ktoks, kh], atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_sampled_rows_match_full_reference_masked(causal):
    """The row samplers read the same mask rows as the full reference, also
    through the packed-row view used at large sizes."""
    w = small_case([150, 90, 70], [180, 90, 70], heads_q=4, heads_kv=2, head_dim=16,
                   window=40, causal=causal, seed=22)
    x = make_inputs(w)
    m = W.random_mask(w, 0.7, seed=23, empty_rows=3)
    view = W.PackedMaskRows(W.pack_mask(m), 180)
    args = (x["q"], x["k"], x["v"], x["do"], x["cu_q"], x["cu_k"], w.scale, w.window, w.causal)
    full = dense.sdpa_reference(*args, panel_rows=37, mask=m)
    rng = np.random.default_rng(1)
    toks = rng.integers(0, w.total_q, 25)
    heads = rng.integers(0, w.heads_q, 25)
    rows = dense.sdpa_query_rows(*args, toks, heads, mask=view)
    np.testing.assert_allclose(rows["o"], full["o"][toks, heads], atol=1e-13)
    np.testing.assert_array_equal(np.isfinite(rows["lse"]), np.isfinite(full["lse"][heads, toks]))
    fin = np.isfinite(rows["lse"])
    np.testing.assert_allclose(rows["lse"][fin], full["lse"][heads, toks][fin], atol=1e-13)
    np.testing.assert_allclose(rows["dq"], full["dq"][toks, heads], atol=1e-13)
    ktoks = np.concatenate([rng.integers(0, w.total_k, 20), [0, 179, 180, 339]])
    kh = rng.integers(0, w.heads_kv, ktoks.size)
    keys = dense.sdpa_key_rows(*args, ktoks, kh, panel_rows=11, mask=view)
    np.testing.assert_allclose(keys["dk"], full["dk"][ktoks, kh], atol=1e-13)
    np.testing.assert_allclose(keys["dv"], full["dv"][ktoks, kh], atol=1e-13)


def test_unvisited_keys_get_exact_zero():
    # fewer queries than keys with a short window: the first keys are seen by nobody
    w = small_case([4], [20], heads_q=2, heads_kv=1, head_dim=3, window=3, seed=22)
    x = make_inputs(w)
    out = dense.sdpa_reference(x["q"], x["k"], x["v"], x["do"], x["cu_q"], x["cu_k"],
                               w.scale, w.window, w.causal)
    assert np.all(out["dk"][:14] == 0) and np.all(out["dv"][:14] == 0)
    assert np.all(np.abs(out["dv"][14:]).sum(-1) > 0)


def test_empty_rows_convention():
    # a sequence with queries but no keys: O = 0, LSE = -inf, dQ = 0
    w = small_case([3], [0], heads_q=1, heads_kv=1, head_dim=2, seed=23)
    x = make_inputs(w)
    out = dense.sdpa_reference(x["q"], x["k"], x["v"], x["do"], x["cu_q"], x["cu_k"],
                               w.scale, INT32_MAX, True)
    assert np.all(out["o"] == 0) and np.all(np.isneginf(out["lse"])) and np.all(out["dq"] == 0)


def test_two_sided_mask_is_the_band():
    m = dense.visible_cells(5, 7, 2, False)
    for i in range(5):
        p = i + 2
        assert [j for j in range(7) if m[i, j]] == [j for j in (p - 1, p, p + 1) if 0 <= j < 7]


def test_host_ram_guard_refuses_up_front():
    w = small_case([64], heads_q=1, heads_kv=1, head_dim=4, seed=24)
    x = make_inputs(w)
    with pytest.raises(dense.HostRamExceeded):
        dense.sdpa_reference(x["q"], x["k"], x["v"], x["do"], x["cu_q"], x["cu_k"], w.scale,
                             8, True, ram_ceiling=1024)


def test_row_and_head_sample_matches_full_reference():
    w = small_case([300, 40], [320, 40], heads_q=4, heads_kv=2, head_dim=8, window=30, seed=25)
    x = make_inputs(w)
    args = (x["q"], x["k"], x["v"], x["do"], x["cu_q"], x["cu_k"], w.scale, w.window, w.causal)
    full = dense.sdpa_reference(*args)
    part = dense.sdpa_reference(*args, heads=[2], query_rows=(17, 250), panel_rows=50)
    for b, (q0, q1) in enumerate(zip(x["cu_q"][:-1], x["cu_q"][1:])):
        r = slice(q0 + 17, min(q1, q0 + 250))
        np.testing.assert_allclose(part["o"][r, 2], full["o"][r, 2], atol=1e-13)
        np.testing.assert_allclose(part["dq"][r, 2], full["dq"][r, 2], atol=1e-13)
        np.testing.assert_allclose(part["lse"][2, r], full["lse"][2, r], atol=1e-13)
    assert np.all(part["o"][:, [0, 1, 3]] == 0)


@pytest.mark.parametrize("lq,lk", [(300, 300), (40, 300), (1, 1), (7, 200), (0, 5), (513, 600),
                                   (300, 40), (64, 1), (5, 0)])
@pytest.mark.parametrize("window", [1, 2, 31, 64, 129, 700, INT32_MAX])
@pytest.mark.parametrize("causal", [True, False])
def test_key_band_holds_every_visible_cell(lq, lk, window, causal):
    """Brute force over every row panel: no visible cell lies outside the band,
    and the band's first and last keys are visible to some row of the panel
    (so the band is exactly the span of the visible keys when that span is not
    empty)."""
    full = dense.visible_cells(lq, lk, window, causal)
    for rows_per in (1, 5, 64, 512):
        for r0 in range(0, lq, rows_per):
            r1 = min(lq, r0 + rows_per)
            c0, c1 = dense.key_band(r0, r1, lq, lk, window, causal)
            part = full[r0:r1]
            outside = np.ones(lk, bool)
            outside[c0:c1] = False
            assert not part[:, outside].any(), (r0, r1, c0, c1)
            if part.any():
                cols = np.nonzero(part.any(axis=0))[0]
                assert (cols[0], cols[-1] + 1) == (c0, c1), (r0, r1, c0, c1, cols[0], cols[-1])


@pytest.mark.parametrize("case", [
    ([300, 1, 517, 64], None, 8, 2, 16, 129, True),
    ([100, 40], [700, 300], 4, 1, 8, 16, True),     # queries shorter than keys
    ([200, 0, 333], None, 4, 2, 8, 65, False),      # two-sided, empty sequence
    ([257], None, 2, 2, 8, 1, True),                # window 1
    ([257, 90], None, 2, 1, 8, INT32_MAX, True),    # plain causal
    ([200, 333], None, 2, 1, 8, INT32_MAX, False),  # full attention
    ([300, 90], [100, 300], 4, 2, 8, 40, True),     # more queries than keys
    ([300, 90], [100, 300], 4, 2, 8, 150, False),   # the same, two-sided
])
@pytest.mark.parametrize("masked", [False, True])
def test_band_reference_matches_full_reference(case, masked):
    lq, lk, hq, hkv, d, win, causal = case
    w = small_case(lq, lk, heads_q=hq, heads_kv=hkv, head_dim=d, window=win, causal=causal, seed=61)
    x = make_inputs(w)
    kw = {}
    if masked:
        kw["mask"] = random_mask(w, 0.6, seed=62, empty_rows=3)
    args = (x["q"], x["k"], x["v"], x["do"], x["cu_q"], x["cu_k"], w.scale, w.window, w.causal)
    full = dense.sdpa_reference(*args, panel_rows=100, **kw)
    band = dense.sdpa_reference(*args, panel_rows=100, band=True, **kw)
    for key in ("o", "lse", "delta", "dq", "dk", "dv"):
        a, b = band[key], full[key]
        fin = np.isfinite(b)
        assert np.array_equal(np.isfinite(a), fin), key
        tol = 1e-12 * max(1.0, float(np.abs(b[fin]).max(initial=0.0)))
        assert float(np.abs(a[fin] - b[fin]).max(initial=0.0)) <= tol, key
