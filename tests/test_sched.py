"""The block-range scheduler (host build, through the C ABI) against brute-force
enumeration of the visibility mask: every visible cell lies in a visited tile,
no visited tile is all-masked, and "full" tiles have no masked cell."""
import itertools

import numpy as np
import pytest

import sliding_window_flash_amd as swa
from oracle.dense import visible_cells
from sliding_window_flash_amd.workloads import INT32_MAX


def params(lq, lk, window, causal):
    return swa.make_params(batch=1, heads_q=1, heads_kv=1, head_dim=64, total_q=lq, total_k=lk,
                           max_seqlen_q=lq, max_seqlen_k=lk, window=window, causal=causal,
                           scale=1.0, dtype=swa.ATTN_F32)


def brute(lq, lk, window, causal, bm, bn):
    mask = visible_cells(lq, lk, window, causal) if lq and lk else np.zeros((lq, lk), bool)
    nqb, nkb = -(-lq // bm), -(-lk // bn)
    any_vis = np.zeros((nqb, nkb), bool)
    full = np.zeros((nqb, nkb), bool)
    for qb, kb in itertools.product(range(nqb), range(nkb)):
        blk = mask[qb * bm:(qb + 1) * bm, kb * bn:(kb + 1) * bn]
        any_vis[qb, kb] = blk.any()
        full[qb, kb] = blk.shape == (bm, bn) and blk.all()
    return any_vis, full


CASES = [
    # lq, lk, window, causal
    (256, 256, 32, True), (1024, 1024, 32, True), (300, 300, 1, True), (300, 300, 127, True),
    (300, 300, 128, True), (300, 300, 129, True), (300, 300, INT32_MAX, True),
    (100, 700, 64, True), (5, 400, 3, True), (0, 50, 8, True), (77, 77, 77, True),
    (200, 260, INT32_MAX, False), (129, 129, 1000, True), (64, 64, 64, True),
    # two-sided windows (no causal mask)
    (300, 300, 1, False), (300, 300, 64, False), (300, 300, 129, False), (100, 700, 64, False),
    (5, 400, 3, False), (200, 260, 100, False), (129, 129, 128, False),
    # more queries than keys (negative positions), and queries without keys
    (400, 100, 64, True), (300, 50, INT32_MAX, True), (130, 1, 1, True), (50, 0, 8, True),
    (300, 50, 64, False), (300, 50, 250, False), (97, 5, 3, False), (50, 0, 8, False),
]


@pytest.mark.parametrize("bm,bn", [(128, 64), (64, 128), (32, 32), (64, 64)])
@pytest.mark.parametrize("lq,lk,window,causal", CASES)
def test_query_major_ranges(lq, lk, window, causal, bm, bn):
    p = params(lq, lk, window, causal)
    any_vis, full = brute(lq, lk, window, causal, bm, bn)
    for qb in range(-(-lq // bm)):
        lo, hi, flo, fhi = swa.query_tile_range(p, [0, lq], [0, lk], 0, qb, bm, bn)
        vis = np.nonzero(any_vis[qb])[0]
        if vis.size == 0:
            assert lo > hi
            continue
        assert (lo, hi) == (vis.min(), vis.max()), (qb, lo, hi, vis)
        assert vis.size == hi - lo + 1          # contiguous: no all-masked tile is visited
        fulls = np.nonzero(full[qb])[0]
        if fulls.size == 0:
            assert flo > fhi
        else:
            assert (flo, fhi) == (fulls.min(), fulls.max()) and fulls.size == fhi - flo + 1


@pytest.mark.parametrize("bm,bn", [(64, 128), (32, 64), (64, 64)])
@pytest.mark.parametrize("lq,lk,window,causal", CASES)
def test_key_major_ranges(lq, lk, window, causal, bm, bn):
    p = params(lq, lk, window, causal)
    any_vis, _ = brute(lq, lk, window, causal, bm, bn)
    for kb in range(-(-lk // bn)):
        lo, hi = swa.key_tile_range(p, [0, lq], [0, lk], 0, kb, bn, bm)
        vis = np.nonzero(any_vis[:, kb])[0] if any_vis.size else np.zeros(0, int)
        if vis.size == 0:
            assert lo > hi, (kb, lo, hi)
        else:
            assert (lo, hi) == (vis.min(), vis.max()) and vis.size == hi - lo + 1


def test_int32_max_window_does_not_overflow():
    p = params(40000, 40000, INT32_MAX, True)
    lo, hi, flo, fhi = swa.query_tile_range(p, [0, 40000], [0, 40000], 0, 100, 128, 64)
    assert lo == 0 and hi == (100 * 128 + 127) // 64 and (flo, fhi) == (0, 199)
    lo, hi = swa.key_tile_range(p, [0, 40000], [0, 40000], 0, 0, 128, 64)
    assert (lo, hi) == (0, (40000 - 1) // 64)


@pytest.mark.parametrize("head_dim", [128, 256, 512])
def test_compiled_tiles_hit_both_silent_cases(head_dim):
    """With the tile sizes the kernels use, N=1024 / w=32 has query tiles whose
    first visited key tile is not tile zero, and L_q < L_k with a short window
    has key tiles that no query visits."""
    bm, bn, kbn, kbm = swa.tile_sizes(head_dim, swa.ATTN_BF16)
    p = params(1024, 1024, 32, True)
    los = [swa.query_tile_range(p, [0, 1024], [0, 1024], 0, qb, bm, bn)[0]
           for qb in range(1024 // bm)]
    assert max(los) > 0
    p = params(100, 1000, 16, True)
    empty = [kb for kb in range(-(-1000 // kbn))
             if (lambda r: r[0] > r[1])(swa.key_tile_range(p, [0, 100], [0, 1000], 0, kb, kbn, kbm))]
    assert empty, "expected unvisited key tiles"


def test_xcd_remap_is_a_bijection():
    """The launch-id remap used by the kernels (host build of the same code,
    re-derived here from its definition) covers every logical id once."""
    for n in (1, 7, 8, 9, 64, 100, 2048, 8191):
        seen = set()
        for i in range(n):
            xcd, slot = i % 8, i // 8
            per, rem = n // 8, n % 8
            L = xcd * (per + 1) + slot if xcd < rem else rem * (per + 1) + (xcd - rem) * per + slot
            assert 0 <= L < n
            seen.add(L)
        assert len(seen) == n
