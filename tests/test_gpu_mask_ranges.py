"""Tile skipping for a window combined with an arbitrary mask: the ranges
attn_mask_ranges writes (where the mask's allowed bits lie, per 32-row and per
32-key block) and the masked kernels that use them to skip the tiles the mask
empties. The lab's list of what is not proved names the window combined with
an arbitrary mask as the case that still falls back to the full score matrix.

The ranges are checked entry by entry against their definition, computed
here on the host from the packed mask; the masked outputs with the ranges must
equal the outputs without them bit for bit (a skipped tile has every cell
masked and adds nothing), on random masks with empty rows, document masks,
queries shorter than keys, two-sided windows, every dtype and head_dim, and
the 32K-token workload packed from short documents; those outputs are also
compared with the fp64 oracle on small cases.
"""
import numpy as np
import pytest

import gpu_helpers as H
import sliding_window_flash_amd as swa
import sliding_window_flash_amd.workloads as W
from sliding_window_flash_amd.workloads import INT32_MAX, make_inputs, small_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _kw(w):
    return dict(max_seqlen_q=w.max_seqlen_q, max_seqlen_k=w.max_seqlen_k, window=w.window, causal=w.causal,
                scale=w.scale)


def _visible_span(i0, i1, lq, lk, window, causal):
    """Keys [jlo, jhi] the window can show some row of [i0, i1] (rows < lq)."""
    d = lk - lq
    jlo = max(0, i0 + d - window + 1)
    jhi = min(lk - 1, i1 + d if causal else i1 + d + window - 1)
    return jlo, jhi


def _seeing_rows(j0, j1, lq, lk, window, causal):
    """Rows [ilo, ihi] the window lets see some key of [j0, j1]."""
    d = lk - lq
    ilo = max(0, j0 - d if causal else j0 - d - window + 1)
    ihi = min(lq - 1, j1 - d + window - 1)
    return ilo, ihi


def expected_ranges(w, bits):
    """The ranges by their definition: whole 32-bit words inside the window's
    band, the first and last block holding a nonzero one; (1, 0) when none."""
    nrb, nkb = -(-w.max_seqlen_q // 32), -(-w.max_seqlen_k // 32)
    rows = np.tile(np.array([1, 0], np.int32), (w.batch, nrb, 1))
    cols = np.tile(np.array([1, 0], np.int32), (w.batch, nkb, 1))
    q0s, k0s = w.cu_seqlens_q(), w.cu_seqlens_k()
    for b in range(w.batch):
        lq, lk, q0 = w.lengths_q[b], w.lengths_k[b], int(q0s[b])
        win = min(w.window, INT32_MAX)
        for rb in range(-(-lq // 32)):
            i0, i1 = 32 * rb, min(lq, 32 * rb + 32) - 1
            jlo, jhi = _visible_span(i0, i1, lq, lk, win, w.causal)
            if jlo > jhi:
                continue
            blk = bits[q0 + i0:q0 + i1 + 1, jlo // 32:jhi // 32 + 1]
            nz = np.nonzero(blk.any(axis=0))[0]
            if nz.size:
                rows[b, rb] = (jlo // 32 + nz[0], jlo // 32 + nz[-1])
        for cb in range(-(-lk // 32)):
            j0, j1 = 32 * cb, min(lk, 32 * cb + 32) - 1
            ilo, ihi = _seeing_rows(j0, j1, lq, lk, win, w.causal)
            if ilo > ihi:
                continue
            col = bits[q0 + ilo:q0 + ihi + 1, cb]
            nz = np.nonzero(col != 0)[0]
            if nz.size:
                cols[b, cb] = ((ilo + nz[0]) // 32, (ilo + nz[-1]) // 32)
    return np.concatenate([rows.ravel(), cols.ravel()])


def _ranges(w, dev, dmask):
    return swa.mask_ranges(dev["q"], dev["k"], dev["cu_q"], dev["cu_k"], dmask, **_kw(w))


CASES = [
    # (lengths_q, lengths_k, heads_q, heads_kv, head_dim, window, causal, dtype, mask kind)
    ([700, 333], [760, 333], 4, 2, 128, 200, True, "bf16", "documents"),
    ([700, 333], [760, 333], 4, 2, 64, 1000, False, "f32", "documents"),
    ([300, 77], None, 4, 2, 128, 96, True, "bf16", "random"),
    ([211], [300], 4, 2, 128, INT32_MAX, True, "fp16", "random-sparse"),
    ([150, 45], [160, 90], 2, 1, 256, 70, True, "bf16", "documents"),
    ([600], None, 4, 2, 512, 300, True, "fp16", "documents"),
    ([900, 200], None, 8, 2, 128, INT32_MAX, True, "bf16", "band"),
    ([400, 90], [100, 300], 4, 2, 128, 64, True, "bf16", "random"),      # L_q > L_k
    ([300, 77], [50, 80], 2, 1, 64, 60, False, "f32", "random"),
]


def _mask_for(w, kind, seed):
    if kind == "documents":
        docs = []
        rng = np.random.default_rng(seed)
        for L in w.lengths_k:
            d, left = [], L
            while left > 0:
                n = int(min(left, rng.integers(1, 200)))
                d.append(n)
                left -= n
            docs.append(d)
        return W.document_mask_bits(w, docs)
    if kind == "band":
        # each query allows only keys within 40 positions behind it: most of a
        # full causal row's tiles are empty
        m = np.zeros((w.total_q, max(w.lengths_k)), bool)
        for b in range(w.batch):
            q0, lq, lk = int(w.cu_seqlens_q()[b]), w.lengths_q[b], w.lengths_k[b]
            for i in range(lq):
                p = i + lk - lq
                m[q0 + i, max(0, p - 40):p + 1] = True
        return W.pack_mask(m, W.mask_row_words(max(w.lengths_k)))
    dens = 0.02 if kind == "random-sparse" else 0.6
    m = W.random_mask(w, dens, seed=seed, empty_rows=3)
    return W.pack_mask(m, W.mask_row_words(max(w.lengths_k)))


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[8]}-{c[7]}-d{c[4]}-w{c[5]}-{'c' if c[6] else 'nc'}")
def test_ranges_and_skipping(case):
    import torch
    lq, lk, hq, hkv, d, win, causal, dt, kind = case
    w = small_case(lq, lk, heads_q=hq, heads_kv=hkv, head_dim=d, window=win, causal=causal, dtype=dt,
                   do_scale=1.0 if dt == "f32" else 0.1, seed=71)
    H.say(f"mask-ranges case {case}")
    x = make_inputs(w)
    dev = H.to_device(w, x)
    bits = _mask_for(w, kind, 72)
    dmask = torch.from_numpy(bits.view(np.int32)).cuda()
    rng_dev = _ranges(w, dev, dmask)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(rng_dev.cpu().numpy(), expected_ranges(w, bits))
    plain = H.run_hip(w, dev, mask=dmask)
    skip = H.run_hip(w, dev, mask=dmask, mask_ranges=rng_dev)
    for key in plain:
        assert torch.equal(plain[key], skip[key]), key
    m = W.unpack_rows(bits, range(w.total_q), max(w.lengths_k))
    stats = H.compare_full(w, x, skip, mask=m, scale_f32=True)
    H.say("   ", {k: {a: f"{b:.2e}" for a, b in v.items()} for k, v in stats.items()})


def test_short_documents_32k_bitwise():
    """The 32K windowed workload packed from documents of at most 512 tokens:
    with the ranges, bitwise the same outputs as without."""
    import torch
    w = W.SWA_32K
    x = make_inputs(w)
    dev = H.to_device(w, x)
    docs = W.short_document_lengths(92, w.lengths_k[0], 512)
    bits = W.document_mask_bits(w, [docs])
    dmask = torch.from_numpy(bits.view(np.int32)).cuda()
    H.say(f"32K short documents: {len(docs)} documents, longest {max(docs)}")
    rng_dev = _ranges(w, dev, dmask)
    plain = H.run_hip(w, dev, mask=dmask)
    skip = H.run_hip(w, dev, mask=dmask, mask_ranges=rng_dev)
    for key in plain:
        assert torch.equal(plain[key], skip[key]), key
