"""Whole-tensor parity at the full measured sizes, in the launch configuration
bench.py times: every element of O, LSE and dQ for the query heads of a chunk
of KV groups, and of dK and dV for those KV heads, against the fp64 oracle.

The chunks together cover every head of the 8K causal, 32K windowed and
ragged 4-sequence workloads and of the head_dim 256 memory-probe shape; the
ragged batch's window sweep covers KV groups 0 and Hkv - 1. The oracle takes
each row panel against the key band that can be visible to it (the cells
outside are masked and add exactly zero), which keeps a full-size head to
about a second on the host.
"""
import numpy as np
import pytest

import gpu_helpers as H
from oracle import dense
from sliding_window_flash_amd import workloads as W
from sliding_window_flash_amd.workloads import make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


_CACHE = {}


def _run(w):
    """Inputs and host fp64 copies of every GPU output for workload w (the
    latest workload only is kept)."""
    if w not in _CACHE:
        _CACHE.clear()
        H.say(f"case {w.name} window={w.window}: full-size run")
        x = make_inputs(w)
        got = H.run_hip(w, H.to_device(w, x))
        _CACHE[w] = (x, {k: H.host64(v) for k, v in got.items()})
        import torch
        del got
        torch.cuda.empty_cache()
    return _CACHE[w]


def _chunks(w, n_chunks):
    per = max(1, w.heads_kv // n_chunks)
    return [(g0, min(w.heads_kv, g0 + per)) for g0 in range(0, w.heads_kv, per)]


def _check(w, g0, g1, zero=()):
    x, got = _run(w)
    grp = w.heads_q // w.heads_kv
    heads = list(range(g0 * grp, g1 * grp))
    ref = dense.sdpa_reference(x["q"], x["k"], x["v"], x["do"], x["cu_q"], x["cu_k"], w.scale, w.window,
                               w.causal, heads=heads, band=True)
    hs, gs = slice(g0 * grp, g1 * grp), slice(g0, g1)
    stats = {
        "o": H.compare(f"{w.name} O heads {heads[0]}-{heads[-1]}", got["o"][:, hs], ref["o"][:, hs], w.dtype),
        "lse": H.compare(f"{w.name} LSE heads {heads[0]}-{heads[-1]}", got["lse"][hs], ref["lse"][hs], w.dtype),
        "dq": H.compare(f"{w.name} dQ heads {heads[0]}-{heads[-1]}", got["dq"][:, hs], ref["dq"][:, hs], w.dtype,
                        zero_ref="dq" in zero),
        "dk": H.compare(f"{w.name} dK kv heads {g0}-{g1 - 1}", got["dk"][:, gs], ref["dk"][:, gs], w.dtype,
                        zero_ref="dk" in zero),
        "dv": H.compare(f"{w.name} dV kv heads {g0}-{g1 - 1}", got["dv"][:, gs], ref["dv"][:, gs], w.dtype),
    }
    H.say(f"  {w.name} w={w.window} kv heads {g0}-{g1 - 1}:",
          {k: {kk: f"{vv:.2e}" for kk, vv in v.items()} for k, v in stats.items()})


FULL = [(wl, c) for wl in (W.CAUSAL_8K, W.SWA_32K, W.VARLEN_4, W.GEMMA_32K) for c in _chunks(wl, 4)]


@pytest.mark.parametrize("w,chunk", FULL, ids=lambda v: v.name if hasattr(v, "name") else f"kv{v[0]}-{v[1] - 1}")
def test_whole_heads(w, chunk):
    _check(w, *chunk)


SWEEP = [(W.VARLEN_4.replace(window=win), c) for win in W.VARLEN_SWEEP_WINDOWS
         for c in ((0, 1), (W.VARLEN_4.heads_kv - 1, W.VARLEN_4.heads_kv))]


@pytest.mark.parametrize("w,chunk", SWEEP,
                         ids=lambda v: f"w{v.window}" if hasattr(v, "name") else f"kv{v[0]}-{v[1] - 1}")
def test_varlen_window_sweep_whole_heads(w, chunk):
    # window 1: each query sees only itself, so the exact dQ and dK are zero
    # and only rounding is left
    _check(w, *chunk, zero=("dq", "dk") if w.window == 1 else ())


# The 32K windowed workload with its tokens packed from documents (a
# block-diagonal mask combined with the window): corpus-like documents, and
# documents of at most 512 tokens run with the mask's tile ranges (the tiles
# the mask empties are skipped). Every element of KV groups 0 and Hkv - 1.
_MCACHE = {}


def _run_masked(kind):
    import torch
    if kind not in _MCACHE:
        _MCACHE.clear()
        w = W.SWA_32K
        docs = (W.document_lengths(91, w.lengths_k[0]) if kind == "documents"
                else W.short_document_lengths(92, w.lengths_k[0], 512))
        bits = W.document_mask_bits(w, [docs])
        H.say(f"case {w.name} {kind}: {len(docs)} documents, full-size run")
        x = make_inputs(w)
        dev = H.to_device(w, x)
        dmask = torch.from_numpy(bits.view(np.int32)).cuda()
        kw = dict(max_seqlen_q=w.max_seqlen_q, max_seqlen_k=w.max_seqlen_k, window=w.window, causal=w.causal,
                  scale=w.scale)
        ranges = None
        if kind == "short":
            import sliding_window_flash_amd as swa
            ranges = swa.mask_ranges(dev["q"], dev["k"], dev["cu_q"], dev["cu_k"], dmask, **kw)
        got = H.run_hip(w, dev, mask=dmask, mask_ranges=ranges)
        _MCACHE[kind] = (w, x, {k: H.host64(v) for k, v in got.items()}, W.PackedMaskRows(bits, w.lengths_k[0]))
        del got
        torch.cuda.empty_cache()
    return _MCACHE[kind]


@pytest.mark.parametrize("kind", ["documents", "short"])
@pytest.mark.parametrize("group", [0, 7])
def test_masked_documents_whole_heads(kind, group):
    w, x, got, view = _run_masked(kind)
    grp = w.heads_q // w.heads_kv
    heads = list(range(group * grp, (group + 1) * grp))
    ref = dense.sdpa_reference(x["q"], x["k"], x["v"], x["do"], x["cu_q"], x["cu_k"], w.scale, w.window,
                               w.causal, heads=heads, band=True, mask=view)
    hs, gs = slice(group * grp, (group + 1) * grp), slice(group, group + 1)
    stats = {
        "o": H.compare(f"{kind} O", got["o"][:, hs], ref["o"][:, hs], w.dtype),
        "lse": H.compare(f"{kind} LSE", got["lse"][hs], ref["lse"][hs], w.dtype),
        "dq": H.compare(f"{kind} dQ", got["dq"][:, hs], ref["dq"][:, hs], w.dtype),
        "dk": H.compare(f"{kind} dK", got["dk"][:, gs], ref["dk"][:, gs], w.dtype),
        "dv": H.compare(f"{kind} dV", got["dv"][:, gs], ref["dv"][:, gs], w.dtype),
    }
    H.say(f"  {kind} kv group {group}:", {k: {kk: f"{vv:.2e}" for kk, vv in v.items()} for k, v in stats.items()})
