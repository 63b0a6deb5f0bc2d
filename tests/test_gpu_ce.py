"""The linear cross-entropy (ce_fwd / ce_bwd) against the fp64 oracle.

Forward outputs (loss, LSE, target logit) are fp32 sums over bf16/fp16
inputs with fp32 accumulation: the bar is max-abs 1e-4 (fp32 rounding over a
4,096-term dot product and a 151,936-term exponential sum stays near 1e-5).
dH is written in the I/O type from dz rounded to it as an MFMA operand, so it
takes the attention outputs' bar for that type. Cases span several tiles with
ragged tails in tokens and vocabulary, several vocabulary chunks (a chunk
holds 16,384 words), a chunk narrower than one 64-word step, one token, targets
at both ends of the vocabulary, and the README's loss-layer shape on sampled
rows.
"""
import numpy as np
import pytest

import gpu_helpers as H
import sliding_window_flash_amd as swa
import sliding_window_flash_amd.workloads as W
from oracle import ce

pytestmark = pytest.mark.gpu

FWD_ABS = 1e-4

CASES = [
    # (n, vocab, hidden, dtype)
    (300, 1000, 256, "bf16"),
    (257, 513, 512, "fp16"),
    (64, 40000, 256, "bf16"),          # three vocabulary chunks
    (513, 16484, 256, "bf16"),         # a second chunk of 100 words
    (1, 7, 256, "fp16"),
    (130, 256, 768, "bf16"),
]


def _dev(x, dtype):
    import torch
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    return (torch.from_numpy(x["h"]).to(dt).cuda(), torch.from_numpy(x["w"]).to(dt).cuda(),
            torch.from_numpy(x["targets"]).cuda(), torch.from_numpy(x["dnll"]).cuda())


def _check(name, got, ref, dtype, rows=None):
    for key in ("nll", "lse", "tgt"):
        err = float(np.max(np.abs(H.host64(got[key]) - ref[key]), initial=0.0))
        assert err <= FWD_ABS, f"{name} {key}: max abs {err}"
    return H.compare(f"{name} dH", H.host64(got["dh"]), ref["dh"], dtype)


@pytest.mark.parametrize("n,vocab,hidden,dtype", CASES)
def test_ce_full_oracle(n, vocab, hidden, dtype):
    w = W.CEWorkload(f"ce_{n}_{vocab}_{hidden}", n, vocab, hidden, dtype, 40 + n % 7)
    H.say(f"ce case {w}")
    x = W.make_ce_inputs(w)
    x["targets"][0] = 0
    x["targets"][-1] = vocab - 1
    h, wt, tg, g = _dev(x, dtype)
    nll, lse, tgt = swa.ce_fwd(h, wt, tg)
    dh = swa.ce_bwd(h, wt, tg, lse, g)
    ref = ce.ce_reference(x["h"], x["w"], x["targets"], x["dnll"])
    stats = _check(w.name, dict(nll=nll, lse=lse, tgt=tgt, dh=dh), ref, dtype)
    H.say("   dH", {k: f"{v:.2e}" for k, v in stats.items()})


def test_ce_no_tokens():
    import torch
    h = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    wt = torch.randn((100, 256), device="cuda").to(torch.bfloat16)
    tg = torch.empty(0, dtype=torch.int32, device="cuda")
    nll, lse, tgt = swa.ce_fwd(h, wt, tg)
    dh = swa.ce_bwd(h, wt, tg, lse, torch.empty(0, device="cuda"))
    assert nll.numel() == 0 and dh.shape == (0, 256)


def test_ce_target_out_of_range_is_nan():
    w = W.CEWorkload("ce_bad_target", 40, 300, 256, "bf16", 3)
    x = W.make_ce_inputs(w)
    x["targets"][5] = 300
    x["targets"][6] = -1
    h, wt, tg, g = _dev(x, "bf16")
    nll, lse, tgt = swa.ce_fwd(h, wt, tg)
    bad = np.isnan(H.host64(nll))
    assert bad[5] and bad[6] and bad.sum() == 2
    assert np.all(np.isfinite(H.host64(lse)))


def test_ce_bench_shape_sampled():
    """The README's loss-layer shape (n 8,192, V 151,936, hidden 4,096, bf16),
    all outputs of sampled tokens against the oracle."""
    w = W.CE_BENCH
    x = W.make_ce_inputs(w)
    h, wt, tg, g = _dev(x, "bf16")
    nll, lse, tgt = swa.ce_fwd(h, wt, tg)
    dh = swa.ce_bwd(h, wt, tg, lse, g)
    rows = np.array([0, 1, 255, 256, 4097, 8191], np.int64)
    ref = ce.ce_reference(x["h"], x["w"], x["targets"], x["dnll"][rows], rows=rows)
    got = {k: v[H.index_tensor(rows)] for k, v in dict(nll=nll, lse=lse, tgt=tgt, dh=dh).items()}
    stats = _check(w.name, got, ref, "bf16")
    H.say("   dH sampled", {k: f"{v:.2e}" for k, v in stats.items()})
    assert np.all(np.isfinite(H.host64(nll)))
