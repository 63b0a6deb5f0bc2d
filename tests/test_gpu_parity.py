"""HIP path (through the C ABI) against the fp64 oracle, element by element.

Small cases span several tiles with ragged tails and compare every output
element with the full dense oracle; the measured workloads compare sampled
rows (computed one by one by the oracle) plus invariants that hold at any
size. Outputs and the workspace are NaN-poisoned before each call.
"""
import zlib

import numpy as np
import pytest

import gpu_helpers as H
import sliding_window_flash_amd as swa
from sliding_window_flash_amd import workloads as W
from sliding_window_flash_amd.workloads import INT32_MAX, make_inputs, small_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.say("device:", torch.cuda.get_device_name(0))


def _run_full(w, window=None, zero=()):
    H.say(f"case {w.name}: lengths_q={w.lengths_q} lengths_k={w.lengths_k} Hq={w.heads_q} "
          f"Hkv={w.heads_kv} d={w.head_dim} window={w.window if window is None else window} "
          f"causal={w.causal} dtype={w.dtype}")
    x = make_inputs(w)
    dev = H.to_device(w, x)
    got = H.run_hip(w, dev, window=window)
    stats = H.compare_full(w, x, got, window=window, zero=zero)
    H.say("  ", {k: {kk: f"{vv:.2e}" for kk, vv in v.items()} for k, v in stats.items()})
    return x, dev, got


def test_tiny_fp32_workload():
    _run_full(W.TINY_F32)


SMALL = [
    # lengths_q, lengths_k, Hq, Hkv, d, window, causal, dtype
    ([1024], None, 4, 2, 128, 32, True, "bf16"),            # first key tile is not tile 0
    ([1024], None, 2, 1, 64, 32, True, "f32"),
    ([300, 1, 517, 64], None, 8, 2, 128, 129, True, "bf16"),  # ragged tails, varlen
    ([300, 1, 517, 64], None, 8, 2, 128, 127, True, "bf16"),
    ([300, 1, 517, 64], None, 8, 2, 128, 128, True, "bf16"),
    ([300, 0, 517, 64], None, 4, 4, 128, INT32_MAX, True, "bf16"),  # empty sequence, MHA
    ([100, 40], [700, 300], 4, 1, 128, 16, True, "bf16"),   # L_q < L_k: unvisited key tiles
    ([100, 40], [700, 300], 2, 1, 64, 16, True, "f32"),
    ([200, 333], None, 4, 2, 128, INT32_MAX, False, "bf16"),  # full (non-causal)
    ([257], None, 2, 2, 128, 1000, True, "f32"),
    ([190, 70], None, 6, 3, 64, 50, True, "bf16"),
    ([300, 1, 517, 64], None, 8, 2, 128, 129, True, "fp16"),  # fp16: ragged, windowed
    ([100, 40], [700, 300], 4, 1, 64, 16, True, "fp16"),
    ([200, 333], None, 4, 2, 128, INT32_MAX, False, "fp16"),
    ([300, 1, 517, 64], None, 8, 4, 256, 129, True, "bf16"),  # head_dim 256: ragged, windowed
    ([100, 40], [700, 300], 4, 2, 256, 16, True, "fp16"),   # L_q < L_k at 256
    ([200, 333], None, 4, 2, 256, INT32_MAX, False, "bf16"),  # full attention at 256
    ([300, 1, 517, 64], None, 8, 2, 128, 65, False, "bf16"),  # two-sided windows
    ([100, 40], [700, 300], 4, 1, 64, 16, False, "f32"),
    ([257, 130], None, 4, 2, 256, 100, False, "fp16"),
    # head_dim 256 with odd KV groups: odd (head, query tile) step counts in the
    # two-pass dK/dV kernel (its stage order depends on the count's parity)
    ([300, 77], None, 3, 1, 256, 100, True, "bf16"),
    ([190, 64], None, 5, 5, 256, 33, False, "fp16"),
    ([200, 333], None, 4, 2, 128, 200, False, "f32"),
    # head_dim 512: output-column passes in the forward, dQ and dK/dV
    ([300, 1, 517, 64], None, 8, 2, 512, 129, True, "bf16"),
    ([100, 40], [700, 300], 4, 2, 512, 16, True, "fp16"),
    ([200, 333], None, 4, 2, 512, INT32_MAX, False, "bf16"),
    ([257, 130], None, 4, 2, 512, 100, False, "fp16"),
    ([300, 77], None, 3, 1, 512, 100, True, "bf16"),
    # more queries than keys: the first L_q - L_k rows sit at negative positions
    # (causal: no key at all; two-sided: a window of at least L_k but below L_q
    # is not full attention); a sequence with queries and no keys
    ([400, 90], [100, 300], 4, 2, 128, 64, True, "bf16"),
    ([400, 90], [100, 300], 4, 2, 128, 150, False, "bf16"),
    ([300, 77], [50, 80], 2, 1, 64, 60, False, "f32"),
    ([300, 77], [50, 80], 4, 2, 256, 100, False, "fp16"),
    ([257, 40], [60, 300], 4, 2, 512, 70, True, "bf16"),
    ([200, 50], [0, 80], 4, 2, 128, 30, True, "bf16"),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c[0]}-{c[1]}-{c[4]}-w{c[5]}-{c[7]}-{'c' if c[6] else 'nc'}")
def test_small_cases_full_oracle(case):
    lq, lk, hq, hkv, d, win, causal, dt = case
    w = small_case(lq, lk, heads_q=hq, heads_kv=hkv, head_dim=d, window=win, causal=causal,
                   dtype=dt, do_scale=1.0 if dt == "f32" else 0.1, seed=zlib.crc32(repr(case).encode()) % 1000)
    _run_full(w)


# Softmax scales away from 1/sqrt(d): near-uniform rows (0.02) and sharp ones
# (2 and 6: score ranges of hundreds in log2 units, so the running reference
# max moves often and most probabilities underflow to 0). dQ and dK carry the
# scale as a factor, so dO shrinks by the scale's ratio to 1/sqrt(d): the
# gradients stay of the size the absolute bars are set for (bf16 itself has a
# half unit of 0.016 at magnitude 4 and 0.03 at 8).
@pytest.mark.parametrize("dt,d,scale,causal", [
    ("bf16", 128, 0.02, True), ("bf16", 128, 2.0, True), ("bf16", 64, 6.0, False),
    ("fp16", 128, 2.0, True), ("f32", 64, 2.0, True), ("bf16", 256, 2.0, True), ("fp16", 512, 0.5, False),
])
def test_softmax_scales(dt, d, scale, causal):
    w = small_case([300, 77], [333, 77], heads_q=4, heads_kv=2, head_dim=d, window=100, causal=causal,
                   dtype=dt, scale=scale, do_scale=0.1 * min(1.0, d ** -0.5 / scale), seed=37)
    H.say(f"scale case: {dt} d={d} scale={scale} causal={causal}")
    x = make_inputs(w)
    got = H.run_hip(w, H.to_device(w, x))
    stats = H.compare_full(w, x, got, scale_f32=True)
    H.say("  ", {k: {kk: f"{vv:.2e}" for kk, vv in v.items()} for k, v in stats.items()})


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("fp16", 64), ("bf16", 256), ("f32", 64), ("fp16", 512)])
def test_window_one_closed_form(dt, d):
    w = small_case([300, 130], [300, 200], heads_q=4, heads_kv=2, head_dim=d, window=1, dtype=dt,
                   do_scale=0.1, seed=31)
    x, dev, got = _run_full(w, zero=("dq", "dk"))
    # each query sees only its own key: O = V. In bf16 and fp16 exactly (P
    # rounds to 1 and the normaliser sums the rounded P); in fp32 within an ulp
    # (P = 2^(s*c - m) with m the rounded s*c is 1 only up to rounding).
    o = H.host64(got["o"])
    for b in range(w.batch):
        q0, k0 = int(x["cu_q"][b]), int(x["cu_k"][b])
        lq, lk = w.lengths_q[b], w.lengths_k[b]
        kv = np.repeat(x["v"][k0 + lk - lq:k0 + lk], 2, axis=1).astype(np.float64)
        if dt in ("bf16", "fp16"):
            assert np.array_equal(o[q0:q0 + lq], kv)
        else:
            assert np.all(np.abs(o[q0:q0 + lq] - kv) <= 1e-6 * np.maximum(1.0, np.abs(kv)))


def test_two_sided_window_one_closed_form():
    w = small_case([300, 130], [300, 200], heads_q=4, heads_kv=2, head_dim=128, window=1, causal=False,
                   dtype="bf16", do_scale=0.1, seed=35)
    x, dev, got = _run_full(w, zero=("dq", "dk"))
    o = H.host64(got["o"])
    for b in range(w.batch):
        q0, k0 = int(x["cu_q"][b]), int(x["cu_k"][b])
        lq, lk = w.lengths_q[b], w.lengths_k[b]
        kv = np.repeat(x["v"][k0 + lk - lq:k0 + lk], 2, axis=1).astype(np.float64)
        assert np.array_equal(o[q0:q0 + lq], kv)


def test_wide_window_bitwise_equals_causal():
    w = small_case([700, 130], heads_q=4, heads_kv=2, head_dim=128, window=700, dtype="bf16",
                   do_scale=0.1, seed=32)
    x = make_inputs(w)
    dev = H.to_device(w, x)
    a = H.run_hip(w, dev)
    b = H.run_hip(w, dev, window=INT32_MAX)
    import torch
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_backward_is_deterministic():
    w = small_case([900, 300], heads_q=8, heads_kv=2, head_dim=128, window=200, dtype="bf16",
                   do_scale=0.1, seed=33)
    x = make_inputs(w)
    dev = H.to_device(w, x)
    a = H.run_hip(w, dev)
    b = H.run_hip(w, dev)
    import torch
    for key in a:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("order", ["delta-dkdv-dq", "dq-dkdv"])
@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f32", 64), ("fp16", 256), ("bf16", 512)])
def test_stages_run_separately(dt, d, order):
    """attn_bwd_stages one stage at a time against the oracle, on a workspace
    poisoned with NaN: the D preprocess as its own launch with dK/dV before dQ,
    and dQ alone forming D for the dK/dV launch after it (what attn_bwd does)."""
    import torch
    w = small_case([300, 77], [340, 77], heads_q=4, heads_kv=2, head_dim=d, window=90, dtype=dt,
                   do_scale=1.0 if dt == "f32" else 0.1, seed=36)
    x = make_inputs(w)
    dev = H.to_device(w, x)
    kw = dict(max_seqlen_q=w.max_seqlen_q, max_seqlen_k=w.max_seqlen_k, window=w.window, causal=w.causal,
              scale=w.scale)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o, lse = swa.fwd(q, k, v, dev["cu_q"], dev["cu_k"], **kw)
    dq, dk, dv = torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
    ws = torch.full((swa.workspace_bytes(swa.params_for(q, k, dev["cu_q"], dev["cu_k"], **kw)),), 255,
                    dtype=torch.uint8, device=q.device)
    stages = {"delta-dkdv-dq": (swa.BWD_DELTA, swa.BWD_DKDV, swa.BWD_DQ),
              "dq-dkdv": (swa.BWD_DQ, swa.BWD_DKDV)}[order]
    for stage in stages:
        swa.bwd(q, k, v, o, lse, do, dev["cu_q"], dev["cu_k"], dq=dq, dk=dk, dv=dv, workspace=ws, stages=stage, **kw)
    torch.cuda.synchronize()
    H.compare_full(w, x, dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv))


@pytest.mark.parametrize("dt,d,causal", [("bf16", 64, True), ("f32", 128, False), ("fp16", 256, True)])
def test_many_short_sequences(dt, d, causal):
    """300 packed sequences of 0 to 70 tokens (many empty, some with more
    queries than keys): the launch-id decode over a large batch, sequences
    that end inside a tile, and work items past a sequence's end."""
    rng = np.random.default_rng(41)
    lq = [0 if rng.random() < 0.2 else int(rng.integers(1, 71)) for _ in range(300)]
    lk = [max(0, q + int(rng.integers(-8, 30))) for q in lq]
    w = small_case(lq, lk, heads_q=4, heads_kv=2, head_dim=d, window=24, causal=causal, dtype=dt,
                   do_scale=1.0 if dt == "f32" else 0.1, seed=42)
    _run_full(w)


def test_gqa_2k_full_oracle():
    _run_full(W.GQA_2K)


def _invariants(w, x, got):
    """Shifting every key leaves each softmax row unchanged, so sum_j dK_j = 0;
    shifting every value shifts O, so sum_j dV_j = the group's sum of dO (per
    sequence and KV head). Checked in fp64 on the GPU outputs: the residual
    must be small against the norm of the summed column, which is what a
    wrong gradient of random sign would leave."""
    dk, dv = H.host64(got["dk"]), H.host64(got["dv"])
    grp = w.heads_q // w.heads_kv
    for b in range(w.batch):
        k0, k1 = int(x["cu_k"][b]), int(x["cu_k"][b + 1])
        q0, q1 = int(x["cu_q"][b]), int(x["cu_q"][b + 1])
        if q1 == q0:
            continue
        for g in range(w.heads_kv):
            want = x["do"][q0:q1, g * grp:(g + 1) * grp].astype(np.float64).sum((0, 1))
            sv = dv[k0:k1, g].sum(0)
            nv = np.linalg.norm(dv[k0:k1, g], axis=0)
            assert np.all(np.abs(sv - want) <= 0.05 * nv + 1e-6), (b, g)
            sk = dk[k0:k1, g].sum(0)
            nk = np.linalg.norm(dk[k0:k1, g], axis=0)
            assert np.all(np.abs(sk) <= 0.05 * nk + 1e-6), (b, g)


@pytest.mark.parametrize("w", [W.CAUSAL_8K, W.SWA_32K, W.VARLEN_4, W.GEMMA_32K], ids=lambda w: w.name)
def test_measured_workloads_sampled(w):
    H.say(f"case {w.name}: sampled rows at full size")
    x = make_inputs(w)
    dev = H.to_device(w, x)
    got = H.run_hip(w, dev)
    stats = H.compare_sampled(w, x, got, n_q=4, n_k=2, seed=w.seed)
    H.say("  ", {k: {kk: f"{vv:.2e}" for kk, vv in v.items()} for k, v in stats.items()})
    _invariants(w, x, got)


def test_tensors_past_2gib_sampled():
    """Two sequences of 150,000 and 150,001 tokens, 32 query / 8 KV heads,
    head_dim 128, window 1,024: Q, O, dO and dQ are 2.46 GB each, so the
    second sequence's rows lie past 2^31 bytes into them. Sampled rows of both
    sequences against the oracle."""
    w = W.SWA_32K.replace(name="bf16_2x150k_w1024_32q8kv_d128", lengths_q=(150000, 150001),
                          lengths_k=(150000, 150001), seed=12)
    assert w.total_q * w.heads_q * w.head_dim * 2 > 2 ** 31
    H.say(f"case {w.name}: sampled rows, tensors past 2 GiB")
    x = make_inputs(w)
    dev = H.to_device(w, x)
    got = H.run_hip(w, dev)
    stats = H.compare_sampled(w, x, got, n_q=4, n_k=2, seed=w.seed)
    H.say("  ", {k: {kk: f"{vv:.2e}" for kk, vv in v.items()} for k, v in stats.items()})


@pytest.mark.parametrize("window", W.VARLEN_SWEEP_WINDOWS)
def test_varlen_window_sweep(window):
    w = W.VARLEN_4.replace(window=window)
    H.say(f"case varlen sweep window={window}")
    x = make_inputs(w)
    dev = H.to_device(w, x)
    got = H.run_hip(w, dev)
    if window == 1:
        o = H.host64(got["o"])
        assert np.array_equal(o, np.repeat(x["v"], 4, axis=1).astype(np.float64))
        assert float(np.abs(H.host64(got["dq"])).max()) <= H.ZERO_REF_ABS["bf16"]
        assert float(np.abs(H.host64(got["dk"])).max()) <= H.ZERO_REF_ABS["bf16"]
    else:
        stats = H.compare_sampled(w, x, got, n_q=2, n_k=1, seed=window)
        H.say("  ", {k: {kk: f"{vv:.2e}" for kk, vv in v.items()} for k, v in stats.items()})
    if window == max(w.lengths_k):
        other = H.run_hip(w, dev, window=INT32_MAX)
        import torch
        for key in got:
            assert torch.equal(got[key], other[key]), key
