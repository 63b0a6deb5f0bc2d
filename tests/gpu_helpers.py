"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
(via the binding) and compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np

import sliding_window_flash_amd as swa
from oracle import dense
from sliding_window_flash_amd.workloads import Workload

# Tolerances: fp32 max-abs 1e-5; bf16 max-abs 2e-2 and relative Frobenius 1e-2.
# fp16 rounds at 2^-11 instead of bf16's 2^-9 (inputs, P and dS as operands,
# outputs), so its bar is a quarter of bf16's.
F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_FRO = 1e-2
FP16_MAX_ABS = BF16_MAX_ABS / 4
FP16_REL_FRO = BF16_REL_FRO / 4
# The fp32 bar is stated for outputs of order one (the fp32 configuration).
# fp32 rounding is relative, so the random sweeps, whose grouped heads and
# longer rows give outputs up to ~10, apply it relative to the output's largest
# magnitude: max-abs <= 1e-5 * max(1, max |ref|) (scale_f32=True).
# Where the exact result is identically zero (window 1: dQ, dK; scale 0), only
# rounding is left; the bar is max-abs 1e-4 in bf16 and 1e-6 in fp32.
ZERO_REF_ABS = {"bf16": 1e-4, "fp16": 1e-4, "f32": 1e-6}
# The backward forms D = rowsum(dO * O) from the stored O (the forward's
# output, in the I/O dtype); the oracle forms it from its exact O. Where a
# row's D lies close to the dP of its visible keys, dS = P (dP - D) cancels and
# that rounding of O dominates dQ and dK. compare_full adds to their relative
# Frobenius bar twice the first-order error the rounding causes, computed from
# the oracle's own values (stored_o_allowance); elsewhere it is far below the
# bar and changes nothing.


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def torch_dtype(w: Workload):
    import torch
    return {"bf16": torch.bfloat16, "fp16": torch.float16}.get(w.dtype, torch.float32)


def to_device(w: Workload, x: dict) -> dict:
    import torch
    dt = torch_dtype(w)
    out = {k: torch.from_numpy(x[k]).to(dt).cuda() for k in ("q", "k", "v", "do")}
    out["cu_q"] = torch.from_numpy(x["cu_q"]).cuda()
    out["cu_k"] = torch.from_numpy(x["cu_k"]).cuda()
    return out


def run_hip(w: Workload, dev: dict, *, window=None, poison=True, with_backward=True, mask=None,
            mask_ranges=None) -> dict:
    """Forward then backward through the C ABI. Outputs and workspace are
    filled with NaN first, so any element the kernels fail to write shows.
    ``mask``: packed mask rows on the device (the masked entry points);
    ``mask_ranges``: the ranges attn_mask_ranges wrote for it."""
    import torch
    window = w.window if window is None else window
    kw = dict(max_seqlen_q=w.max_seqlen_q, max_seqlen_k=w.max_seqlen_k, window=window,
              causal=w.causal, scale=w.scale)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    if poison:
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
    o, lse = swa.fwd(q, k, v, dev["cu_q"], dev["cu_k"], out=o, lse=lse, mask=mask, mask_ranges=mask_ranges, **kw)
    res = dict(o=o, lse=lse)
    if with_backward:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        p = swa.params_for(q, k, dev["cu_q"], dev["cu_k"], **kw)
        ws = torch.empty(swa.workspace_bytes(p), dtype=torch.uint8, device=q.device)
        if poison:
            for t in (dq, dk, dv):
                t.fill_(float("nan"))
            ws.fill_(0xFF)
        swa.bwd(q, k, v, o, lse, do, dev["cu_q"], dev["cu_k"], dq=dq, dk=dk, dv=dv, workspace=ws, mask=mask,
                mask_ranges=mask_ranges, **kw)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return res


def host64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def compare(name: str, got, ref, dtype: str, zero_ref: bool = False, scale_f32: bool = False,
            rel_allow: float = 0.0) -> dict:
    """``rel_allow``: added to the 16-bit relative Frobenius bar (see
    stored_o_allowance)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{name}: non-finite pattern differs (unwritten output?)"
    diff = np.abs(got[fin] - ref[fin])
    max_abs = float(diff.max(initial=0.0))
    nrm = float(np.linalg.norm(ref[fin]))
    rel = float(np.linalg.norm(got[fin] - ref[fin]) / nrm) if nrm > 0 else 0.0
    stats = dict(max_abs=max_abs, rel_fro=rel)
    if zero_ref:
        assert max_abs <= ZERO_REF_ABS[dtype], f"{name}: {stats} (zero reference)"
    elif dtype == "f32":
        bar = F32_MAX_ABS * (max(1.0, float(np.abs(ref[fin]).max(initial=0.0))) if scale_f32 else 1.0)
        if scale_f32:
            say(f"  {name}: max-abs {max_abs:.2e} (scaled bar {bar:.2e}), rel-Fro {rel:.2e}")
        assert max_abs <= bar, f"{name}: {stats} (bar {bar:.2e})"
    else:
        bar_abs, bar_rel = (FP16_MAX_ABS, FP16_REL_FRO) if dtype == "fp16" else (BF16_MAX_ABS, BF16_REL_FRO)
        if rel_allow > 0.1 * bar_rel:
            say(f"  {name}: rel-Fro {rel:.2e}, bar {bar_rel:.1e} + stored-O allowance {rel_allow:.2e}")
        assert max_abs <= bar_abs and rel <= bar_rel + rel_allow, f"{name}: {stats} (allowance {rel_allow:.2e})"
    return stats


def full_reference(w: Workload, x: dict, window=None, mask=None) -> dict:
    """The whole oracle output; each row panel takes the key band that can be
    visible to it (the cells outside are masked and add exactly zero)."""
    window = w.window if window is None else window
    kw = {} if mask is None else dict(mask=mask)
    return dense.sdpa_reference(x["q"], x["k"], x["v"], x["do"], x["cu_q"], x["cu_k"], w.scale,
                                window, w.causal, band=True, **kw)


def stored_o_allowance(w: Workload, x: dict, ref: dict, window=None, mask=None) -> dict:
    """Twice the relative Frobenius error, to first order, that forming D from
    O rounded to the I/O dtype causes in dQ and dK, from the oracle's values.
    With dD = rowsum(dO * (round(O) - O)), dS = P (dP - D) moves by -P dD, so
    dQ moves by -scale dD (P K) and dK by -scale P^T (dD Q), summed over the
    group. P K is the oracle's forward with K as the values; P^T (dD Q) its dV
    with dD Q as the output gradient. Twice: the kernels' O also carries the
    forward's own rounding (P as a 16-bit operand), of the same order."""
    from sliding_window_flash_amd.workloads import _round_16
    window = w.window if window is None else window
    kw = {} if mask is None else dict(mask=mask)
    o = ref["o"]
    dd = ((_round_16(o.astype(np.float32), w.dtype).astype(np.float64) - o) * x["do"]).sum(-1)  # [T_q, Hq]
    common = (x["cu_q"], x["cu_k"], w.scale, window, w.causal)
    pk = dense.sdpa_reference(x["q"], x["k"], x["k"], x["do"], *common, with_backward=False, band=True, **kw)["o"]
    pdq = dense.sdpa_reference(x["q"], x["k"], x["v"], dd[..., None] * x["q"], *common, band=True, **kw)["dv"]
    out = {}
    for key, err in (("dq", w.scale * dd[..., None] * pk), ("dk", w.scale * pdq)):
        nrm = float(np.linalg.norm(ref[key]))
        out[key] = 2.0 * float(np.linalg.norm(err)) / nrm if nrm > 0 else 0.0
    return out


def compare_full(w: Workload, x: dict, got: dict, window=None, zero=(), mask=None, scale_f32=False) -> dict:
    """``mask``: the boolean mask rows (oracle side) when the run used one;
    ``scale_f32``: the fp32 bar relative to the output's largest magnitude.
    In bf16 and fp16 the dQ and dK bars take the stored-O allowance."""
    ref = full_reference(w, x, window, mask)
    allow = stored_o_allowance(w, x, ref, window, mask) if w.dtype in ("bf16", "fp16") and "dq" in got else {}
    out = {}
    for key in ("o", "lse", "dq", "dk", "dv"):
        if key in got:
            out[key] = compare(f"{w.name} {key}", host64(got[key]), ref[key], w.dtype,
                               zero_ref=key in zero, scale_f32=scale_f32, rel_allow=allow.get(key, 0.0))
    return out


def sample_rows(w: Workload, n_random: int, seed: int, tile: int = 128, few: bool = False):
    """Packed token indices: each sequence's first and last rows, rows around
    tile and window edges, and random rows (``few``: a smaller edge set)."""
    rng = np.random.default_rng(seed)
    toks = []
    for b in range(w.batch):
        start = int(sum(w.lengths_q[:b]))
        L = w.lengths_q[b]
        if L == 0:
            continue
        if few:
            cand = {0, L - 1, tile, w.window}
        else:
            cand = {0, 1, L - 1, L - 2, tile - 1, tile, w.window - 1, w.window, w.window + 1}
        cand |= set(int(c) for c in rng.integers(0, L, n_random))
        toks += [start + c for c in sorted(cand) if 0 <= c < L]
    return np.array(toks, np.int64)


def compare_sampled(w: Workload, x: dict, got: dict, n_q: int = 6, n_k: int = 3, seed: int = 0,
                    window=None, mask=None) -> dict:
    """Sampled query rows (O, LSE, dQ) and key rows (dK, dV) against the oracle
    computed one row at a time. ``mask``: boolean rows or a packed-row view."""
    window = w.window if window is None else window
    rng = np.random.default_rng(seed)
    args = (x["q"], x["k"], x["v"], x["do"], x["cu_q"], x["cu_k"], w.scale, window, w.causal)
    qt = sample_rows(w, n_q, seed)
    qh = rng.integers(0, w.heads_q, qt.size)
    rq = dense.sdpa_query_rows(*args, qt, qh, mask=mask)
    kt = sample_rows(w.replace(lengths_q=w.lengths_k), n_k, seed + 1, few=True)
    kh = rng.integers(0, w.heads_kv, kt.size)
    rk = dense.sdpa_key_rows(*args, kt, kh, mask=mask)

    def pick(t, i0, i1):
        return host64(t[index_tensor(i0), index_tensor(i1)])

    stats = {}
    stats["o"] = compare(f"{w.name} O rows", pick(got["o"], qt, qh), rq["o"], w.dtype)
    stats["lse"] = compare(f"{w.name} LSE rows", pick(got["lse"], qh, qt), rq["lse"], w.dtype)
    stats["dq"] = compare(f"{w.name} dQ rows", pick(got["dq"], qt, qh), rq["dq"], w.dtype)
    stats["dk"] = compare(f"{w.name} dK rows", pick(got["dk"], kt, kh), rk["dk"], w.dtype)
    stats["dv"] = compare(f"{w.name} dV rows", pick(got["dv"], kt, kh), rk["dv"], w.dtype)
    return stats


def index_tensor(a: np.ndarray):
    import torch
    return torch.from_numpy(np.asarray(a, np.int64)).cuda()
