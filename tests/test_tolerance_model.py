"""The stored-O allowance of the 16-bit dQ / dK bars (gpu_helpers.
stored_o_allowance), checked on the host against a direct recomputation.

dS = P (dP - D) is linear in D, so the allowance's first-order error is the
exact change of dQ and dK when D is formed from O rounded to the I/O dtype.
Here that change is computed independently, per sequence and head, with dense
numpy matrices and D taken from the rounded O, and compared with half the
allowance (the allowance is twice the model error).
"""
import numpy as np
import pytest

import gpu_helpers as H
import sliding_window_flash_amd.workloads as W
from sliding_window_flash_amd.workloads import make_inputs, small_case


def _direct(w, x, mask):
    """dQ and dK from D of the rounded O, and from D of the exact O."""
    q, k, v, do = (x[n].astype(np.float64) for n in ("q", "k", "v", "do"))
    cq, ck = x["cu_q"], x["cu_k"]
    grp = w.heads_q // w.heads_kv
    out = {}
    for tag in ("exact", "rounded"):
        dq = np.zeros_like(q)
        dk = np.zeros_like(k)
        for b in range(w.batch):
            q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
            lq, lk = q1 - q0, k1 - k0
            vis = np.zeros((lq, lk), bool)
            for i in range(lq):
                p = i + lk - lq
                for j in range(lk):
                    vis[i, j] = (j <= p and p - j < w.window) if w.causal else abs(p - j) < w.window
            if mask is not None:
                vis &= mask[q0:q1, :lk]
            for h in range(w.heads_q):
                g = h // grp
                s = w.scale * q[q0:q1, h] @ k[k0:k1, g].T
                s[~vis] = -np.inf
                mx = s.max(1, keepdims=True)
                mx[~np.isfinite(mx)] = 0.0
                e = np.exp(s - mx)
                den = e.sum(1, keepdims=True)
                pm = np.divide(e, den, out=np.zeros_like(e), where=den > 0)
                o = pm @ v[k0:k1, g]
                if tag == "rounded":
                    o = W._round_16(o.astype(np.float32), w.dtype).astype(np.float64)
                dd = (do[q0:q1, h] * o).sum(1, keepdims=True)
                ds = pm * (do[q0:q1, h] @ v[k0:k1, g].T - dd)
                dq[q0:q1, h] = w.scale * ds @ k[k0:k1, g]
                dk[k0:k1, g] += w.scale * ds.T @ q[q0:q1, h]
        out[tag] = dict(dq=dq, dk=dk)
    return out


CASES = [
    # (lengths_q, lengths_k, heads_q, heads_kv, head_dim, window, causal, dtype, mask density)
    ([2], None, 1, 1, 64, 300, False, "bf16", None),
    ([37, 5], [40, 9], 4, 2, 64, 7, True, "bf16", 0.6),
    ([23], None, 3, 1, 32, 1000, False, "fp16", 0.4),
    ([50], None, 2, 2, 64, 16, True, "bf16", None),
]


@pytest.mark.parametrize("case", CASES)
def test_allowance_is_twice_the_exact_change(case):
    lq, lk, hq, hkv, d, win, causal, dt, dens = case
    w = small_case(lq, lk, heads_q=hq, heads_kv=hkv, head_dim=d, window=win, causal=causal, dtype=dt,
                   do_scale=0.1, seed=17)
    x = make_inputs(w)
    mask = None if dens is None else W.random_mask(w, dens, seed=18, empty_rows=1)
    ref = H.full_reference(w, x, None, mask)
    allow = H.stored_o_allowance(w, x, ref, None, mask)
    direct = _direct(w, x, mask)
    for key in ("dq", "dk"):
        # the direct exact-O results are the oracle's (up to summation order)
        np.testing.assert_allclose(direct["exact"][key], ref[key], rtol=1e-9, atol=1e-12)
        change = np.linalg.norm(direct["rounded"][key] - direct["exact"][key]) / np.linalg.norm(ref[key])
        assert allow[key] == pytest.approx(2.0 * change, rel=1e-6, abs=1e-15), key


def test_allowance_vanishes_when_o_is_representable():
    """Window 1 with every row seeing only itself: O = V exactly, so rounding
    O changes nothing and the allowance is zero."""
    w = small_case([30], None, heads_q=2, heads_kv=1, head_dim=64, window=1, causal=True, dtype="bf16",
                   do_scale=0.1, seed=19)
    x = make_inputs(w)
    ref = H.full_reference(w, x)
    allow = H.stored_o_allowance(w, x, ref)
    assert allow["dq"] < 1e-12 and allow["dk"] < 1e-12
