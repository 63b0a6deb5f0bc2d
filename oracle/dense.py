"""Dense fp64 reference: the plain definition of windowed attention and its VJP.

TEST INFRASTRUCTURE ONLY (see the package header): never imported by the
product path.

What is computed, per packed sequence b, query head h (KV head g = h // G with
G = Hq / Hkv), query row i and key j:

  visibility   "Off NVIDIA, you fix the platform yourself" (labs.layer2c.com),
               section "What was broken?": under the sliding-window rule a
               token sees only the most recent tokens before it; under the
               plain causal rule it sees every earlier token. Reading used:
               query i sits at key position p = i + (L_k - L_q) (queries are
               the last L_q positions; the lab's "Method and disclosure"
               section has key tiles left unvisited when there are fewer
               queries than keys, which needs that alignment). Cell (i, j) is
               visible iff j <= p and p - j < w: w keys counting the token
               itself, so w = 1 sees only itself (the record entry "Gradient
               parity, small shapes": at window 1 the true gradient is zero).
               Without the causal mask (the same entry sweeps windows "causal
               and not"), the window is two-sided: visible iff |p - j| < w, so
               w = 1 again sees only the token itself and any w >=
               max(L_q, L_k) sees every key (plain non-causal attention).
               With more queries than keys the first L_q - L_k positions are
               negative and the same rules apply as written.
  forward      s_ij = scale * q_i . k_j on visible cells, -inf elsewhere;
               LSE_i = log sum_j exp(s_ij) (natural log); P_ij = exp(s_ij - LSE_i);
               O_i = sum_j P_ij v_j. The saved state is O and LSE (mlx-train-perf
               README, flash-attention passage: the flash path keeps the
               attention output and the log-sum-exp, O(N) state).
  backward     the vector-Jacobian product of the loss L = sum(O * dO):
               dP_ij = dO_i . v_j, D_i = dO_i . O_i, dS_ij = P_ij (dP_ij - D_i),
               dQ_i = scale sum_j dS_ij k_j,
               dK_j = scale sum_{h in group} sum_i dS_ij q_i,
               dV_j = sum_{h in group} sum_i P_ij dO_i.
               (The lab's "What did fixing it take?" section: the backward
               must give every query and key its gradient, including key
               blocks no query visits, whose gradient is zero.)
  empty rows   a query with no visible key gets O = 0, LSE = -inf, dQ = 0
               (without a mask only when L_q > L_k: a causal query at a
               negative position, or a two-sided one more than w - 1 before
               key 0).
  mask         optional, combined with the window. The lab's "What's not
               proved" list says a window combined with an arbitrary mask still
               falls back to the full score matrix in training; its record
               entry on backward memory measures against the boolean mask that
               mlx-lm passes. Reading used: the arbitrary mask is such a
               boolean matrix, one per sequence and shared by every head, and
               a cell is visible iff the window shows it AND the mask allows
               it. Here ``mask`` is boolean [T_q, W] with W >= every L_k: row
               t is packed query token t, column j is key j of that token's
               sequence (0-based within the sequence); columns past L_k are
               ignored.

The full L_q x L_k masked matrix is built for each (sequence, head), a panel of
at most ``panel_rows`` query rows at a time, so memory stays bounded while
nothing is tiled along keys. The mask comes from arange comparisons.
"""
from __future__ import annotations

import os
from typing import Iterable, Optional

import numpy as np

F64 = np.float64


class HostRamExceeded(MemoryError):
    """Raised before an allocation that would exceed the host-RAM ceiling."""


CUSHION_BYTES = 2 << 30


def available_host_bytes() -> int:
    """MemAvailable from /proc/meminfo (bytes); a large number if unreadable."""
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemAvailable:"):
                    return int(line.split()[1]) * 1024
    except OSError:
        pass
    return 1 << 62


def check_host_ram(nbytes: int, ceiling: Optional[int] = None) -> None:
    """Refuse up front, rather than thrash, if ``nbytes`` exceeds the ceiling.

    The ceiling defaults to what the machine has available minus a 2 GiB
    cushion (the mlx-train-perf README's memory-guard passage sets its ceiling
    from the machine's own free memory minus such a cushion).
    """
    if ceiling is None:
        ceiling = available_host_bytes() - CUSHION_BYTES
    if nbytes > ceiling:
        raise HostRamExceeded(
            f"oracle step needs {nbytes} bytes of host RAM, ceiling is {ceiling}")


def visible_cells(lq: int, lk: int, window: int, causal: bool,
                  rows: Optional[np.ndarray] = None, allowed: Optional[np.ndarray] = None,
                  cols: Optional[tuple] = None) -> np.ndarray:
    """Boolean [len(rows), c1 - c0] mask of visible (query, key) cells over
    keys [c0, c1) = ``cols`` (default: all lk keys). ``allowed``, if given, is
    the caller's mask for these rows ([len(rows), >= lk])."""
    c0, c1 = (0, lk) if cols is None else cols
    i = np.arange(lq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    j = np.arange(c0, c1, dtype=np.int64)
    pos = (i + (lk - lq))[:, None]
    if not causal:
        vis = np.abs(pos - j[None, :]) < window
    else:
        vis = (j[None, :] <= pos) & (pos - j[None, :] < window)
    if allowed is not None:
        vis = vis & np.asarray(allowed, dtype=bool)[:, c0:c1]
    return vis


def key_band(r0: int, r1: int, lq: int, lk: int, window: int, causal: bool) -> tuple:
    """Keys [c0, c1) outside which query rows [r0, r1) of one sequence see
    nothing: their positions run from p0 = r0 + (lk - lq) to p1 = r1 - 1 +
    (lk - lq), a causal row sees keys (p - window, p] and a two-sided row keys
    (p - window, p + window). Every cell outside the band is masked (-inf),
    so its exp is exactly 0 and it adds nothing to any sum: leaving it out
    changes no result beyond the order of the sums."""
    delta = lk - lq
    p0, p1 = r0 + delta, r1 - 1 + delta
    c0 = max(0, p0 - window + 1)
    c1 = min(lk, p1 + 1) if causal else min(lk, p1 + window)
    return c0, max(c0, c1)


def _mask_rows(mask, q0, rows):
    """The caller's mask rows for query rows ``rows`` of the sequence starting
    at packed token q0 (None without a mask)."""
    return None if mask is None else mask[q0 + np.asarray(rows, dtype=np.int64)]


def _panel(qh, kg, vg, doh, mask, scale, with_backward):
    """One panel of query rows against every key of the sequence (fp64)."""
    s = scale * (qh @ kg.T)
    s = np.where(mask, s, -np.inf)
    has_key = mask.any(axis=1)
    m = np.where(has_key, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.exp(s - m[:, None])                      # exp(-inf) = 0 on masked cells
    z = e.sum(axis=1)
    zs = np.where(has_key, z, 1.0)
    lse = np.where(has_key, m + np.log(zs), -np.inf)
    p = e / zs[:, None]
    o = p @ vg
    if not with_backward:
        return dict(p=p, o=o, lse=lse)
    dp = doh @ vg.T
    dlt = np.sum(doh * o, axis=1)
    ds = p * (dp - dlt[:, None])
    return dict(p=p, o=o, lse=lse, delta=dlt, ds=ds)


def _as64(a):
    return np.asarray(a, dtype=F64)


def _check_shapes(q, k, v, do, cu_q, cu_k):
    tq, hq, d = q.shape
    tk, hkv, dk = k.shape
    if v.shape != k.shape or dk != d or (do is not None and do.shape != q.shape):
        raise ValueError("shape mismatch")
    if hq % hkv:
        raise ValueError("heads_q must be a multiple of heads_kv")
    if len(cu_q) != len(cu_k) or cu_q[-1] != tq or cu_k[-1] != tk:
        raise ValueError("cu_seqlens do not match the packed tensors")
    return tq, tk, hq, hkv, d


def sdpa_reference(q, k, v, do, cu_q, cu_k, scale: float, window: int, causal: bool, *,
                   with_backward: bool = True, panel_rows: int = 512,
                   ram_ceiling: Optional[int] = None, heads: Optional[Iterable[int]] = None,
                   query_rows: Optional[tuple] = None, mask: Optional[np.ndarray] = None,
                   band: bool = False) -> dict:
    """Full forward (and backward) over a packed batch.

    q, do: [T_q, Hq, d]; k, v: [T_k, Hkv, d]; cu_q, cu_k: [B+1] offsets.
    Returns fp64 arrays: o [T_q, Hq, d], lse [Hq, T_q], and with the backward
    delta (= D) [Hq, T_q], dq [T_q, Hq, d], dk, dv [T_k, Hkv, d].

    ``heads`` and ``query_rows`` = (r0, r1) restrict the work to those query
    heads and to rows r0 <= i < r1 of every sequence (a timing sample; rows
    and heads left out stay at their initial values, and dK/dV then hold only
    the contributions of the rows computed). ``mask``: see the module header.
    ``band``: each panel takes only the keys of :func:`key_band` instead of all
    L_k keys (the cells left out are masked, so the result is the same up to
    summation order; at a window far below L_k it is far cheaper).
    """
    tq, tk, hq, hkv, d = _check_shapes(q, k, v, do if with_backward else None, cu_q, cu_k)
    grp = hq // hkv
    o = np.zeros((tq, hq, d), F64)
    lse = np.full((hq, tq), -np.inf, F64)
    out = dict(o=o, lse=lse)
    if with_backward:
        delta = np.zeros((hq, tq), F64)
        dq = np.zeros((tq, hq, d), F64)
        dk = np.zeros((tk, hkv, d), F64)
        dv = np.zeros((tk, hkv, d), F64)
        out.update(delta=delta, dq=dq, dk=dk, dv=dv)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        lq, lk = q1 - q0, k1 - k0
        if lq == 0:
            continue
        rows_per = max(1, min(panel_rows, lq))
        # ~8 panel-sized fp64 arrays live at once
        check_host_ram(8 * rows_per * max(lk, 1) * 8, ram_ceiling)
        row_lo, row_hi = (0, lq) if query_rows is None else (max(0, query_rows[0]),
                                                            min(lq, query_rows[1]))
        for h in (range(hq) if heads is None else heads):
            g = h // grp
            kg = _as64(k[k0:k1, g, :])
            vg = _as64(v[k0:k1, g, :])
            for r0 in range(row_lo, row_hi, rows_per):
                r1 = min(row_hi, r0 + rows_per)
                rr = np.arange(r0, r1)
                c0, c1 = key_band(r0, r1, lq, lk, window, causal) if band else (0, lk)
                vis = visible_cells(lq, lk, window, causal, rr, _mask_rows(mask, q0, rr), cols=(c0, c1))
                qh = _as64(q[q0 + r0:q0 + r1, h, :])
                doh = _as64(do[q0 + r0:q0 + r1, h, :]) if with_backward else None
                kb, vb = kg[c0:c1], vg[c0:c1]
                res = _panel(qh, kb, vb, doh, vis, scale, with_backward)
                o[q0 + r0:q0 + r1, h, :] = res["o"]
                lse[h, q0 + r0:q0 + r1] = res["lse"]
                if with_backward:
                    ds = res["ds"]
                    delta[h, q0 + r0:q0 + r1] = res["delta"]
                    dq[q0 + r0:q0 + r1, h, :] = scale * (ds @ kb)
                    dk[k0 + c0:k0 + c1, g, :] += scale * (ds.T @ qh)
                    dv[k0 + c0:k0 + c1, g, :] += res["p"].T @ doh
    return out


def _locate(cu, t):
    b = int(np.searchsorted(cu, t, side="right") - 1)
    return b, int(t - cu[b])


def sdpa_query_rows(q, k, v, do, cu_q, cu_k, scale, window, causal,
                    tokens: Iterable[int], heads: Iterable[int], mask: Optional[np.ndarray] = None) -> dict:
    """O, LSE, D and dQ for selected (packed query token, query head) rows.

    Each row is the same plain definition as :func:`sdpa_reference`, built as a
    one-row panel against all keys of its sequence.
    """
    _check_shapes(q, k, v, do, cu_q, cu_k)
    grp = q.shape[1] // k.shape[1]
    res = dict(o=[], lse=[], delta=[], dq=[])
    for t, h in zip(tokens, heads):
        b, i = _locate(cu_q, t)
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        lq = int(cu_q[b + 1] - cu_q[b])
        g = h // grp
        kg, vg = _as64(k[k0:k1, g, :]), _as64(v[k0:k1, g, :])
        vis = visible_cells(lq, k1 - k0, window, causal, np.array([i]),
                            _mask_rows(mask, int(cu_q[b]), [i]))
        r = _panel(_as64(q[t:t + 1, h, :]), kg, vg, _as64(do[t:t + 1, h, :]), vis, scale, True)
        res["o"].append(r["o"][0])
        res["lse"].append(r["lse"][0])
        res["delta"].append(r["delta"][0])
        res["dq"].append(scale * (r["ds"] @ kg)[0])
    return {key: np.array(val) for key, val in res.items()}


def sdpa_key_rows(q, k, v, do, cu_q, cu_k, scale, window, causal,
                  tokens: Iterable[int], kv_heads: Iterable[int], *,
                  panel_rows: int = 512, mask: Optional[np.ndarray] = None) -> dict:
    """dK and dV for selected (packed key token, KV head) rows.

    Every query row that sees the key is rebuilt in full (its whole masked
    score row), so its P and dS come from the same definition as above.
    """
    _check_shapes(q, k, v, do, cu_q, cu_k)
    grp = q.shape[1] // k.shape[1]
    res = dict(dk=[], dv=[])
    for t, g in zip(tokens, kv_heads):
        b, j = _locate(cu_k, t)
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        lq, lk = q1 - q0, k1 - k0
        kg, vg = _as64(k[k0:k1, g, :]), _as64(v[k0:k1, g, :])
        # The column of the visibility matrix for key j, built 1024 rows at a
        # time over the rows whose position p = i + (L_k - L_q) the window lets
        # reach j (j <= p < j + w causal, |p - j| < w two-sided); every other
        # row's cell is masked by the window itself.
        shift = lk - lq
        lo = j - shift if causal else j - shift - window + 1
        hi = j - shift + window - 1
        lo, hi = max(0, lo), min(lq - 1, hi)
        col = np.concatenate([
            visible_cells(lq, lk, window, causal, np.arange(r, min(hi + 1, r + 1024)),
                          _mask_rows(mask, q0, np.arange(r, min(hi + 1, r + 1024))))[:, j]
            for r in range(lo, hi + 1, 1024)]) if hi >= lo else np.zeros(0, bool)
        rows = lo + np.nonzero(col)[0]
        dk_j = np.zeros(k.shape[2], F64)
        dv_j = np.zeros(k.shape[2], F64)
        for h in range(g * grp, (g + 1) * grp):
            for r0 in range(0, rows.size, panel_rows):
                rr = rows[r0:r0 + panel_rows]
                vis = visible_cells(lq, lk, window, causal, rr, _mask_rows(mask, q0, rr))
                qh = _as64(q[q0 + rr, h, :])
                doh = _as64(do[q0 + rr, h, :])
                r = _panel(qh, kg, vg, doh, vis, scale, True)
                dk_j += scale * (r["ds"][:, j] @ qh)
                dv_j += r["p"][:, j] @ doh
        res["dk"].append(dk_j)
        res["dv"].append(dv_j)
    return {key: np.array(val) for key, val in res.items()}


def oracle_threads() -> int:
    """Host cores this process may use (what BLAS is asked to use)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1
