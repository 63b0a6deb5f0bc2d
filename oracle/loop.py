"""Brute-force attention, one query at a time, in plain Python floats.

TEST INFRASTRUCTURE ONLY (see the package header). Independent of
``oracle.dense``: it shares no helper with it. It walks each query, lists the
keys it may see with explicit comparisons, and applies the softmax and its
vector-Jacobian product with ``math.fsum`` sums. Tiny shapes only.

Visibility, softmax, saved state and gradients are the same definitions as in
``oracle.dense`` (pages: "Off NVIDIA, you fix the platform yourself", sections
"What was broken?" and "What did fixing it take?"; the mlx-train-perf README's
flash-attention passage for the O + log-sum-exp saved state).
"""
from __future__ import annotations

import math

import numpy as np


def _dot(a, b):
    return math.fsum(x * y for x, y in zip(a, b))


def sdpa_loop(q, k, v, do, cu_q, cu_k, scale, window, causal, mask=None) -> dict:
    """``mask`` (optional): boolean [T_q, >= every L_k]; key j of the query at
    packed token t is visible only where mask[t][j] is true, on top of the
    window (the same reading as ``oracle.dense``)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    grp = hq // hkv
    o = np.zeros((tq, hq, d))
    lse = np.full((hq, tq), -math.inf)
    delta = np.zeros((hq, tq))
    dq = np.zeros((tq, hq, d))
    dk = [[[[] for _ in range(d)] for _ in range(hkv)] for _ in range(tk)]
    dv = [[[[] for _ in range(d)] for _ in range(hkv)] for _ in range(tk)]
    for b in range(len(cu_q) - 1):
        qa, qb, ka, kb = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        shift = (kb - ka) - (qb - qa)
        for h in range(hq):
            g = h // grp
            for i in range(qb - qa):
                me = i + shift
                keys = []
                for j in range(kb - ka):
                    if mask is not None and not mask[qa + i][j]:
                        continue
                    if causal:
                        if j <= me and me - j < window:
                            keys.append(j)
                    elif -window < me - j < window:  # two-sided window
                        keys.append(j)
                if not keys:
                    continue
                qi = q[qa + i, h]
                doi = do[qa + i, h]
                sc = [scale * _dot(qi, k[ka + j, g]) for j in keys]
                top = max(sc)
                lsum = top + math.log(math.fsum(math.exp(x - top) for x in sc))
                pr = [math.exp(x - lsum) for x in sc]
                oi = [math.fsum(pr[n] * v[ka + j, g, c] for n, j in enumerate(keys))
                      for c in range(d)]
                dd = _dot(doi, oi)
                dsc = [pr[n] * (_dot(doi, v[ka + j, g]) - dd) for n, j in enumerate(keys)]
                o[qa + i, h] = oi
                lse[h, qa + i] = lsum
                delta[h, qa + i] = dd
                for c in range(d):
                    dq[qa + i, h, c] = scale * math.fsum(
                        dsc[n] * k[ka + j, g, c] for n, j in enumerate(keys))
                for n, j in enumerate(keys):
                    for c in range(d):
                        dk[ka + j][g][c].append(scale * dsc[n] * qi[c])
                        dv[ka + j][g][c].append(pr[n] * doi[c])
    dk_arr = np.array([[[math.fsum(x) for x in row] for row in head] for head in dk]).reshape(tk, hkv, d)
    dv_arr = np.array([[[math.fsum(x) for x in row] for row in head] for head in dv]).reshape(tk, hkv, d)
    return dict(o=o, lse=lse, delta=delta, dq=dq, dk=dk_arr, dv=dv_arr)


def ce_loop(h, w, targets, dnll) -> dict:
    """Linear cross-entropy, one token at a time in plain Python floats: the
    logits h_i . w_v by explicit sums, the log-sum-exp over the vocabulary
    with the largest logit factored out, and dH_i = g_i (sum_v p_iv w_v -
    w_{y_i}) (the same definitions as ``oracle.ce``; the mlx-train-perf
    README's logit-free cross-entropy passage). Tiny shapes only."""
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    n, dim = h.shape
    vocab = w.shape[0]
    nll, lse, tgt = [], [], []
    dh = np.zeros((n, dim))
    for i in range(n):
        z = [_dot(h[i], w[v]) for v in range(vocab)]
        top = max(z)
        ls = top + math.log(math.fsum(math.exp(x - top) for x in z))
        y = int(targets[i])
        lse.append(ls)
        tgt.append(z[y])
        nll.append(ls - z[y])
        p = [math.exp(x - ls) for x in z]
        for c in range(dim):
            dh[i, c] = float(dnll[i]) * (math.fsum(p[v] * w[v, c] for v in range(vocab)) - w[y, c])
    return dict(nll=np.array(nll), lse=np.array(lse), tgt=np.array(tgt), dh=dh)
