"""Dense fp64 reference for the linear cross-entropy loss and its gradient.

TEST INFRASTRUCTURE ONLY (see the package header): never imported by the
product path.

What is computed (the mlx-train-perf README, the passage on the logit-free
linear cross-entropy): hidden states H [n, D], an output head W [V, D] and
targets y [n]. The logits z = H W^T [n, V] are the tensor the fused loss never
builds. Per token i:

  lse_i    = log sum_v exp(z_iv)          (natural log)
  tgt_i    = z_{i, y_i}                    (the target logit)
  nll_i    = lse_i - tgt_i                 (the per-token loss)

These are the three length-n arrays the README's forward returns. The
backward is the gradient back into the hidden states (the README: only the
per-token loss and a gradient into the hidden states are needed; the head is
not trained), for an upstream gradient g = dL/dnll [n]:

  dH_i = g_i * ( sum_v p_iv W_v - W_{y_i} ),   p_iv = exp(z_iv - lse_i).

Here the full row of logits is built for a panel of rows at a time (the
plain definition; the memory it takes is the point of the fused kernel, not of
this reference).
"""
from __future__ import annotations

from typing import Optional

import numpy as np

F64 = np.float64


def ce_reference(h, w, targets, dnll=None, *, rows: Optional[np.ndarray] = None,
                 panel_rows: int = 64) -> dict:
    """nll, lse, tgt (fp64 [len(rows)]) and, with ``dnll``, dh [len(rows), D].

    ``rows`` restricts the work to those token rows (default: all n); ``dnll``
    then holds one upstream gradient per selected row, in the same order.
    """
    h = np.asarray(h)
    w64 = np.asarray(w, dtype=F64)
    targets = np.asarray(targets, dtype=np.int64)
    rows = np.arange(h.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    n = rows.size
    out = dict(nll=np.zeros(n), lse=np.zeros(n), tgt=np.zeros(n))
    if dnll is not None:
        out["dh"] = np.zeros((n, w64.shape[1]))
    for r0 in range(0, n, panel_rows):
        rr = rows[r0:r0 + panel_rows]
        hp = np.asarray(h[rr], dtype=F64)
        z = hp @ w64.T                                   # [panel, V]
        m = z.max(axis=1)
        lse = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
        tgt = z[np.arange(rr.size), targets[rr]]
        out["lse"][r0:r0 + rr.size] = lse
        out["tgt"][r0:r0 + rr.size] = tgt
        out["nll"][r0:r0 + rr.size] = lse - tgt
        if dnll is not None:
            p = np.exp(z - lse[:, None])
            g = np.asarray(dnll, dtype=F64)[r0:r0 + rr.size]
            out["dh"][r0:r0 + rr.size] = g[:, None] * (p @ w64 - w64[targets[rr]])
    return out
