"""Central finite differences of the loss L = sum(O * dO).

TEST INFRASTRUCTURE ONLY (see the package header). Pins the backward formula of
``oracle.dense`` to its forward: the gradient it returns must be the derivative
of that forward, element by element, by the textbook two-sided difference
(L(x + h) - L(x - h)) / 2h. Tiny shapes only (two forward passes per element).
"""
from __future__ import annotations

import numpy as np

from . import dense


def loss(q, k, v, do, cu_q, cu_k, scale, window, causal, forward=None, mask=None) -> float:
    forward = dense.sdpa_reference if forward is None else forward
    kw = {} if mask is None else dict(mask=mask)
    out = forward(q, k, v, None, cu_q, cu_k, scale, window, causal, with_backward=False, **kw)
    return float(np.sum(out["o"] * np.asarray(do, dtype=np.float64)))


def grads(q, k, v, do, cu_q, cu_k, scale, window, causal, step: float = 1e-5,
          forward=None, mask=None) -> dict:
    """dQ, dK, dV of L by central differences; ``forward`` defaults to the
    dense oracle's forward."""
    args = dict(q=np.array(q, dtype=np.float64), k=np.array(k, dtype=np.float64),
                v=np.array(v, dtype=np.float64))
    out = {}
    for name in ("q", "k", "v"):
        x = args[name]
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + step
            up = loss(args["q"], args["k"], args["v"], do, cu_q, cu_k, scale, window, causal,
                      forward, mask)
            x[idx] = keep - step
            dn = loss(args["q"], args["k"], args["v"], do, cu_q, cu_k, scale, window, causal,
                      forward, mask)
            x[idx] = keep
            g[idx] = (up - dn) / (2 * step)
        out["d" + name] = g
    return out
