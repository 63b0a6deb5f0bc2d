"""The forward and the no-allocation backward (attn_fwd, attn_bwd_noalloc)
captured in one HIP graph through the C ABI and replayed: callers that cannot
allocate, such as code under stream capture, are what attn_bwd_noalloc is for.
Between replays the inputs get new values and the same calls run eagerly;
every replay must give the eager outputs bit for bit (the same kernels on the
same inputs), and the first must meet the oracle's tolerance."""
import numpy as np
import pytest

import gpu_helpers as H
import sliding_window_flash_amd as swa
from sliding_window_flash_amd.workloads import make_inputs, small_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_captured_forward_and_noalloc_backward_replay_like_eager():
    import torch
    w = small_case([300, 77], None, heads_q=4, heads_kv=2, head_dim=128, window=96, dtype="bf16",
                   do_scale=0.1, seed=51)
    H.say(f"graph case {w.name}: lengths {w.lengths_q}, window {w.window}")
    kw = dict(max_seqlen_q=w.max_seqlen_q, max_seqlen_k=w.max_seqlen_k, window=w.window, causal=w.causal,
              scale=w.scale)
    x0 = make_inputs(w)
    dev = H.to_device(w, x0)
    q, k, v, do, cu_q, cu_k = (dev[n] for n in ("q", "k", "v", "do", "cu_q", "cu_k"))
    o, lse = torch.empty_like(q), torch.empty((w.heads_q, w.total_q), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step(out, stream=None):
        swa.fwd(q, k, v, cu_q, cu_k, out=out[0], lse=out[1], stream=stream, **kw)
        swa.bwd_noalloc(q, k, v, out[0], out[1], do, cu_q, cu_k, dq=out[2], dk=out[3], dv=out[4],
                        stream=stream, **kw)

    graph_out = (o, lse, dq, dk, dv)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(graph_out, s)  # eager first call on this GPU: the scratch address is looked up here
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(graph_out, s)
    torch.cuda.synchronize()

    for rep in range(3):
        x = x0 if rep == 0 else make_inputs(w, seed=w.seed + 100 + rep)
        for name in ("q", "k", "v", "do"):
            dev[name].copy_(torch.from_numpy(x[name]).to(q.dtype))
        torch.cuda.synchronize()
        ref = tuple(torch.full_like(t, float("nan")) for t in graph_out)
        step(ref)
        torch.cuda.synchronize()
        for t in graph_out:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), graph_out, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
        H.say(f"  replay {rep}: outputs equal to the eager call")
        if rep == 0:
            stats = H.compare_full(w, x, dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv))
            H.say("  ", {kk: {k2: f"{v2:.2e}" for k2, v2 in vv.items()} for kk, vv in stats.items()})
