"""attn_bwd_noalloc (no workspace argument, the library's fixed per-GPU
scratch for D and LSE * log2 e) against attn_bwd on the same inputs, through
the C ABI: two calls in a row, the second on a smaller problem, so the second
runs on scratch still holding the first call's values. dQ must equal
attn_bwd's bit for bit (the same kernel reads the same values); so must dK and
dV when attn_bwd does not split the dK/dV launch over query heads (the first
call, whose key tiles fill the GPU). With the split (the second call) attn_bwd
adds the heads' partial sums in another order, so dK and dV are held to the
oracle's tolerance against it. Each call's outputs must also meet the
oracle's tolerance."""
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


def _case(w, bitwise_dkdv):
    import torch
    H.say(f"no-alloc case {w.name}: lengths_q={w.lengths_q} lengths_k={w.lengths_k} Hq={w.heads_q} "
          f"Hkv={w.heads_kv} d={w.head_dim} window={w.window} dtype={w.dtype}")
    x = make_inputs(w)
    dev = H.to_device(w, x)
    kw = dict(max_seqlen_q=w.max_seqlen_q, max_seqlen_k=w.max_seqlen_k, window=w.window, causal=w.causal,
              scale=w.scale)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o, lse = swa.fwd(q, k, v, dev["cu_q"], dev["cu_k"], **kw)
    ref = swa.bwd(q, k, v, o, lse, do, dev["cu_q"], dev["cu_k"], **kw)
    got = [torch.full_like(t, float("nan")) for t in ref]
    swa.bwd_noalloc(q, k, v, o, lse, do, dev["cu_q"], dev["cu_k"], dq=got[0], dk=got[1], dv=got[2], **kw)
    torch.cuda.synchronize()
    assert torch.equal(got[0], ref[0]), "dq differs from attn_bwd"
    for name, a, b in zip(("dk", "dv"), got[1:], ref[1:]):
        if bitwise_dkdv:
            assert torch.equal(a, b), f"{name} differs from attn_bwd"
        else:
            H.compare(f"{name} against attn_bwd", H.host64(a), H.host64(b), w.dtype)
    stats = H.compare_full(w, x, dict(dq=got[0], dk=got[1], dv=got[2]))
    H.say("  ", {kk: {k2: f"{v2:.2e}" for k2, v2 in vv.items()} for kk, vv in stats.items()})


def test_two_calls_second_smaller():
    # 32 key tiles x 8 KV heads = 256 dK/dV workgroups: attn_bwd does not split
    first = small_case([4096], None, heads_q=16, heads_kv=8, head_dim=128, window=129,
                       dtype="bf16", do_scale=0.1, seed=41)
    second = small_case([100, 40], [700, 300], heads_q=4, heads_kv=1, head_dim=64, window=16,
                        dtype="bf16", do_scale=0.1, seed=42)
    assert first.heads_q * first.total_q > second.heads_q * second.total_q
    _case(first, bitwise_dkdv=True)
    _case(second, bitwise_dkdv=False)


def test_refuses_beyond_scratch():
    import torch
    # 32 heads x 140,000 tokens: 2 x 32 x 140,000 x 4 bytes of D and LSE*log2e > 32 MiB
    p = swa.make_params(batch=1, heads_q=32, heads_kv=8, head_dim=128, total_q=140000, total_k=140000,
                        max_seqlen_q=140000, max_seqlen_k=140000, window=1024)
    assert swa.workspace_bytes(p) > swa.NOALLOC_SCRATCH_BYTES
    import ctypes
    t = torch.empty(16, dtype=torch.uint8, device="cuda")
    ptr = t.data_ptr()
    st = swa.lib().attn_bwd_noalloc(ctypes.byref(p), *([ptr] * 11), None)
    assert st == 8, st
