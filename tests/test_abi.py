"""The C-ABI library loads without a GPU, exports what include/swa_attn.h
declares, and refuses bad arguments up front (no launch is attempted)."""
import ctypes
import os
import re

import pytest

import sliding_window_flash_amd as swa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for hdr in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if hdr.endswith(".h"):
            text = open(os.path.join(ROOT, "include", hdr)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b((?:attn|ce)_\w+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 8, names
    L = swa.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(swa.EXPORTED)


def good(**kw):
    base = dict(batch=1, heads_q=4, heads_kv=2, head_dim=128, total_q=100, total_k=100,
                max_seqlen_q=100, max_seqlen_k=100, window=16, causal=True, scale=0.1,
                dtype=swa.ATTN_BF16)
    base.update(kw)
    return swa.make_params(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(), 0),
    (dict(batch=0), 2),
    (dict(heads_q=3), 2),
    (dict(heads_kv=0), 2),
    (dict(total_q=-1), 2),
    (dict(max_seqlen_q=101), 2),
    (dict(window=0), 3),
    (dict(window=-5), 3),
    (dict(head_dim=96), 4),
    (dict(head_dim=512), 0),
    (dict(head_dim=512, dtype=swa.ATTN_F16), 0),
    (dict(head_dim=512, dtype=swa.ATTN_F32), 4),
    (dict(head_dim=1024), 4),
    # a 128-row tile of 16384 heads x 512 bf16 columns spans 2^31 bytes
    (dict(heads_q=16384, heads_kv=16384, head_dim=512), 2),
    (dict(heads_q=8192, heads_kv=8192, head_dim=512), 0),
    (dict(dtype=7), 4),
    (dict(causal=False, window=50), 0),     # two-sided window
    (dict(heads_q=1, heads_kv=1, total_q=2**30 + 8, total_k=2**30 + 8, max_seqlen_q=2**30 + 8,
          max_seqlen_k=2**30 + 8, causal=False, window=50), 4),  # two-sided beyond 2^30 keys
    (dict(heads_q=1, heads_kv=1, total_q=2**30 + 8, total_k=64, max_seqlen_q=2**30 + 8,
          max_seqlen_k=64, causal=False, window=100), 4),  # two-sided beyond 2^30 queries
    (dict(heads_q=1, heads_kv=1, total_q=2**30 + 8, total_k=64, max_seqlen_q=2**30 + 8,
          max_seqlen_k=64, causal=False, window=2**30 + 8), 0),  # full attention: no limit
    (dict(heads_q=1, heads_kv=1, total_q=2**30 + 8, total_k=64, max_seqlen_q=2**30 + 8,
          max_seqlen_k=64, causal=True, window=100), 0),  # causal: no limit
    (dict(causal=False, window=100), 0),
    (dict(window=swa.INT32_MAX), 0),
    (dict(dtype=swa.ATTN_F32, head_dim=64), 0),
    (dict(dtype=swa.ATTN_F16), 0),
    (dict(head_dim=256), 0),
    (dict(head_dim=256, dtype=swa.ATTN_F16), 0),
    (dict(head_dim=256, dtype=swa.ATTN_F32), 4),
    (dict(dtype=3), 4),
    (dict(scale=0.0), 4),
    (dict(scale=-0.1), 4),
    (dict(scale=float("inf")), 4),
    # work items beyond a 32-bit launch id: many sequences, one of them long
    (dict(batch=2**20, heads_q=64, heads_kv=8, total_q=2**24, total_k=2**24, max_seqlen_q=2**14,
          max_seqlen_k=2**14), 2),
    (dict(batch=2**10, heads_q=64, heads_kv=8, total_q=2**24, total_k=2**24, max_seqlen_q=2**14,
          max_seqlen_k=2**14), 0),
    (dict(scale=float("nan")), 4),
    (dict(heads_q=16384, heads_kv=16384), 0),
    (dict(heads_q=16386, heads_kv=2), 2),
])
def test_parameter_checks(kw, code):
    assert swa.check_params(good(**kw)) == code


def test_status_strings():
    L = swa.lib()
    for code in range(9):
        s = L.attn_status_str(code).decode()
        assert s and s != "unknown status"
    assert L.attn_status_str(99).decode() == "unknown status"


def _fwd(p, q=16, k=16, v=16, cq=16, ck=16, o=16, lse=16):
    L = swa.lib()
    return L.attn_fwd(ctypes.byref(p) if p is not None else None, q, k, v, cq, ck, o, lse, None)


def test_forward_refuses_before_launch():
    assert _fwd(None) == 1
    assert _fwd(good(window=0)) == 3
    assert _fwd(good(), q=None) == 1
    assert _fwd(good(), cq=None) == 1
    assert _fwd(good(), lse=None) == 1
    assert _fwd(good(), o=24) == 7       # not 16-byte aligned
    assert _fwd(good(), cq=18) == 7      # int32 offsets need 4 bytes
    assert _fwd(good(head_dim=32)) == 4


def test_backward_refuses_before_launch():
    L = swa.lib()
    p = good()
    need = swa.workspace_bytes(p)
    assert need >= 4 * 4 * 100 and need % 256 == 0
    args = [16] * 11
    assert L.attn_bwd(ctypes.byref(p), *args, 16, need - 1, None) == 5
    assert L.attn_bwd(ctypes.byref(p), *args, None, need, None) == 5
    bad = list(args)
    bad[8] = None  # dq
    assert L.attn_bwd(ctypes.byref(p), *bad, 16, need, None) == 1
    # refused before any launch (the pointers are not device memory)
    assert L.attn_bwd(ctypes.byref(good(head_dim=96)), *args, 16, need, None) == 4
    assert L.attn_bwd(ctypes.byref(good(head_dim=256, dtype=swa.ATTN_F32)), *args, 16, need, None) == 4
    assert swa.workspace_bytes(good(window=0)) == 0


def test_tile_sizes():
    bm, bn, kbn, kbm = swa.tile_sizes(128, swa.ATTN_BF16)
    assert bm % 32 == 0 and bn % 32 == 0 and kbn % 32 == 0 and kbm % 32 == 0
    assert swa.tile_sizes(128, swa.ATTN_F16) == (bm, bn, kbn, kbm)
    assert swa.tile_sizes(256, swa.ATTN_BF16)[2:] == (128, 32)
    assert swa.tile_sizes(512, swa.ATTN_BF16) == (128, 32, 128, 32)
    with pytest.raises(swa.AttnError):
        swa.tile_sizes(256, swa.ATTN_F32)
    with pytest.raises(swa.AttnError):
        swa.tile_sizes(512, swa.ATTN_F32)
    with pytest.raises(swa.AttnError):
        swa.tile_sizes(96, swa.ATTN_BF16)


def _mask(bits=16, row_words=4):
    return swa.AttnMask(bits, row_words)


def test_masked_entry_points_refuse_before_launch():
    """Every configuration here is refused by the checks; no kernel is launched
    (the pointers are not device memory)."""
    L = swa.lib()
    p = good()   # max_seqlen_k = 100: at least 4 words per row
    fw = lambda m, **kw: L.attn_fwd_masked(ctypes.byref(kw.get("p", p)), m, 16, 16, 16, 16, 16, 16, 16, None)
    assert fw(None) == 1
    assert fw(ctypes.byref(_mask(bits=None))) == 1
    assert fw(ctypes.byref(_mask(bits=24))) == 7          # not 16-byte aligned
    assert fw(ctypes.byref(_mask(row_words=6))) == 2      # not a multiple of 4
    assert fw(ctypes.byref(_mask(row_words=0))) == 2
    big = good(total_q=200, total_k=200, max_seqlen_k=200, max_seqlen_q=200)
    assert fw(ctypes.byref(_mask(row_words=4)), p=big) == 2   # 200 keys need 7 words
    assert fw(ctypes.byref(_mask(row_words=(1 << 24) + 4))) == 4
    # a 64-row mask tile spans 64 x row_words x 4 bytes, which must stay below
    # 2^32: 2^24 words is refused, the largest multiple of 4 below it accepted
    # (the call then stops at the NULL LSE that follows the mask checks)
    assert fw(ctypes.byref(_mask(row_words=1 << 24))) == 4
    assert L.attn_fwd_masked(ctypes.byref(p), ctypes.byref(_mask(row_words=(1 << 24) - 4)), 16, 16, 16, 16, 16,
                             16, None, None) == 1
    assert fw(ctypes.byref(_mask()), p=good(window=0)) == 3  # parameter checks come first
    need = swa.workspace_bytes(p)
    args = [16] * 11
    bw = lambda m: L.attn_bwd_masked(ctypes.byref(p), m, *args, 16, need, None)
    assert bw(None) == 1
    assert bw(ctypes.byref(_mask(row_words=2))) == 2
    assert bw(ctypes.byref(_mask(bits=8))) == 7
    assert L.attn_bwd_masked(ctypes.byref(p), ctypes.byref(_mask()), *args, 16, need - 1, None) == 5


@pytest.mark.parametrize("kw,code", [
    (dict(), 0),
    (dict(n=0), 0),
    (dict(n=-1), 2),
    (dict(vocab=0), 2),
    (dict(hidden=300), 2),
    (dict(hidden=0), 2),
    (dict(dtype=swa.ATTN_F32), 4),
    (dict(dtype=9), 4),
    (dict(n=1 << 20, hidden=4096), 2),   # n * hidden >= 2^31
])
def test_ce_parameter_checks(kw, code):
    base = dict(n=100, vocab=1000, hidden=512, dtype=swa.ATTN_BF16)
    base.update(kw)
    assert swa.lib().ce_check_params(ctypes.byref(swa.ce_params(**base))) == code


def test_ce_refuses_before_launch():
    """Every call here is refused by the checks (the pointers are not device memory)."""
    L = swa.lib()
    p = swa.ce_params(100, 1000, 512, swa.ATTN_BF16)
    fw = L.ce_fwd_workspace_bytes(ctypes.byref(p))
    bw = L.ce_bwd_workspace_bytes(ctypes.byref(p))
    assert fw >= 4 * 100 * 8 and fw % 256 == 0 and bw >= 100 * 1024 * 2
    assert L.ce_fwd(None, 16, 16, 16, 16, 16, 16, 16, fw, None) == 1
    assert L.ce_fwd(ctypes.byref(p), None, 16, 16, 16, 16, 16, 16, fw, None) == 1
    assert L.ce_fwd(ctypes.byref(p), 24, 16, 16, 16, 16, 16, 16, fw, None) == 7
    assert L.ce_fwd(ctypes.byref(p), 16, 16, 16, 16, 16, 16, 16, fw - 1, None) == 5
    assert L.ce_fwd(ctypes.byref(p), 16, 16, 16, 16, 16, 16, None, fw, None) == 5
    assert L.ce_bwd(ctypes.byref(p), 16, 16, 16, 16, 16, 16, 16, bw - 1, None) == 5
    assert L.ce_bwd(ctypes.byref(p), 16, 16, 16, 16, None, 16, 16, bw, None) == 1
    assert L.ce_bwd(ctypes.byref(swa.ce_params(100, 1000, 512, swa.ATTN_F32)), 16, 16, 16, 16, 16, 16, 16, bw,
                    None) == 4
    # several vocabulary chunks need the fp32 dH accumulator as well
    big = swa.ce_params(64, 40000, 256, swa.ATTN_BF16)
    assert L.ce_bwd_workspace_bytes(ctypes.byref(big)) >= 64 * 16384 * 2 + 64 * 256 * 4


def test_noalloc_backward_refuses_before_any_hip_call():
    L = swa.lib()
    args = [16] * 11
    assert L.attn_bwd_noalloc(ctypes.byref(good(window=0)), *args, None) == 3
    bad = list(args)
    bad[8] = None  # dq
    assert L.attn_bwd_noalloc(ctypes.byref(good()), *bad, None) == 1
    # 2 x 32 heads x 140,000 tokens x 4 bytes of D and LSE*log2e exceed the fixed scratch
    big = good(heads_q=32, heads_kv=8, total_q=140000, total_k=140000, max_seqlen_q=140000,
               max_seqlen_k=140000)
    assert swa.workspace_bytes(big) > swa.NOALLOC_SCRATCH_BYTES
    assert L.attn_bwd_noalloc(ctypes.byref(big), *args, None) == 8


def test_mask_ranges_refuses_before_launch():
    L = swa.lib()
    p = good()   # batch 1, 100 queries and keys: 4 + 4 blocks -> 16 int32
    assert L.attn_mask_ranges_bytes(ctypes.byref(p)) == 2 * (4 + 4) * 4
    assert L.attn_mask_ranges_bytes(ctypes.byref(good(window=0))) == 0
    m = swa.AttnMask(16, 4)
    assert L.attn_mask_ranges(ctypes.byref(good(window=0)), ctypes.byref(m), 16, 16, 16, None) == 3
    assert L.attn_mask_ranges(ctypes.byref(p), None, 16, 16, 16, None) == 1
    assert L.attn_mask_ranges(ctypes.byref(p), ctypes.byref(swa.AttnMask(16, 2)), 16, 16, 16, None) == 2
    assert L.attn_mask_ranges(ctypes.byref(p), ctypes.byref(m), None, 16, 16, None) == 1
    assert L.attn_mask_ranges(ctypes.byref(p), ctypes.byref(m), 16, 16, None, None) == 1
    assert L.attn_mask_ranges(ctypes.byref(p), ctypes.byref(m), 16, 16, 18, None) == 7
    # the forward refuses a misaligned ranges pointer in the mask
    bad = swa.AttnMask(16, 4, 18)
    assert L.attn_fwd_masked(ctypes.byref(p), ctypes.byref(bad), 16, 16, 16, 16, 16, 16, 16, None) == 7
