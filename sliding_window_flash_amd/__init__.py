"""Sliding-window flash attention for MI355X (gfx950): Python binding.

A thin ctypes layer over the C ABI in include/swa_attn.h (libswa_attn.so,
built in-tree by ``sliding_window_flash_amd.build``). It marshals arguments
only: every step of the forward and backward runs in the HIP kernels. PyTorch
supplies device memory and the stream. There is no CPU path: if the library
is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libswa_attn.so")

ATTN_F32, ATTN_BF16, ATTN_F16 = 0, 1, 2
INT32_MAX = 2**31 - 1

STATUS = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_WINDOW",
    4: "ATTN_ERR_UNSUPPORTED", 5: "ATTN_ERR_WORKSPACE", 6: "ATTN_ERR_HIP", 7: "ATTN_ERR_ALIGN",
    8: "ATTN_ERR_TOO_LARGE",
}
NOALLOC_SCRATCH_BYTES = 32 << 20   # ATTN_NOALLOC_SCRATCH_BYTES

BWD_DELTA, BWD_DQ, BWD_DKDV, BWD_ALL = 1, 2, 4, 7

EXPORTED = ("attn_fwd", "attn_bwd", "attn_bwd_stages", "attn_bwd_workspace_bytes", "attn_status_str",
            "attn_check_params", "attn_tile_sizes", "attn_query_tile_range",
            "attn_key_tile_range", "attn_fwd_masked", "attn_bwd_masked", "attn_bwd_noalloc",
            "attn_mask_ranges_bytes", "attn_mask_ranges",
            "ce_check_params", "ce_fwd_workspace_bytes", "ce_fwd", "ce_bwd_workspace_bytes", "ce_bwd")


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_status_str(status)})")


class AttnParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("total_q", ctypes.c_int32), ("total_k", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32),
        ("window", ctypes.c_int32), ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


class CEParams(ctypes.Structure):
    """ce_params_t (include/swa_ce.h)."""
    _fields_ = [("n", ctypes.c_int32), ("vocab", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class AttnMask(ctypes.Structure):
    """attn_mask_t: bit-packed rows of a boolean mask combined with the window,
    and optionally the ranges attn_mask_ranges wrote for it."""
    _fields_ = [("bits", ctypes.c_void_p), ("row_words", ctypes.c_int64), ("ranges", ctypes.c_void_p)]


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded C library. Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sliding_window_flash_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(AttnParams)
        vp, i32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)
        L.attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        L.attn_fwd.restype = ctypes.c_int
        L.attn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.attn_bwd.restype = ctypes.c_int
        L.attn_bwd_stages.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, vp, ctypes.c_size_t, vp]
        L.attn_bwd_stages.restype = ctypes.c_int
        L.attn_bwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.attn_bwd_noalloc.restype = ctypes.c_int
        L.attn_bwd_workspace_bytes.argtypes = [P]
        L.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
        M = ctypes.POINTER(AttnMask)
        L.attn_fwd_masked.argtypes = [P, M, vp, vp, vp, vp, vp, vp, vp, vp]
        L.attn_fwd_masked.restype = ctypes.c_int
        L.attn_bwd_masked.argtypes = [P, M, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      ctypes.c_size_t, vp]
        L.attn_bwd_masked.restype = ctypes.c_int
        L.attn_mask_ranges_bytes.argtypes = [P]
        L.attn_mask_ranges_bytes.restype = ctypes.c_size_t
        L.attn_mask_ranges.argtypes = [P, M, vp, vp, vp, vp]
        L.attn_mask_ranges.restype = ctypes.c_int
        C = ctypes.POINTER(CEParams)
        L.ce_check_params.argtypes = [C]
        L.ce_check_params.restype = ctypes.c_int
        L.ce_fwd_workspace_bytes.argtypes = [C]
        L.ce_fwd_workspace_bytes.restype = ctypes.c_size_t
        L.ce_bwd_workspace_bytes.argtypes = [C]
        L.ce_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.ce_fwd.argtypes = [C, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.ce_fwd.restype = ctypes.c_int
        L.ce_bwd.argtypes = [C, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.ce_bwd.restype = ctypes.c_int
        L.attn_status_str.argtypes = [ctypes.c_int]
        L.attn_status_str.restype = ctypes.c_char_p
        L.attn_check_params.argtypes = [P]
        L.attn_check_params.restype = ctypes.c_int
        L.attn_tile_sizes.argtypes = [ctypes.c_int32, ctypes.c_int32, i32p, i32p, i32p, i32p]
        L.attn_tile_sizes.restype = ctypes.c_int
        L.attn_query_tile_range.argtypes = [P, i32p, i32p, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, i32p, i32p, i32p, i32p]
        L.attn_query_tile_range.restype = ctypes.c_int
        L.attn_key_tile_range.argtypes = [P, i32p, i32p, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, i32p, i32p]
        L.attn_key_tile_range.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _status_str(status: int) -> str:
    try:
        return lib().attn_status_str(status).decode()
    except Exception:  # pragma: no cover - only while reporting another error
        return "?"


def make_params(*, batch, heads_q, heads_kv, head_dim, total_q, total_k, max_seqlen_q,
                max_seqlen_k, window=INT32_MAX, causal=True, scale=None, dtype=ATTN_BF16) -> AttnParams:
    if scale is None:
        scale = head_dim ** -0.5
    return AttnParams(int(batch), int(heads_q), int(heads_kv), int(head_dim), int(total_q),
                      int(total_k), int(max_seqlen_q), int(max_seqlen_k),
                      int(min(window, INT32_MAX)), int(bool(causal)), float(scale), int(dtype))


def check_params(p: AttnParams) -> int:
    return lib().attn_check_params(ctypes.byref(p))


def workspace_bytes(p: AttnParams) -> int:
    return int(lib().attn_bwd_workspace_bytes(ctypes.byref(p)))


def tile_sizes(head_dim: int, dtype: int) -> Tuple[int, int, int, int]:
    out = [ctypes.c_int32() for _ in range(4)]
    st = lib().attn_tile_sizes(head_dim, dtype, *[ctypes.byref(x) for x in out])
    if st:
        raise AttnError(st, "attn_tile_sizes")
    return tuple(x.value for x in out)


def _i32_array(xs):
    arr = (ctypes.c_int32 * len(xs))(*[int(x) for x in xs])
    return arr


def query_tile_range(p: AttnParams, cu_q, cu_k, b: int, qb: int, bm: int, bn: int):
    out = [ctypes.c_int32() for _ in range(4)]
    st = lib().attn_query_tile_range(ctypes.byref(p), _i32_array(cu_q), _i32_array(cu_k), b, qb,
                                     bm, bn, *[ctypes.byref(x) for x in out])
    if st:
        raise AttnError(st, "attn_query_tile_range")
    return tuple(x.value for x in out)


def key_tile_range(p: AttnParams, cu_q, cu_k, b: int, kb: int, bn: int, bm: int):
    out = [ctypes.c_int32() for _ in range(2)]
    st = lib().attn_key_tile_range(ctypes.byref(p), _i32_array(cu_q), _i32_array(cu_k), b, kb,
                                   bn, bm, *[ctypes.byref(x) for x in out])
    if st:
        raise AttnError(st, "attn_key_tile_range")
    return tuple(x.value for x in out)


# ---------------------------------------------------------------- torch glue
def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_ptr(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def params_for(q, k, cu_q, cu_k, *, max_seqlen_q, max_seqlen_k, window=INT32_MAX, causal=True,
               scale=None) -> AttnParams:
    torch = _torch()
    dt = {torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16, torch.float32: ATTN_F32}.get(q.dtype)
    if dt is None:
        raise AttnError(4, f"dtype {q.dtype}")
    return make_params(batch=cu_q.numel() - 1, heads_q=q.shape[1], heads_kv=k.shape[1],
                       head_dim=q.shape[2], total_q=q.shape[0], total_k=k.shape[0],
                       max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k, window=window,
                       causal=causal, scale=scale, dtype=dt)


def _require(t, name):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    return t


def _expect(t, name, shape, dtype):
    """``t`` must have exactly this shape and dtype (checked before any pointer
    is taken: the C ABI takes every size from q and k alone, so a mismatched
    tensor would be read or written out of its bounds)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _check_attn(q, k, v, cu_q, cu_k, *, o=None, lse=None, do=None, dq=None, dk=None, dv=None,
                mask=None, workspace=None, need_ws=0, devices=True):
    """Shapes and dtypes of every tensor against q ([T_q, Hq, d]) and k
    ([T_k, Hkv, d]), then (``devices``) device residency and contiguity.
    Raises ValueError."""
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [total_q, heads_q, head_dim] and k [total_k, heads_kv, head_dim]")
    tq, hq, d = q.shape
    tk, hkv, dk_ = k.shape
    if dk_ != d:
        raise ValueError(f"k head_dim {dk_} differs from q head_dim {d}")
    if k.dtype != q.dtype:
        raise ValueError(f"k has dtype {k.dtype}, expected {q.dtype}")
    _expect(v, "v", k.shape, q.dtype)
    if cu_q.dim() != 1 or cu_k.dim() != 1 or cu_q.numel() < 2 or cu_q.numel() != cu_k.numel():
        raise ValueError("cu_q and cu_k must be 1-D with batch + 1 (>= 2) elements each")
    for t, n in ((cu_q, "cu_q"), (cu_k, "cu_k")):
        if t.dtype != torch.int32:
            raise ValueError(f"{n} has dtype {t.dtype}, expected torch.int32")
    named = [(o, "o", q.shape, q.dtype), (do, "do", q.shape, q.dtype), (dq, "dq", q.shape, q.dtype),
             (dk, "dk", k.shape, q.dtype), (dv, "dv", k.shape, q.dtype),
             (lse, "lse", (hq, tq), torch.float32)]
    for t, n, shp, dt in named:
        if t is not None:
            _expect(t, n, shp, dt)
    if mask is not None:
        if mask.dim() != 2 or mask.element_size() != 4 or mask.shape[0] != tq:
            raise ValueError(f"mask must be [total_q = {tq}, row_words] of 32-bit words, "
                             f"got {tuple(mask.shape)} of {mask.dtype}")
    if workspace is not None and workspace.numel() * workspace.element_size() < need_ws:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                         f"needs {need_ws}")
    if not devices:
        return
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (cu_q, "cu_q"), (cu_k, "cu_k"), (o, "o"), (lse, "lse"),
                 (do, "do"), (dq, "dq"), (dk, "dk"), (dv, "dv"), (mask, "mask"), (workspace, "workspace")):
        if t is not None:
            _require(t, n)
            if t.device != q.device:
                raise ValueError(f"{n} is on {t.device}, q on {q.device}")


def _mask_arg(mask, ranges=None):
    """attn_mask_t for a device tensor of packed rows ([T_q, row_words], 32-bit
    words; bit j % 32 of word j // 32 allows key j of the row's sequence) and
    optional ranges from :func:`mask_ranges`."""
    return AttnMask(mask.data_ptr(), mask.shape[1], _ptr(ranges))


def _check_ranges(ranges, p, mask, q):
    torch = _torch()
    if ranges is None:
        return
    if mask is None:
        raise ValueError("mask_ranges given without a mask")
    n = int(lib().attn_mask_ranges_bytes(ctypes.byref(p))) // 4
    _expect(ranges, "mask_ranges", (n,), torch.int32)
    _require(ranges, "mask_ranges")
    if ranges.device != q.device:
        raise ValueError(f"mask_ranges is on {ranges.device}, q on {q.device}")


def mask_ranges(q, k, cu_q, cu_k, mask, *, max_seqlen_q, max_seqlen_k, window=INT32_MAX, causal=True,
                scale=None, out=None, stream=None):
    """attn_mask_ranges: where the mask's allowed bits lie (int32 device
    tensor), for fwd/bwd's ``mask_ranges``; q and k give the shapes."""
    torch = _torch()
    _check_attn(q, k, k, cu_q, cu_k, mask=mask)
    p = params_for(q, k, cu_q, cu_k, max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k,
                   window=window, causal=causal, scale=scale)
    n = int(lib().attn_mask_ranges_bytes(ctypes.byref(p))) // 4
    out = torch.empty(max(n, 1), dtype=torch.int32, device=q.device) if out is None else out
    if out.numel() < n or out.dtype != torch.int32:
        raise ValueError(f"mask_ranges out must be int32 with {n} elements")
    _require(out, "mask_ranges out")
    if out.device != q.device:
        raise ValueError(f"mask_ranges out is on {out.device}, q on {q.device}")
    m = _mask_arg(mask)
    st = lib().attn_mask_ranges(ctypes.byref(p), ctypes.byref(m), _ptr(cu_q), _ptr(cu_k), _ptr(out),
                                _stream_ptr(stream))
    if st:
        raise AttnError(st, "attn_mask_ranges")
    return out[:n]


def fwd(q, k, v, cu_q, cu_k, *, max_seqlen_q, max_seqlen_k, window=INT32_MAX, causal=True,
        scale=None, out=None, lse=None, stream=None, mask=None, mask_ranges=None):
    """O [T_q, Hq, d] (q.dtype) and LSE [Hq, T_q] (fp32) through attn_fwd, or
    attn_fwd_masked when ``mask`` (packed rows, see :func:`_mask_arg`) is given
    (with ``mask_ranges`` from :func:`mask_ranges`: tiles the mask empties are
    skipped)."""
    torch = _torch()
    _check_attn(q, k, v, cu_q, cu_k, o=out, lse=lse, mask=mask)
    p = params_for(q, k, cu_q, cu_k, max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k,
                   window=window, causal=causal, scale=scale)
    _check_ranges(mask_ranges, p, mask, q)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(cu_q), _ptr(cu_k), _ptr(out), _ptr(lse), _stream_ptr(stream))
    if mask is None:
        st, what = lib().attn_fwd(ctypes.byref(p), *args), "attn_fwd"
    else:
        m = _mask_arg(mask, mask_ranges)
        st, what = lib().attn_fwd_masked(ctypes.byref(p), ctypes.byref(m), *args), "attn_fwd_masked"
    if st:
        raise AttnError(st, what)
    return out, lse


def bwd(q, k, v, o, lse, do, cu_q, cu_k, *, max_seqlen_q, max_seqlen_k, window=INT32_MAX,
        causal=True, scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None,
        stages=BWD_ALL, mask=None, mask_ranges=None):
    """dQ, dK, dV through attn_bwd_stages (the VJP of sum(O * dO)); ``stages``
    selects a subset of the backward's launches (all three by default). With
    ``mask`` (the forward's), through attn_bwd_masked (all stages), and with
    ``mask_ranges`` skipping the tiles the mask empties."""
    torch = _torch()
    _check_attn(q, k, v, cu_q, cu_k, o=o, lse=lse, do=do, dq=dq, dk=dk, dv=dv, mask=mask, devices=False)
    p = params_for(q, k, cu_q, cu_k, max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k,
                   window=window, causal=causal, scale=scale)
    nbytes = workspace_bytes(p)
    _check_attn(q, k, v, cu_q, cu_k, o=o, lse=lse, do=do, dq=dq, dk=dk, dv=dv, mask=mask,
                workspace=workspace, need_ws=nbytes)
    _check_ranges(mask_ranges, p, mask, q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(cu_q), _ptr(cu_k), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream_ptr(stream))
    if mask is None:
        st, what = lib().attn_bwd_stages(ctypes.byref(p), int(stages), *args), "attn_bwd_stages"
    else:
        if stages != BWD_ALL:
            raise ValueError("the masked backward runs all stages")
        m = _mask_arg(mask, mask_ranges)
        st, what = lib().attn_bwd_masked(ctypes.byref(p), ctypes.byref(m), *args), "attn_bwd_masked"
    if st:
        raise AttnError(st, what)
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, lse, do, cu_q, cu_k, *, max_seqlen_q, max_seqlen_k, window=INT32_MAX,
                causal=True, scale=None, dq=None, dk=None, dv=None, stream=None):
    """dQ, dK, dV through attn_bwd_noalloc: no workspace, the library's fixed
    per-GPU scratch instead (calls that overlap on one GPU race). Pass dq, dk
    and dv to allocate nothing here either."""
    torch = _torch()
    _check_attn(q, k, v, cu_q, cu_k, o=o, lse=lse, do=do, dq=dq, dk=dk, dv=dv)
    p = params_for(q, k, cu_q, cu_k, max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k,
                   window=window, causal=causal, scale=scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    st = lib().attn_bwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                _ptr(cu_q), _ptr(cu_k), _ptr(dq), _ptr(dk), _ptr(dv), _stream_ptr(stream))
    if st:
        raise AttnError(st, "attn_bwd_noalloc")
    return dq, dk, dv


# ---------------------------------------------------------------- linear cross-entropy
def ce_params(n: int, vocab: int, hidden: int, dtype: int) -> CEParams:
    return CEParams(n, vocab, hidden, dtype)


def ce_params_for(h, w) -> CEParams:
    torch = _torch()
    dt = {torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16, torch.float32: ATTN_F32}.get(h.dtype)
    if dt is None or w.dtype != h.dtype:
        raise AttnError(4, f"dtypes {h.dtype}, {w.dtype}")
    return CEParams(h.shape[0], w.shape[0], h.shape[1], dt)


def _check_ce(h, w, targets, *, f32=(), dh=None, workspace=None, need_ws=0, devices=True):
    """Shapes and dtypes against h ([n, hidden]) and w ([vocab, hidden]), then
    device residency and contiguity. ``f32``: (tensor, name) pairs that must
    be fp32 [n]. Raises ValueError."""
    torch = _torch()
    if h.dim() != 2 or w.dim() != 2 or h.shape[1] != w.shape[1]:
        raise ValueError(f"h must be [n, hidden] and w [vocab, hidden], got {tuple(h.shape)}, {tuple(w.shape)}")
    n = h.shape[0]
    _expect(targets, "targets", (n,), torch.int32)
    for t, nme in f32:
        if t is not None:
            _expect(t, nme, (n,), torch.float32)
    if dh is not None:
        _expect(dh, "dh", h.shape, h.dtype)
    if workspace is not None and workspace.numel() * workspace.element_size() < need_ws:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                         f"needs {need_ws}")
    if not devices:
        return
    for t, nme in [(h, "h"), (w, "w"), (targets, "targets"), (dh, "dh"), (workspace, "workspace")] + list(f32):
        if t is not None:
            _require(t, nme)
            if t.device != h.device:
                raise ValueError(f"{nme} is on {t.device}, h on {h.device}")


def ce_fwd(h, w, targets, *, nll=None, lse=None, tgt=None, workspace=None, stream=None):
    """Per-token loss, LSE and target logit (fp32 [n] each) of the linear
    cross-entropy with logits h @ w.T, through ce_fwd (no logits tensor)."""
    torch = _torch()
    f32 = ((nll, "nll"), (lse, "lse"), (tgt, "tgt"))
    _check_ce(h, w, targets, f32=f32, devices=False)
    p = ce_params_for(h, w)
    need = int(lib().ce_fwd_workspace_bytes(ctypes.byref(p)))
    _check_ce(h, w, targets, f32=f32, workspace=workspace, need_ws=need)
    n = h.shape[0]
    nll = torch.empty(n, dtype=torch.float32, device=h.device) if nll is None else nll
    lse = torch.empty(n, dtype=torch.float32, device=h.device) if lse is None else lse
    tgt = torch.empty(n, dtype=torch.float32, device=h.device) if tgt is None else tgt
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=h.device)
    st = lib().ce_fwd(ctypes.byref(p), _ptr(h), _ptr(w), _ptr(targets), _ptr(nll), _ptr(lse), _ptr(tgt),
                      _ptr(workspace), workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    if st:
        raise AttnError(st, "ce_fwd")
    return nll, lse, tgt


def ce_bwd(h, w, targets, lse, dnll, *, dh=None, workspace=None, stream=None):
    """dH [n, hidden] (h.dtype) of sum(dnll * nll), through ce_bwd."""
    torch = _torch()
    f32 = ((lse, "lse"), (dnll, "dnll"))
    _check_ce(h, w, targets, f32=f32, dh=dh, devices=False)
    p = ce_params_for(h, w)
    need = int(lib().ce_bwd_workspace_bytes(ctypes.byref(p)))
    _check_ce(h, w, targets, f32=f32, dh=dh, workspace=workspace, need_ws=need)
    dh = torch.empty_like(h) if dh is None else dh
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=h.device)
    st = lib().ce_bwd(ctypes.byref(p), _ptr(h), _ptr(w), _ptr(targets), _ptr(lse), _ptr(dnll), _ptr(dh),
                      _ptr(workspace), workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    if st:
        raise AttnError(st, "ce_bwd")
    return dh
