"""Seeded synthetic workloads for windowed, grouped-query attention.

This module holds shapes and random draws only. It contains none of the
attention arithmetic, so both the HIP path (through the binding) and the fp64
CPU oracle can take their inputs from it without sharing any of the method.

Workloads follow the shapes the pages measure:
  * "Off NVIDIA, you fix the platform yourself" (labs.layer2c.com), record
    entry "Attention backward memory, one sliding-window layer": bf16, 32 query
    heads, a 1,024-token window, 8K to 32K tokens.
  * the mlx-train-perf README, attention-op timing passage: batch 1, 32 query /
    8 KV heads, 8,192 tokens, head_dim 128, causal.
  * the lab's "load" entry: a corpus of transcripts with mean 8,663 tokens and
    longest 30,553, trained 4 per step. That corpus is not available; ragged
    batches are drawn from a lognormal with that mean, clipped to that longest.

Draw order for one workload with seed s (numpy ``default_rng(s)``):
  1. ragged workloads only: 4 sequence lengths,
     ``clip(rint(lognormal(8.9085, 0.5627, 4)), 512, 30553)``;
  2. Q, K, V, dO in that order, each ``standard_normal(shape, float32)`` over
     the packed shape ``[T, H, d]``;
  3. dO is multiplied by the workload's dO scale in fp32;
  4. bf16 workloads round all four tensors to bf16 (round to nearest even,
     done by torch on the CPU). The oracle sees exactly these rounded values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

INT32_MAX = 2**31 - 1

# Lognormal fitted so that 171 draws have mean ~8,663 and a typical maximum
# near the 30,553-token longest transcript of the lab's corpus.
LOGNORMAL_MU = 8.9085
LOGNORMAL_SIGMA = 0.5627
LEN_MIN, LEN_MAX = 512, 30553


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    lengths_q: tuple          # per-sequence query lengths (packed in order)
    lengths_k: tuple          # per-sequence key lengths, each >= the query length
    heads_q: int
    heads_kv: int
    head_dim: int
    window: int               # >= 1; INT32_MAX or >= every key length means none
    causal: bool
    dtype: str                # "f32", "bf16" or "fp16"
    scale: float
    do_scale: float
    seed: int
    lengths_drawn: bool = False  # lengths were the first draw from ``seed``

    @property
    def batch(self) -> int:
        return len(self.lengths_q)

    @property
    def total_q(self) -> int:
        return int(sum(self.lengths_q))

    @property
    def total_k(self) -> int:
        return int(sum(self.lengths_k))

    @property
    def max_seqlen_q(self) -> int:
        return int(max(self.lengths_q)) if self.lengths_q else 0

    @property
    def max_seqlen_k(self) -> int:
        return int(max(self.lengths_k)) if self.lengths_k else 0

    def cu_seqlens_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths_q)]).astype(np.int32)

    def cu_seqlens_k(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths_k)]).astype(np.int32)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def ragged_lengths(seed: int, n: int = 4) -> tuple:
    """Step 1 of the draw order: n lognormal sequence lengths."""
    rng = np.random.default_rng(seed)
    lens = np.clip(np.rint(rng.lognormal(LOGNORMAL_MU, LOGNORMAL_SIGMA, n)), LEN_MIN, LEN_MAX)
    return tuple(int(x) for x in lens)


def _fixed(name, n, hq, hkv, d, window, dtype, scale, do_scale, seed, batch=1):
    return Workload(name, (n,) * batch, (n,) * batch, hq, hkv, d, window, True, dtype,
                    scale, do_scale, seed)


# The five measured workloads, by what they are.
TINY_F32 = _fixed("tiny_f32_n256_w32_gqa2_d64", 256, 2, 1, 64, 32, "f32", 1 / 8, 1.0, 1)
GQA_2K = _fixed("bf16_n2048_w1024_32q8kv_d128", 2048, 32, 8, 128, 1024, "bf16",
                1 / math.sqrt(128), 0.1, 2)
CAUSAL_8K = _fixed("bf16_n8192_causal_32q8kv_d128", 8192, 32, 8, 128, 8192, "bf16",
                   1 / math.sqrt(128), 0.1, 3)
SWA_32K = _fixed("bf16_n32768_w1024_32q8kv_d128", 32768, 32, 8, 128, 1024, "bf16",
                 1 / math.sqrt(128), 0.1, 4)
# The memory-probe shape of one sliding-window layer (head_dim 256, 32 query /
# 16 KV heads, window 1024, bf16), at its longest length; 8K and 16K are the
# same workload with shorter sequences.
GEMMA_32K = _fixed("bf16_n32768_w1024_32q16kv_d256", 32768, 32, 16, 256, 1024, "bf16",
                   1 / math.sqrt(256), 0.1, 6)


def varlen_workload(seed: int = 5, window: int = 1024) -> Workload:
    lens = ragged_lengths(seed)
    return Workload(f"bf16_varlen4_w{window}_32q8kv_d128", lens, lens, 32, 8, 128, window,
                    True, "bf16", 1 / math.sqrt(128), 0.1, seed, lengths_drawn=True)


VARLEN_4 = varlen_workload()

WORKLOADS = {w.name: w for w in (TINY_F32, GQA_2K, CAUSAL_8K, SWA_32K, VARLEN_4, GEMMA_32K)}

# Edge sweep windows for the ragged batch: 1, around one 128-key tile, and the
# longest sequence (equivalent to plain causal).
VARLEN_SWEEP_WINDOWS = (1, 127, 128, 129, max(VARLEN_4.lengths_k))


def _round_16(x: np.ndarray, dtype: str) -> np.ndarray:
    import torch  # plumbing only: torch's fp32 -> bf16 / fp16 casts round to nearest even

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    dt = torch.bfloat16 if dtype == "bf16" else torch.float16
    return t.to(dt).to(torch.float32).numpy()


def make_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """Draw Q, K, V, dO for workload ``w`` (fp32 arrays; bf16- or
    fp16-representable values for those dtypes) plus the int32 cumulative
    offsets.

    The ragged length draw (step 1) is made by :func:`varlen_workload`, with the
    same generator state the tensors then continue from, so that a ragged
    workload built from seed s and its tensors come from one stream.
    """
    s = w.seed if seed is None else seed
    rng = np.random.default_rng(s)
    if w.lengths_drawn and s == w.seed:
        # one stream: the lengths were the first draw from this seed
        rng.lognormal(LOGNORMAL_MU, LOGNORMAL_SIGMA, w.batch)
    tq, tk, hq, hkv, d = w.total_q, w.total_k, w.heads_q, w.heads_kv, w.head_dim
    q = rng.standard_normal((tq, hq, d), dtype=np.float32)
    k = rng.standard_normal((tk, hkv, d), dtype=np.float32)
    v = rng.standard_normal((tk, hkv, d), dtype=np.float32)
    do = rng.standard_normal((tq, hq, d), dtype=np.float32)
    if w.do_scale != 1.0:
        do *= np.float32(w.do_scale)
    if w.dtype in ("bf16", "fp16"):
        q, k, v, do = (_round_16(a, w.dtype) for a in (q, k, v, do))
    return dict(q=q, k=k, v=v, do=do, cu_q=w.cu_seqlens_q(), cu_k=w.cu_seqlens_k())


def small_case(lengths_q: Sequence[int], lengths_k: Optional[Sequence[int]] = None, *,
               heads_q=2, heads_kv=1, head_dim=64, window=INT32_MAX, causal=True,
               dtype="f32", scale=None, do_scale=1.0, seed=0) -> Workload:
    """A custom (test-sized) workload with explicit lengths."""
    lengths_k = tuple(lengths_q) if lengths_k is None else tuple(lengths_k)
    if scale is None:
        scale = 1 / math.sqrt(head_dim)
    return Workload(f"case_s{seed}", tuple(int(x) for x in lengths_q),
                    tuple(int(x) for x in lengths_k), heads_q, heads_kv, head_dim, window,
                    causal, dtype, float(scale), do_scale, seed)


# ---------------------------------------------------------------- masks
# An arbitrary boolean mask combined with the window: one matrix per packed
# batch, shared by every head. Row t is packed query token t; column j is key j
# of that token's sequence (0-based within the sequence). The C ABI takes it
# bit-packed: row t is ``row_words`` uint32 words, bit j % 32 of word j // 32
# holds column j; ``row_words`` is a multiple of 4 (16-byte rows).
# Mask draws use their own generator, ``default_rng(seed)``, independent of
# the tensor draw.

def mask_row_words(max_len_k: int) -> int:
    """Words per packed row: ceil(max_len_k / 32) rounded up to a multiple of 4."""
    words = (max(int(max_len_k), 1) + 31) // 32
    return (words + 3) // 4 * 4


def random_mask(w: Workload, density: float, seed: int, empty_rows: int = 0) -> np.ndarray:
    """Boolean [T_q, max L_k]: each cell allowed with probability ``density``;
    ``empty_rows`` rows, picked at random, allow no key at all."""
    rng = np.random.default_rng(seed)
    m = rng.random((w.total_q, max(w.lengths_k, default=1))) < density
    if empty_rows:
        m[rng.choice(w.total_q, size=min(empty_rows, w.total_q), replace=False)] = False
    return m


def pack_mask(mask: np.ndarray, row_words: Optional[int] = None) -> np.ndarray:
    """uint32 [T_q, row_words] from a boolean [T_q, W] mask (bit j % 32 of word
    j // 32 is column j)."""
    mask = np.asarray(mask, dtype=bool)
    words = mask_row_words(mask.shape[1]) if row_words is None else int(row_words)
    padded = np.zeros((mask.shape[0], words * 32), dtype=bool)
    padded[:, :mask.shape[1]] = mask
    bits = padded.reshape(mask.shape[0], words, 32).astype(np.uint64)
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    return (bits * weights).sum(axis=2).astype(np.uint32)


def unpack_rows(bits: np.ndarray, rows, width: int) -> np.ndarray:
    """Boolean [len(rows), width] from packed rows ``rows`` of ``bits``."""
    sel = np.ascontiguousarray(np.asarray(bits, dtype=np.uint32)[np.asarray(rows, dtype=np.int64)])
    as_bytes = sel.astype("<u4").view(np.uint8)   # word w's byte b holds columns 32 w + 8 b ..
    return np.unpackbits(as_bytes, axis=1, bitorder="little")[:, :width].astype(bool)


class PackedMaskRows:
    """Boolean row view of a packed mask: ``m[rows]`` unpacks only those rows,
    so a mask over tens of thousands of tokens never exists as booleans."""

    def __init__(self, bits: np.ndarray, width: int):
        self.bits, self.width = bits, int(width)

    def __getitem__(self, rows):
        return unpack_rows(self.bits, np.atleast_1d(rows), self.width)


def document_mask_bits(w: Workload, doc_lengths: Sequence[Sequence[int]], row_words: Optional[int] = None) -> np.ndarray:
    """Packed block-diagonal mask: sequence b's keys are split into documents
    of lengths ``doc_lengths[b]`` (summing to L_k(b)); the query at key position
    p = i + L_k - L_q may see key j only inside p's document."""
    words = mask_row_words(max(w.lengths_k, default=1)) if row_words is None else int(row_words)
    bits = np.zeros((w.total_q, words), dtype=np.uint32)
    full = np.uint32(0xFFFFFFFF)
    t = 0
    for b in range(w.batch):
        lq, lk = w.lengths_q[b], w.lengths_k[b]
        docs = [int(x) for x in doc_lengths[b]]
        assert sum(docs) == lk, "documents must cover the sequence's keys"
        starts = np.cumsum([0] + docs)
        for d in range(len(docs)):
            a, e = int(starts[d]), int(starts[d + 1])  # keys [a, e)
            # queries whose position p lies in [a, e)
            i0, i1 = max(0, a - (lk - lq)), max(0, e - (lk - lq))
            if i1 <= i0:
                continue
            row = np.zeros(words, dtype=np.uint32)
            for wd in range(a // 32, (e + 31) // 32):
                lo, hi = max(a, 32 * wd) - 32 * wd, min(e, 32 * wd + 32) - 32 * wd
                span = full if hi - lo == 32 else np.uint32(((1 << (hi - lo)) - 1) << lo)
                row[wd] = span
            bits[t + i0:t + i1] = row
        t += lq
    return bits


def document_lengths(seed: int, total: int) -> list:
    """Documents drawn like the corpus's transcripts (the lognormal above,
    clipped to [LEN_MIN, LEN_MAX]) until ``total`` keys are covered; the last
    one is cut to fit."""
    rng = np.random.default_rng(seed)
    out, left = [], int(total)
    while left > 0:
        n = int(np.clip(np.rint(rng.lognormal(LOGNORMAL_MU, LOGNORMAL_SIGMA)), LEN_MIN, LEN_MAX))
        out.append(min(n, left))
        left -= out[-1]
    return out


def short_document_lengths(seed: int, total: int, longest: int = 512) -> list:
    """Short documents, lengths uniform on [64, longest], drawn until ``total``
    keys are covered (the last one cut to fit): packed rows in which most of
    a 1,024-token window's tiles belong to other documents."""
    rng = np.random.default_rng(seed)
    out, left = [], int(total)
    while left > 0:
        n = int(rng.integers(64, longest + 1))
        out.append(min(n, left))
        left -= out[-1]
    return out


# ------------------------------------------- linear cross-entropy (second workload)
# The mlx-train-perf README measures its loss layer at n = 8,192 tokens,
# vocabulary 151,936, hidden size 4,096, bf16. The hidden states and head are
# synthetic: H ~ N(0, 1), W ~ N(0, 1) / sqrt(D) (so that the logits are of
# order one), targets uniform over the vocabulary, upstream gradients N(0, 1)
# (tests) or the mean loss's 1/n (bench). Draw order from default_rng(seed):
# H, W, targets, dnll; 16-bit dtypes round H and W to nearest even.

@dataclasses.dataclass(frozen=True)
class CEWorkload:
    name: str
    n: int            # tokens
    vocab: int        # V
    hidden: int       # D
    dtype: str        # "bf16", "fp16" or "f32"
    seed: int


CE_BENCH = CEWorkload("ce_bf16_n8192_v151936_d4096", 8192, 151936, 4096, "bf16", 7)


def make_ce_inputs(w: CEWorkload, mean_dnll: bool = False) -> dict:
    rng = np.random.default_rng(w.seed)
    h = rng.standard_normal((w.n, w.hidden), dtype=np.float32)
    head = rng.standard_normal((w.vocab, w.hidden), dtype=np.float32) * np.float32(1 / math.sqrt(w.hidden))
    targets = rng.integers(0, w.vocab, w.n, dtype=np.int64).astype(np.int32)
    dnll = rng.standard_normal(w.n, dtype=np.float32)
    if mean_dnll:
        dnll[:] = np.float32(1.0 / w.n)
    if w.dtype in ("bf16", "fp16"):
        h, head = _round_16(h, w.dtype), _round_16(head, w.dtype)
    return dict(h=h, w=head, targets=targets, dnll=dnll)
