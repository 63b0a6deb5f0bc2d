"""The synthetic workloads use the shapes the pages print (tests/golden)."""
import json
import os

import numpy as np

from sliding_window_flash_amd import workloads as W

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_shapes.json")))


def test_window_and_token_counts_come_from_the_pages():
    assert W.SWA_32K.window == GOLDEN["sliding_window_tokens"]["value"]
    assert W.SWA_32K.max_seqlen_q in GOLDEN["memory_probe_tokens"]["value"]
    op = GOLDEN["op_timing_shape"]["value"]
    c = W.CAUSAL_8K
    assert (c.batch, c.heads_q, c.heads_kv, c.max_seqlen_q, c.head_dim) == (
        op["batch"], op["heads_q"], op["heads_kv"], op["tokens"], op["head_dim"])
    assert c.window >= c.max_seqlen_k  # plain causal
    probe = GOLDEN["memory_probe_heads"]["value"]
    g = W.GEMMA_32K
    assert (g.heads_q, g.heads_kv, g.head_dim, g.dtype) == (
        probe["heads_q"], probe["heads_kv"], probe["head_dim"], probe["dtype"])
    assert g.max_seqlen_q == max(GOLDEN["memory_probe_tokens"]["value"])
    assert g.window == GOLDEN["sliding_window_tokens"]["value"]


def test_ragged_lengths_follow_the_corpus_statistics():
    corpus = GOLDEN["corpus_lengths"]["value"]
    v = W.VARLEN_4
    assert v.batch == corpus["per_step"]
    assert v.lengths_q == (4709, 3510, 6430, 9368)  # seed 5, numpy default_rng
    assert all(W.LEN_MIN <= n <= corpus["longest"] for n in v.lengths_q)
    # the lognormal's mean matches the corpus mean to within 1%
    mean = np.exp(W.LOGNORMAL_MU + W.LOGNORMAL_SIGMA ** 2 / 2)
    assert abs(mean - corpus["mean"]) / corpus["mean"] < 0.01


def test_inputs_are_seeded_and_bf16_representable():
    a = W.make_inputs(W.TINY_F32)
    b = W.make_inputs(W.TINY_F32)
    for k in a:
        assert np.array_equal(a[k], b[k])
    w = W.small_case([33], heads_q=2, heads_kv=1, head_dim=8, dtype="bf16", do_scale=0.1, seed=3)
    x = W.make_inputs(w)
    for k in ("q", "k", "v", "do"):
        bits = x[k].view(np.uint32)
        assert np.all(bits & 0xFFFF == 0), k
    x = W.make_inputs(w.replace(dtype="fp16"))
    for k in ("q", "k", "v", "do"):
        assert np.array_equal(x[k].astype(np.float16).astype(np.float32), x[k]), k


def test_mask_packing_bit_order():
    """Bit j % 32 of word j // 32 holds column j; rows are padded to 4 words."""
    m = np.zeros((2, 70), bool)
    m[0, [0, 31, 32]] = True
    m[1, 69] = True
    b = W.pack_mask(m)
    assert b.shape == (2, 4) and b.dtype == np.uint32
    assert b[0].tolist() == [0x80000001, 0x1, 0, 0]
    assert b[1].tolist() == [0, 0, 0x20, 0]
    assert np.array_equal(W.unpack_rows(b, [0, 1], 70), m)
    assert W.mask_row_words(1) == 4 and W.mask_row_words(128) == 4 and W.mask_row_words(129) == 8


def test_document_mask_rows():
    """Query i (key position p = i + L_k - L_q) sees exactly the keys of p's document."""
    w = W.small_case([5, 7], [6, 9], window=3, seed=1)
    docs = [[2, 4], [3, 3, 3]]
    got = W.unpack_rows(W.document_mask_bits(w, docs), range(w.total_q), 9)
    t = 0
    for b in range(w.batch):
        lq, lk = w.lengths_q[b], w.lengths_k[b]
        owner = np.repeat(np.arange(len(docs[b])), docs[b])
        for i in range(lq):
            want = np.zeros(9, bool)
            want[:lk] = owner == owner[i + lk - lq]
            assert np.array_equal(got[t + i], want), (b, i)
        t += lq
    assert sum(W.document_lengths(7, 32768)) == 32768
