"""Pins for the backward oracle and the Q-side block lists.

The gradients are checked against central finite differences of the forward
oracle (itself pinned elsewhere), which catches any dropped term, wrong sign,
missing scale or score derivative, transposed operand or wrong GQA sum; and
against closed forms of special cases (one visible key per row, equal keys,
zero queries, shift invariance of the softmax).  The Q-side lists are checked
against the transpose of the tile grid printed on the pages and against
brute-force column scans of the tile classes.
"""
import math

import numpy as np
import pytest

from golden.fixtures import load
from oracle import (MaskMod, ScoreMod, attention, attention_backward, build_block_mask,
                    transpose_block_mask)
from oracle.blockmask import tile_classes


def _inputs(seed, B, Hq, Hkv, L, S, D, qscale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, L, D)) * qscale
    k = rng.standard_normal((B, Hkv, S, D))
    v = rng.standard_normal((B, Hkv, S, D))
    do = rng.standard_normal((B, Hq, L, D))
    return q, k, v, do


def _loss(q, k, v, do, scale, score, mask, q_offset):
    out, _ = attention(q, k, v, scale=scale, score=score, mask=mask, q_offset=q_offset)
    return float((out * do).sum())


def _fd_grad(x, f, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + h
        fp = f()
        x[i] = old - h
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


DOC = np.array([0, 0, 0, 1, 1, 2, 2, 2, 2, 3, 3, 3], dtype=np.int32)

FD_CASES = [
    ("none_causal_gqa", ScoreMod(), MaskMod("causal"), 2),
    ("softcap_window", ScoreMod("softcap", cap=1.5), MaskMod("causal_window_sinks", window=3, sinks=1), 2),
    ("softcap_alibi_noop", ScoreMod("softcap_alibi", cap=2.0, alibi_m=8.0), MaskMod("noop"), 0),
    ("alibi_doc", ScoreMod("alibi", alibi_m=4.0), MaskMod("doc_causal", doc_id=DOC), 3),
    ("program_empty_rows", ScoreMod("softcap", cap=3.0),
     MaskMod("program", clauses=((("causal", 0),), (("window", 2), ("kv_lt", 1)))), -2),
]


@pytest.mark.parametrize("name,score,mask,q_offset", FD_CASES, ids=[c[0] for c in FD_CASES])
def test_gradients_match_finite_differences(name, score, mask, q_offset):
    B, Hq, Hkv, L, S, D = 1, 4, 2, 5, 7, 4
    q, k, v, do = _inputs(11, B, Hq, Hkv, L, S, D, qscale=1.5)
    scale = 0.8
    dq, dk, dv = attention_backward(q, k, v, do, scale=scale, score=score, mask=mask, q_offset=q_offset)
    f = lambda: _loss(q, k, v, do, scale, score, mask, q_offset)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        fd = _fd_grad(x, f)
        assert np.allclose(g, fd, rtol=1e-6, atol=1e-7), (name, np.abs(g - fd).max())


def test_per_batch_offsets_and_lengths_match_finite_differences():
    # per-batch query offsets and filled lengths (decode section of the blog),
    # through the forward oracle's own per-batch handling
    B, Hq, Hkv, L, S, D = 2, 2, 1, 4, 7, 4
    q, k, v, do = _inputs(17, B, Hq, Hkv, L, S, D, qscale=1.2)
    q_offsets, kv_lens = [2, -1], [5, 7]
    score, mask = ScoreMod("softcap", cap=2.5), MaskMod("causal")
    dq, dk, dv = attention_backward(q, k, v, do, scale=0.9, score=score, mask=mask, q_offset=q_offsets,
                                    kv_len=kv_lens)

    def f():
        out, _ = attention(q, k, v, scale=0.9, score=score, mask=mask, q_offset=q_offsets, kv_len=kv_lens)
        return float((out * do).sum())

    for x, g in ((q, dq), (k, dk), (v, dv)):
        fd = _fd_grad(x, f)
        assert np.allclose(g, fd, rtol=1e-6, atol=1e-7), np.abs(g - fd).max()
    # keys past a batch's filled length get nothing
    assert np.all(dk[0, :, 5:] == 0) and np.all(dv[0, :, 5:] == 0)


def test_filled_length_equals_truncated_cache():
    # kv_len = n is the same problem as a cache holding only the first n keys
    q, k, v, do = _inputs(19, 1, 4, 2, 6, 10, 8)
    kw = dict(scale=0.6, score=ScoreMod("alibi", alibi_m=4.0), mask=MaskMod("causal"), q_offset=3)
    dq, dk, dv = attention_backward(q, k, v, do, kv_len=7, **kw)
    dq2, dk2, dv2 = attention_backward(q, k[:, :, :7], v[:, :, :7], do, **kw)
    assert np.allclose(dq, dq2, rtol=0, atol=1e-13)
    assert np.allclose(dk[:, :, :7], dk2, rtol=0, atol=1e-13) and np.all(dk[:, :, 7:] == 0)
    assert np.allclose(dv[:, :, :7], dv2, rtol=0, atol=1e-13) and np.all(dv[:, :, 7:] == 0)


def test_empty_rows_have_zero_query_gradient():
    # q_offset -2 under causal: rows 0 and 1 see no key
    q, k, v, do = _inputs(3, 1, 2, 2, 4, 6, 8)
    dq, dk, dv = attention_backward(q, k, v, do, scale=0.5, score=ScoreMod(), mask=MaskMod("causal"), q_offset=-2)
    assert np.all(dq[:, :, :2] == 0)
    # the same keys without those rows give the same K/V gradients
    dq2, dk2, dv2 = attention_backward(q[:, :, 2:], k, v, do[:, :, 2:], scale=0.5, score=ScoreMod(),
                                       mask=MaskMod("causal"), q_offset=0)
    assert np.allclose(dk, dk2, rtol=0, atol=1e-13) and np.allclose(dv, dv2, rtol=0, atol=1e-13)


def test_single_visible_key_closed_form():
    # window 1: row i sees only key q_pos = i + 3, so P = 1 and out_i = v_{i+3};
    # dv of that key is dO_i, and q, k receive nothing
    q, k, v, do = _inputs(5, 1, 2, 1, 4, 7, 8)
    mask = MaskMod("causal_window_sinks", window=1, sinks=0)
    dq, dk, dv = attention_backward(q, k, v, do, scale=1.0, score=ScoreMod("softcap", cap=2.0), mask=mask,
                                    q_offset=3)
    assert np.allclose(dq, 0, atol=1e-14) and np.allclose(dk, 0, atol=1e-14)
    expect = np.zeros_like(v)
    expect[0, 0, 3:7] = do[0, 0] + do[0, 1]      # both query heads share the K/V head
    assert np.allclose(dv, expect, rtol=0, atol=1e-14)


def test_equal_keys_give_zero_query_gradient():
    # all keys equal: every visible score of a row is the same constant, which
    # the softmax ignores, so the loss does not depend on q
    q, k, v, do = _inputs(7, 1, 2, 2, 6, 6, 8)
    k[:] = k[:, :, :1]
    for score in (ScoreMod(), ScoreMod("softcap", cap=2.0)):
        dq, _, _ = attention_backward(q, k, v, do, scale=0.7, score=score, mask=MaskMod("causal"), q_offset=0)
        assert np.allclose(dq, 0, atol=1e-13)


def test_zero_queries_closed_form():
    # q = 0: uniform weights 1/n_i over the n_i visible keys, dk = 0 and
    # dv_j = sum over rows i that see j of dO_i / n_i
    _, k, v, do = _inputs(9, 1, 1, 1, 5, 5, 4)
    q = np.zeros((1, 1, 5, 4))
    dq, dk, dv = attention_backward(q, k, v, do, scale=1.0, score=ScoreMod(), mask=MaskMod("causal"), q_offset=0)
    assert np.allclose(dk, 0, atol=1e-15)
    expect = np.zeros_like(v)
    for i in range(5):
        for j in range(i + 1):
            expect[0, 0, j] += do[0, 0, i] / (i + 1)
    assert np.allclose(dv, expect, rtol=0, atol=1e-14)


@pytest.mark.parametrize("score", [ScoreMod(), ScoreMod("alibi", alibi_m=8.0)], ids=["none", "alibi"])
def test_key_gradients_sum_to_zero_without_cap(score):
    # shifting every score of a row by a constant changes nothing, so each row's
    # score gradients sum to zero, and so does sum_j dk_j when g' = 1
    q, k, v, do = _inputs(13, 2, 4, 2, 9, 11, 8)
    _, dk, _ = attention_backward(q, k, v, do, scale=0.3, score=score, mask=MaskMod("causal"), q_offset=2)
    assert np.allclose(dk.sum(axis=2), 0, atol=1e-12)


def test_value_gradient_is_linear_in_upstream():
    q, k, v, do = _inputs(17, 1, 2, 1, 6, 8, 4)
    m = MaskMod("causal_window_sinks", window=3, sinks=2)
    s = ScoreMod("softcap_alibi", cap=2.0)
    g1 = attention_backward(q, k, v, do, scale=0.5, score=s, mask=m, q_offset=2)
    g2 = attention_backward(q, k, v, 3.0 * do, scale=0.5, score=s, mask=m, q_offset=2)
    for a, b in zip(g1, g2):
        assert np.allclose(3.0 * a, b, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------- Q-side block lists
def test_transposed_lists_of_printed_grid():
    fx = load("causal6_tile2.txt")
    n, t = fx["length"], fx["tile"]
    bm = build_block_mask(MaskMod("causal"), n, n, t, t)
    tq = transpose_block_mask(bm)
    grid = np.array(fx["grid"])          # rows Q blocks, columns KV blocks
    cols = grid.T                        # rows KV blocks, columns Q blocks
    for kb in range(cols.shape[0]):
        part = [qb for qb in range(cols.shape[1]) if cols[kb, qb] == "P"]
        full = [qb for qb in range(cols.shape[1]) if cols[kb, qb] == "F"]
        assert tq["q_num_blocks"][0, 0, kb] == len(part)
        assert tq["full_q_num_blocks"][0, 0, kb] == len(full)
        assert tq["q_indices"][0, 0, kb, :len(part)].tolist() == part
        assert tq["full_q_indices"][0, 0, kb, :len(full)].tolist() == full


def test_transposed_lists_brute_force():
    doc = np.repeat(np.arange(7), [5, 40, 3, 70, 1, 60, 21]).astype(np.int32)
    cases = [
        (MaskMod("causal_window_sinks", window=40, sinks=4), 150, 200, 32, 16, 1, 1, 50),
        (MaskMod("doc_causal", doc_id=doc), 200, 200, 16, 32, 1, 1, 0),
        (MaskMod("program", clauses=((("head_lt", 1), ("chunk", 24)),)), 90, 70, 16, 8, 2, 2, 3),
    ]
    for mask, L, S, qb, kb, B, H, off in cases:
        bm = build_block_mask(mask, L, S, qb, kb, B=B, H=H, q_offset=off)
        tq = transpose_block_mask(bm)
        cls = tile_classes(bm)
        nQB, nKB = cls.shape[2], cls.shape[3]
        for b in range(B):
            for h in range(H):
                for c in range(nKB):
                    for tag, num, ind in (("P", "q_num_blocks", "q_indices"), ("F", "full_q_num_blocks", "full_q_indices")):
                        on = [r for r in range(nQB) if cls[b, h, r, c] == tag]
                        off_ = [r for r in range(nQB) if cls[b, h, r, c] != tag]
                        assert tq[num][b, h, c] == len(on)
                        assert tq[ind][b, h, c].tolist() == on + off_


def test_row_chunks_change_nothing():
    q, k, v, do = _inputs(21, 2, 4, 2, 37, 29, 8)
    kw = dict(scale=0.6, score=ScoreMod("softcap_alibi", cap=2.0), mask=MaskMod("causal_window_sinks", window=7,
                                                                                 sinks=2), q_offset=3)
    whole = attention_backward(q, k, v, do, **kw)
    parts = attention_backward(q, k, v, do, row_chunk=5, **kw)
    for a, b in zip(whole, parts):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-13)
