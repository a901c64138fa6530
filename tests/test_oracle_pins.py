"""Pins for the CPU oracle: printed worked examples, closed forms, library
routines, invariants and brute force.  None of these re-types the formula
under test; each is chosen so that a dropped term, a wrong sign or index, or a
transposed operand in the oracle makes at least one of them fail.
"""
import itertools
import math

import numpy as np
import pytest
import torch

from golden.fixtures import load
from oracle import (MaskMod, ScoreMod, attention, blockwise_attention, build_block_mask,
                    sparsity, to_dense, visible_cells)
from oracle.blockmask import tile_classes

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _attn(q, k, v, score=ScoreMod(), mask=MaskMod(), q_offset=0, scale=None):
    D = q.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    return attention(q, k, v, scale=scale, score=score, mask=mask, q_offset=q_offset)


# ---------------------------------------------------------------- P1: ordering
def test_softcap_then_mask_order():
    fx = load("softcap_order.txt")
    cap = fx["cap"]
    # q = 0 makes every raw score 0, the page's scores; causal at q_pos 0 allows
    # key 0 and hides key 1, the page's allow list; one-hot values expose weights.
    q = np.zeros((1, 1, 1, 4))
    k = np.random.default_rng(0).standard_normal((1, 1, 2, 4))
    v = np.eye(2).reshape(1, 1, 2, 2)
    out, lse = _attn(q, k, v, ScoreMod("softcap", cap=cap), MaskMod("causal"))
    assert np.allclose(out[0, 0, 0], fx["correct"], atol=0, rtol=0)
    # the wrong order would turn -inf into -cap: the page's printed weights
    wrong = np.array([0.0, -cap])
    w = np.exp(wrong - wrong.max())
    w /= w.sum()
    assert np.allclose(np.round(w, 6), fx["mask_then_cap"])
    assert not np.allclose(out[0, 0, 0], w)


# ------------------------------------------------------- P2: 6-token 2x2 tiles
def test_causal6_tile_classes_and_counts():
    fx = load("causal6_tile2.txt")
    n, t = fx["length"], fx["tile"]
    m = MaskMod("causal")
    bm = build_block_mask(m, n, n, t, t)
    assert tile_classes(bm)[0, 0].tolist() == fx["grid"]
    cls = tile_classes(bm)[0, 0].ravel().tolist()
    assert {c: cls.count(c) for c in "FP0"} == fx["counts"]
    vis = visible_cells(m, 0, 0, n, n, 0, 0, n, 0, n)
    assert vis.size == fx["connections"]
    assert vis.sum() == fx["visible"]
    visited = (bm["kv_num_blocks"].sum() + bm["full_kv_num_blocks"].sum()) * t * t
    assert visited == fx["visited_cells"]
    dense_tiles = np.kron(to_dense(bm)[0, 0], np.ones((t, t), dtype=int)).astype(bool)
    assert (dense_tiles & ~vis).sum() == fx["masked_in_visited"]


# -------------------------------------------- P3: 16 tokens, 3 docs, block 4
def test_doc16_dense_grids_and_sparsity():
    fx = load("doc16_block4.txt")
    doc = np.array(fx["doc_id"], dtype=np.int32)
    n, blk = doc.size, fx["block"]
    for kind, key in (("causal", "causal"), ("doc_causal", "doc_causal")):
        bm = build_block_mask(MaskMod(kind, doc_id=doc), n, n, blk, blk)
        assert to_dense(bm)[0, 0].tolist() == fx[key + "_dense"]
        assert round(sparsity(bm), 2) == fx[key + "_sparsity"]


def test_doc16_attention_matches_sdpa_with_dense_mask():
    fx = load("doc16_block4.txt")
    doc = np.array(fx["doc_id"], dtype=np.int32)
    n = doc.size
    g = torch.Generator().manual_seed(0)
    q, k, v = (torch.randn(1, 2, n, 8, generator=g, dtype=torch.float64) for _ in range(3))
    dense = torch.from_numpy((doc[:, None] == doc[None, :]) & np.tri(n, dtype=bool))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=dense)
    out, _ = _attn(q.numpy(), k.numpy(), v.numpy(), mask=MaskMod("doc_causal", doc_id=doc))
    assert np.abs(out - ref.numpy()).max() < 1e-12


# ------------------------------------------------- P4: (T+1)/(2T) closed form
@pytest.mark.parametrize("n,blk", [(256, 64), (64, 8), (96, 32), (40, 4)])
def test_square_causal_closed_form(n, blk):
    T = n // blk
    bm = build_block_mask(MaskMod("causal"), n, n, blk, blk)
    visited = bm["kv_num_blocks"].sum() + bm["full_kv_num_blocks"].sum()
    assert visited == T * (T + 1) // 2
    assert bm["kv_num_blocks"].sum() == T          # one diagonal tile per row
    assert math.isclose(visited / T ** 2, (T + 1) / (2 * T))


def test_nonsquare_tile_causal_counts():
    # 128 x 64 tiles on L = S = 2048: Q-block row i holds 2i full and 2 partial tiles
    bm = build_block_mask(MaskMod("causal"), 2048, 2048, 128, 64)
    assert bm["full_kv_num_blocks"][0, 0].tolist() == [2 * i for i in range(16)]
    assert bm["kv_num_blocks"][0, 0].tolist() == [2] * 16
    assert bm["full_kv_num_blocks"].sum() == 240 and bm["kv_num_blocks"].sum() == 32


# -------------------------------------------------- P5: decode offset + window
def test_decode_offset_window_visible_keys():
    fx = load("decode_offset_window.txt")
    m = MaskMod("causal_window_sinks", window=fx["window"], sinks=0)
    vis = visible_cells(m, 0, 0, 1, fx["valid_length"], fx["q_offset"] , fx["q_idx"], 1, 0, fx["capacity"])
    assert np.nonzero(vis[0])[0].tolist() == fx["visible"]


def test_window_sink_rule_edges():
    # the tensorcad generated mask_mod_1: causal, 1024-key window, 4 sinks
    m = MaskMod("causal_window_sinks", window=1024, sinks=4)
    q = 2000
    cases = {3: True, 4: False, 975: False, 976: False, 977: True, 2000: True, 2001: False}
    for kv, want in cases.items():
        assert bool(m(0, 0, q, kv)) is want, kv


# ------------------------------------------- P6: bottom-right decode alignment
def test_bottom_right_decode_weights():
    fx = load("bottom_right_decode.txt")
    q = np.ones((1, 1, 1, 4))
    k = np.ones((1, 1, 5, 4))
    v = np.eye(5).reshape(1, 1, 5, 5)
    br, _ = _attn(q, k, v, mask=MaskMod("causal"), q_offset=5 - 1)
    tl, _ = _attn(q, k, v, mask=MaskMod("causal"), q_offset=0)
    assert br[0, 0, 0].tolist() == fx["bottom_right"]
    assert tl[0, 0, 0].tolist() == fx["top_left"]


# ------------------------------------------- P7: reduction to torch SDPA (fp64)
@pytest.mark.parametrize("B,H,L,S,D", [(2, 4, 128, 128, 64), (1, 3, 7, 19, 5), (2, 2, 33, 33, 16)])
def test_matches_sdpa_noop_and_causal(B, H, L, S, D):
    g = torch.Generator().manual_seed(L * 31 + S)
    q = torch.randn(B, H, L, D, generator=g, dtype=torch.float64)
    k = torch.randn(B, H, S, D, generator=g, dtype=torch.float64)
    v = torch.randn(B, H, S, D + 3, generator=g, dtype=torch.float64)
    F = torch.nn.functional.scaled_dot_product_attention
    out, _ = _attn(q.numpy(), k.numpy(), v.numpy())
    assert np.abs(out - F(q, k, v).numpy()).max() < 1e-12
    # causal, bottom-right aligned: row r sees the first S - L + r + 1 keys
    lower_right = torch.ones(L, S, dtype=torch.bool).tril(diagonal=S - L)
    ref = F(q, k, v, attn_mask=lower_right)
    out, _ = _attn(q.numpy(), k.numpy(), v.numpy(), mask=MaskMod("causal"), q_offset=S - L)
    assert np.abs(out - ref.numpy()).max() < 1e-12
    # explicit scale is used as given
    ref = F(q, k, v, scale=0.37)
    out, _ = _attn(q.numpy(), k.numpy(), v.numpy(), scale=0.37)
    assert np.abs(out - ref.numpy()).max() < 1e-12


@pytest.mark.parametrize("D", [1, 2, 3, 4, 5, 16, 64, 96, 128, 256])
def test_default_scale_is_one_over_sqrt_d_in_float32(D):
    """The default scale (2kiu guide, section 6.2: 1/sqrt(E), E the embedding
    dimension) as the float32 value handed to the kernel: the float32 nearest
    to 1/sqrt(D).  Exact for squares of powers of two; otherwise s is within
    half an ulp of 1/sqrt(D), checked through s^2 * D = 1 to first order, and
    torch's SDPA with its own default scale matches the oracle run with it."""
    from oracle import default_scale
    s = default_scale(D)
    assert np.float32(s) == s
    exact = 1.0 / math.sqrt(D)
    assert abs(s - exact) <= np.spacing(np.float32(exact)) / 2
    if D in (1, 4, 16, 64, 256):
        assert s == {1: 1.0, 4: 0.5, 16: 0.25, 64: 0.125, 256: 0.0625}[D]
    assert abs(s * s * D - 1.0) <= 2 * 2.0 ** -24
    g = torch.Generator().manual_seed(D)
    q, k, v = (torch.randn(1, 1, 9, D, generator=g, dtype=torch.float64) for _ in range(3))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v).numpy()
    out, _ = attention(q.numpy(), k.numpy(), v.numpy(), scale=s, score=ScoreMod(), mask=MaskMod(), q_offset=0)
    # the float32 rounding of the scale moves the result by at most ~1e-7 relative
    assert np.abs(out - ref).max() < 1e-6


def test_lse_matches_torch_logsumexp():
    g = torch.Generator().manual_seed(5)
    q = torch.randn(1, 2, 9, 8, generator=g, dtype=torch.float64)
    k = torch.randn(1, 2, 11, 8, generator=g, dtype=torch.float64)
    v = torch.randn(1, 2, 11, 8, generator=g, dtype=torch.float64)
    s = q @ k.transpose(-1, -2) * 0.5
    vis = torch.ones(9, 11, dtype=torch.bool).tril(diagonal=2)
    ref = torch.logsumexp(s.masked_fill(~vis, float("-inf")), dim=-1)
    _, lse = _attn(q.numpy(), k.numpy(), v.numpy(), mask=MaskMod("causal"), q_offset=2, scale=0.5)
    assert np.abs(lse - ref.numpy()).max() < 1e-12


# ----------------------------------------------------- P8: closed forms, q = 0
def test_uniform_scores_give_prefix_means():
    rng = np.random.default_rng(1)
    L, D = 12, 6
    q = np.zeros((1, 1, L, D))
    k = rng.standard_normal((1, 1, L, D))
    v = rng.standard_normal((1, 1, L, D))
    want = np.cumsum(v[0, 0], axis=0) / np.arange(1, L + 1)[:, None]
    for sc in (ScoreMod(), ScoreMod("softcap", cap=3.0)):
        out, lse = _attn(q, k, v, sc, MaskMod("causal"))
        assert np.abs(out[0, 0] - want).max() < 1e-12
        assert np.abs(lse[0, 0] - np.log(np.arange(1, L + 1))).max() < 1e-12


def test_alibi_geometric_weights():
    # heads = 8, m = 8: the bias slopes are 1/2, 1/4, ..., 1/256
    slopes = [0.5, 0.25, 0.125, 0.0625, 0.03125, 0.015625, 0.0078125, 0.00390625]
    rng = np.random.default_rng(2)
    L, D, H = 10, 4, 8
    q = np.zeros((1, H, L, D))
    k = rng.standard_normal((1, H, L, D))
    v = rng.standard_normal((1, H, L, D))
    out, lse = _attn(q, k, v, ScoreMod("softcap_alibi", cap=7.0, alibi_m=8.0), MaskMod("causal"))
    for h, a in enumerate(slopes):
        r = math.exp(-a)
        for i in range(L):
            w = np.array([r ** (i - j) for j in range(i + 1)])
            assert abs(lse[0, h, i] - math.log((1 - r ** (i + 1)) / (1 - r))) < 1e-12
            assert np.abs(out[0, h, i] - (w @ v[0, h, :i + 1]) / w.sum()).max() < 1e-12


def test_huge_cap_reduces_to_plain_scores():
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((1, 2, 16, 8)) for _ in range(3))
    a, la = _attn(q, k, v, ScoreMod("softcap", cap=1e8), MaskMod("causal"))
    b, lb = _attn(q, k, v, ScoreMod(), MaskMod("causal"))
    assert np.abs(a - b).max() < 1e-9 and np.abs(la - lb).max() < 1e-9


def test_softcap_saturates_at_plus_minus_cap():
    # raw scores +-100 with cap 1 behave like scores +-1: weights are logistic(2)
    q = np.array([[[[10.0]]]])
    k = np.array([[[[10.0], [-10.0]]]])
    v = np.eye(2).reshape(1, 1, 2, 2)
    out, _ = _attn(q, k, v, ScoreMod("softcap", cap=1.0), scale=1.0)
    assert np.abs(out[0, 0, 0] - [0.8807970779778823, 0.11920292202211755]).max() < 1e-12


def test_softcap_half_point():
    # every raw score equal to c*atanh(1/2) is capped to exactly c/2: lse = c/2 + ln n
    c, n = 30.0, 7
    x = c * math.atanh(0.5)
    q = np.ones((1, 1, 1, 1))
    k = np.full((1, 1, n, 1), x)
    v = np.random.default_rng(4).standard_normal((1, 1, n, 3))
    out, lse = _attn(q, k, v, ScoreMod("softcap", cap=c), scale=1.0)
    assert abs(lse[0, 0, 0] - (c / 2 + math.log(n))) < 1e-12
    assert np.abs(out[0, 0, 0] - v[0, 0].mean(axis=0)).max() < 1e-12


# ------------------------------------------------------------ P9: invariants
def test_probability_rows_and_lse_bound():
    rng = np.random.default_rng(6)
    L, S, D = 20, 23, 8
    q = rng.standard_normal((1, 1, L, D))
    k = rng.standard_normal((1, 1, S, D))
    doc = np.repeat(np.arange(4), [5, 6, 7, 5]).astype(np.int32)
    v_eye = np.eye(S).reshape(1, 1, S, S)
    for mask in (MaskMod("causal"), MaskMod("causal_window_sinks", window=5, sinks=2),
                 MaskMod("doc_causal", doc_id=doc), MaskMod("noop")):
        P, lse = _attn(q, k, v_eye, mask=mask, q_offset=S - L)
        P = P[0, 0]
        vis = mask(0, 0, (np.arange(L) + S - L)[:, None], np.arange(S)[None, :])
        live = vis.any(axis=1)
        assert np.abs(P[live].sum(axis=1) - 1).max() < 1e-12
        assert (P[~vis] == 0).all() and (P >= 0).all() and (P <= 1 + 1e-15).all()
        s = (q[0, 0] @ k[0, 0].T) / math.sqrt(D)
        top = np.where(vis, s, -np.inf).max(axis=1)
        assert (lse[0, 0][live] >= top[live] - 1e-12).all()


# ----------------------------------------------------------- P10: empty rows
def test_rows_without_keys_are_zero_and_neg_inf():
    fx = load("empty_row_numerics.txt")
    assert fx["neg_inf_rows"][0] == ["nan"] * 3          # what the naive formula gives
    rng = np.random.default_rng(7)
    L, S, D = 9, 4, 8
    q = rng.standard_normal((1, 2, L, D))
    k = rng.standard_normal((1, 2, S, D))
    v = rng.standard_normal((1, 2, S, D))
    out, lse = _attn(q, k, v, ScoreMod("softcap", cap=5.0), MaskMod("causal"), q_offset=S - L)
    empty = np.arange(L) < L - S
    assert not np.isnan(out).any() and not np.isnan(lse).any()
    assert (out[:, :, empty] == 0).all() and np.isneginf(lse[:, :, empty]).all()
    assert np.isfinite(lse[:, :, ~empty]).all()
    # the live rows fall back to the fixture's pattern: uniform over what they see
    out_u, _ = _attn(np.zeros_like(q), k, np.eye(S).reshape(1, 1, S, S).repeat(2, 1),
                     mask=MaskMod("causal"), q_offset=S - L)
    assert np.allclose(out_u[0, 0, L - S + 1], [0.5, 0.5, 0, 0])


# ------------------------------- brute force: scalar loops in the pages' notation
def _brute(q, k, v, scale, score, mask, q_offset):
    B, Hq, L, D = q.shape
    Hkv, S, Dv = k.shape[1], k.shape[2], v.shape[-1]
    out = np.zeros((B, Hq, L, Dv))
    lse = np.zeros((B, Hq, L))
    for b, h, i in itertools.product(range(B), range(Hq), range(L)):
        kh = h // (Hq // Hkv)
        p = i + q_offset
        terms = []
        for j in range(S):
            if not bool(mask(b, h, p, j)):
                continue
            s = scale * sum(float(q[b, h, i, d]) * float(k[b, kh, j, d]) for d in range(D))
            terms.append((float(score(s, b, h, p, j, Hq)), j))
        if not terms:
            lse[b, h, i] = -math.inf
            continue
        top = max(t for t, _ in terms)
        den = sum(math.exp(t - top) for t, _ in terms)
        for t, j in terms:
            out[b, h, i] += math.exp(t - top) / den * v[b, kh, j]
        lse[b, h, i] = top + math.log(den)
    return out, lse


def _menu(doc):
    scores = [ScoreMod(), ScoreMod("softcap", cap=2.5), ScoreMod("softcap_alibi", cap=4.0, alibi_m=8.0)]
    masks = [MaskMod("noop"), MaskMod("causal"), MaskMod("causal_window_sinks", window=3, sinks=2),
             MaskMod("doc_causal", doc_id=doc)]
    return scores, masks


def test_dense_oracle_equals_scalar_brute_force():
    rng = np.random.default_rng(8)
    B, Hq, Hkv, D = 1, 4, 2, 3
    for L, S in ((5, 7), (7, 7), (8, 3)):
        q = rng.standard_normal((B, Hq, L, D))
        k = rng.standard_normal((B, Hkv, S, D))
        v = rng.standard_normal((B, Hkv, S, 2))
        doc = np.sort(rng.integers(0, 3, size=max(L, S) + S)).astype(np.int32)
        scores, masks = _menu(doc)
        for sc, mk in itertools.product(scores, masks):
            for off in {S - L, 0}:
                if mk.kind == "doc_causal" and off < 0:
                    continue
                a, la = attention(q, k, v, scale=0.7, score=sc, mask=mk, q_offset=off)
                b, lb = _brute(q, k, v, 0.7, sc, mk, off)
                assert np.abs(a - b).max() < 1e-12
                fin = np.isfinite(lb)
                assert (np.isfinite(la) == fin).all() and np.abs(la[fin] - lb[fin]).max() < 1e-12


def _brute_block_mask(mask, L, S, QB, KB, q_offset):
    nQB, nKB = -(-L // QB), -(-S // KB)
    part, full = [], []
    for qb in range(nQB):
        prow, frow = [], []
        for kb in range(nKB):
            seen = 0
            for i in range(qb * QB, qb * QB + QB):
                for j in range(kb * KB, kb * KB + KB):
                    if i < L and j < S and bool(mask(0, 0, i + q_offset, j)):
                        seen += 1
            if seen == QB * KB:
                frow.append(kb)
            elif seen:
                prow.append(kb)
        part.append(prow)
        full.append(frow)
    return part, full


def test_block_mask_equals_cell_loop_and_list_layout():
    rng = np.random.default_rng(9)
    for _ in range(60):
        L, S = int(rng.integers(1, 13)), int(rng.integers(1, 13))
        QB, KB = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        doc = np.sort(rng.integers(0, 4, size=L + S)).astype(np.int32)
        _, masks = _menu(doc)
        for mk in masks:
            for off in {S - L, 0}:
                if mk.kind == "doc_causal" and off < 0:
                    continue
                bm = build_block_mask(mk, L, S, QB, KB, q_offset=off)
                part, full = _brute_block_mask(mk, L, S, QB, KB, off)
                nKB = -(-S // KB)
                for r in range(len(part)):
                    for lst, num, ind in ((part[r], "kv_num_blocks", "kv_indices"),
                                          (full[r], "full_kv_num_blocks", "full_kv_indices")):
                        rest = [x for x in range(nKB) if x not in lst]
                        assert bm[num][0, 0, r] == len(lst)
                        assert bm[ind][0, 0, r].tolist() == lst + rest


# ------------------------------------- P11: block lists lose nothing (exactness)
def test_blockwise_over_lists_equals_dense():
    rng = np.random.default_rng(10)
    for trial in range(40):
        L, S = int(rng.integers(1, 13)), int(rng.integers(1, 13))
        QB, KB = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        Hq, Hkv, D = 2, 1, 3
        q = rng.standard_normal((1, Hq, L, D))
        k = rng.standard_normal((1, Hkv, S, D))
        v = rng.standard_normal((1, Hkv, S, D))
        doc = np.sort(rng.integers(0, 4, size=L + S)).astype(np.int32)
        scores, masks = _menu(doc)
        for sc, mk in itertools.product(scores, masks):
            for off in {S - L, 0}:
                if mk.kind == "doc_causal" and off < 0:
                    continue
                bm = build_block_mask(mk, L, S, QB, KB, q_offset=off)
                cnt = bm["counts"][0, 0]
                d = to_dense(bm)[0, 0]
                assert ((cnt > 0) == (d == 1)).all()
                a, la = attention(q, k, v, scale=0.9, score=sc, mask=mk, q_offset=off)
                b, lb = blockwise_attention(q, k, v, bm, scale=0.9, score=sc, mask=mk, q_offset=off)
                assert np.abs(a - b).max() < 1e-12
                fin = np.isfinite(la)
                assert (np.isfinite(lb) == fin).all() and np.abs(la[fin] - lb[fin]).max() < 1e-12


# ------------------------------------------------------------------ P12: GQA
def test_gqa_equals_repeated_heads_and_sdpa():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, L, S, D = 2, 8, 2, 10, 13, 4
    q = rng.standard_normal((B, Hq, L, D))
    k = rng.standard_normal((B, Hkv, S, D))
    v = rng.standard_normal((B, Hkv, S, D))
    sc, mk = ScoreMod("softcap_alibi", cap=3.0), MaskMod("causal")
    a, la = _attn(q, k, v, sc, mk, q_offset=S - L)
    b, lb = _attn(q, np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1), sc, mk, q_offset=S - L)
    assert np.abs(a - b).max() == 0 and np.abs(la - lb).max() == 0
    F = torch.nn.functional.scaled_dot_product_attention
    ref = F(*(torch.from_numpy(x) for x in (q, k, v)), enable_gqa=True)
    out, _ = _attn(q, k, v)
    assert np.abs(out - ref.numpy()).max() < 1e-12


# ------------------------------------- the menu's program masks and plain ALiBi
# tensorcad "Attention expressions", Examples table; 2kiu guide, section 4.3
# (and_masks folds from all-true with &, or_masks from all-false with |).
def _visible_counts(mask, L, S, q_offset=0, h=0):
    q = np.arange(L)[:, None] + q_offset
    kv = np.arange(S)[None, :]
    return mask(0, h, q, kv).sum(axis=1)


def test_prefix_lm_counts():
    # causal off, "kv <= q or kv < 16": row q sees max(q + 1, 16) keys
    m = MaskMod("program", clauses=((("causal", 0), ("kv_lt", 16)),))
    L = S = 40
    assert list(_visible_counts(m, L, S)) == [max(q + 1, 16) for q in range(L)]


def test_chunked_counts():
    # causal on, "floor(q / C) == floor(kv / C)": row q sees the keys of its own
    # chunk up to itself, q mod C + 1 of them
    C = 8
    m = MaskMod("program", clauses=((("causal", 0),), (("chunk", C),)))
    L = S = 50
    assert list(_visible_counts(m, L, S)) == [q % C + 1 for q in range(L)]


def test_every_fourth_key_counts():
    # causal on, "(q - kv) % 4 == 0": keys q, q-4, ..., floor(q/4) + 1 of them
    m = MaskMod("program", clauses=((("causal", 0),), (("stride", 4),)))
    L = S = 37
    assert list(_visible_counts(m, L, S)) == [q // 4 + 1 for q in range(L)]


def test_half_heads_global_counts():
    # causal on, "h < heads / 2 or q - kv < W" with 4 heads, W = 5
    m = MaskMod("program", clauses=((("causal", 0),), (("head_lt", 2), ("window", 5))))
    L = S = 30
    for h in range(4):
        want = [q + 1 if h < 2 else min(q + 1, 5) for q in range(L)]
        assert list(_visible_counts(m, L, S, h=h)) == want, h


def test_programs_reproduce_the_fixed_menu():
    # and_masks(causal, or_masks(window, sinks)) is the causal window with sinks,
    # and_masks(causal, doc) the document mask; both are pinned above
    rng = np.random.default_rng(21)
    doc = np.repeat(np.arange(5), rng.integers(1, 9, size=5)).astype(np.int32)
    S = len(doc)
    q = np.arange(-3, S)[:, None]
    kv = np.arange(S)[None, :]
    a = MaskMod("program", clauses=((("causal", 0),), (("window", 7), ("kv_lt", 3))))
    b = MaskMod("causal_window_sinks", window=7, sinks=3)
    assert (a(0, 0, q, kv) == b(0, 0, q, kv)).all()
    c = MaskMod("program", clauses=((("causal", 0),), (("doc", 0),)), doc_id=doc)
    d = MaskMod("doc_causal", doc_id=doc)
    q = np.arange(S)[:, None]
    assert (c(0, 0, q, kv) == d(0, 0, q, kv)).all()
    # folding identities: no clause is all-true; a clause is the OR of its predicates
    assert MaskMod("program", clauses=())(0, 0, q, kv).all()
    one = MaskMod("program", clauses=((("causal", 0), ("kv_lt", 2)),))(0, 0, q, kv)
    assert (one == ((kv <= q) | (kv < 2))).all()


def test_negative_positions_floor_semantics():
    # with a negative q_offset the chunk and stride predicates use floor division
    # and a non-negative remainder (Python operators, as on the page)
    m = MaskMod("program", clauses=((("chunk", 3),), (("stride", 2),)))
    for p in range(-7, 7):
        for j in range(0, 9):
            want = (p // 3 == j // 3) and ((p - j) % 2 == 0)
            assert bool(m(0, 0, np.array(p), np.array(j))) == want, (p, j)


def test_uncapped_alibi_geometric_weights():
    # tensorcad Examples, the ALiBi row without a cap: with q = 0 every score is
    # 0, so the weights are r^(i - j), r = e^-slope (same closed form as above)
    rng = np.random.default_rng(22)
    L, D, H = 9, 4, 4
    q = np.zeros((1, H, L, D))
    k = rng.standard_normal((1, H, L, D))
    v = rng.standard_normal((1, H, L, D))
    out, lse = _attn(q, k, v, ScoreMod("alibi", alibi_m=8.0), MaskMod("causal"))
    for h in range(H):
        r = math.exp(-2.0 ** (-8.0 * (h + 1) / H))
        for i in range(L):
            w = np.array([r ** (i - j) for j in range(i + 1)])
            assert abs(lse[0, h, i] - math.log((1 - r ** (i + 1)) / (1 - r))) < 1e-12
            assert np.abs(out[0, h, i] - (w @ v[0, h, :i + 1]) / w.sum()).max() < 1e-12
    # an uncapped score differs from a capped one once scores are large
    q2 = rng.standard_normal((1, H, L, D)) * 6
    a, _ = _attn(q2, k, v, ScoreMod("alibi"), MaskMod("causal"), scale=1.0)
    b, _ = _attn(q2, k, v, ScoreMod("softcap_alibi", cap=1.0), MaskMod("causal"), scale=1.0)
    assert np.abs(a - b).max() > 1e-3


def test_max_scores_closed_forms():
    # row maxima of the scores entering the softmax: with q = 0 and ALiBi the
    # row's own key has bias 0 and every other visible key a negative one
    rng = np.random.default_rng(23)
    L, D, H = 8, 4, 2
    q = np.zeros((1, H, L, D))
    k = rng.standard_normal((1, H, L, D))
    v = rng.standard_normal((1, H, L, D))
    _, lse, mx = attention(q, k, v, scale=0.5, score=ScoreMod("alibi"), mask=MaskMod("causal"), q_offset=0,
                           with_max=True)
    assert np.abs(mx).max() == 0.0
    assert (lse >= mx).all()
    # rows that see no key have max -inf; plain scores: the max is the largest dot
    q3 = rng.standard_normal((1, 1, 4, D))
    k3 = rng.standard_normal((1, 1, 6, D))
    v3 = rng.standard_normal((1, 1, 6, D))
    _, _, mx3 = attention(q3, k3, v3, scale=1.0, score=ScoreMod(), mask=MaskMod("causal"), q_offset=-2,
                          with_max=True)
    dots = q3[0, 0] @ k3[0, 0].T
    assert mx3[0, 0, 0] == -np.inf and mx3[0, 0, 1] == -np.inf
    assert abs(mx3[0, 0, 2] - dots[2, 0]) < 1e-12
    assert abs(mx3[0, 0, 3] - dots[3, :2].max()) < 1e-12
