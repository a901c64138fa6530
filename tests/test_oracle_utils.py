"""Pins for the oracle's BlockMask utilities (slicing, cropping, the pooled
grid and its ASCII picture), against the tile grid printed on the pages and
against rebuilding the mask from its definition."""
import numpy as np
import pytest

from golden.fixtures import load
from oracle import (MaskMod, adjust_block_mask, build_block_mask, grid_classes, slice_block_mask, to_dense,
                    to_string)
from oracle.blockmask import tile_classes

LISTS = ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices")


def test_picture_of_the_printed_grid():
    # the charlestar blog's length-6 causal grid with 2x2 tiles: F full, P partial, 0 skipped
    fx = load("causal6_tile2.txt")
    bm = build_block_mask(MaskMod("causal"), fx["length"], fx["length"], fx["tile"], fx["tile"])
    glyph = {"F": "█", "P": "░", "0": " "}
    expect = ["b=0 h=0"] + ["".join(glyph[c] for c in row) for row in fx["grid"]]
    assert to_string(bm) == "\n".join(expect)
    # the same grid pooled 2x2: windows mixing classes draw as partial
    assert grid_classes(bm, 2, 2)[0, 0].tolist() == [[1, 0], [2, 1]]
    # a grid no smaller than the tile grid is the tile grid
    code = {"F": 2, "P": 1, "0": 0}
    assert grid_classes(bm, 3, 3)[0, 0].tolist() == [[code[c] for c in row] for row in fx["grid"]]


def test_picture_limit_and_pooling_extremes():
    bm = build_block_mask(MaskMod("causal_window_sinks", window=3, sinks=1), 20, 20, 2, 2, B=2, H=3)
    assert to_string(bm, limit=2).count("b=") == 2
    one = grid_classes(bm, 1, 1)
    assert one.shape == (2, 3, 1, 1) and (one == 1).all()          # empty and full tiles mixed
    full = build_block_mask(MaskMod("noop"), 16, 16, 4, 4)
    assert (grid_classes(full, 1, 1) == 2).all()
    empty_rows = build_block_mask(MaskMod("causal"), 8, 8, 4, 4)
    assert grid_classes(empty_rows, 2, 2)[0, 0, 0, 1] == 0


@pytest.mark.parametrize("mask,off", [(MaskMod("causal"), 37), (MaskMod("causal_window_sinks", window=50, sinks=3), 0),
                                      (MaskMod("program", clauses=((("causal", 0), ("kv_lt", 30)),)), 5)])
def test_row_slice_equals_rebuild_of_those_rows(mask, off):
    L, S, qb, kb = 300, 340, 32, 16
    bm = build_block_mask(mask, L, S, qb, kb, q_offset=off)
    for r0, r1 in ((0, 1), (3, 7), (9, 10)):
        sl = slice_block_mask(bm, rows=(r0, r1))
        sub_L = min(L - r0 * qb, (r1 - r0) * qb)
        ref = build_block_mask(mask, sub_L, S, qb, kb, q_offset=off + r0 * qb)
        for name in LISTS:
            assert np.array_equal(sl[name], ref[name]), (r0, r1, name)


def test_batch_and_head_slices_keep_dimensions():
    mask = MaskMod("program", clauses=((("causal", 0),), (("head_lt", 2), ("window", 8))))
    bm = build_block_mask(mask, 64, 64, 8, 8, B=2, H=4)
    sl = slice_block_mask(bm, batches=(1, 2), heads=(2, 3), rows=(1, 2))
    assert sl["kv_indices"].shape == (1, 1, 1, 8)
    assert np.array_equal(tile_classes(sl)[0, 0, 0], tile_classes(bm)[1, 2, 1])


@pytest.mark.parametrize("mask,off", [(MaskMod("causal"), 0), (MaskMod("causal_window_sinks", window=40, sinks=2), 0),
                                      (MaskMod("noop"), 0)])
def test_adjust_on_tile_boundaries_equals_rebuild(mask, off):
    bm = build_block_mask(mask, 256, 320, 32, 64, q_offset=off)
    for nl, ns in ((128, 192), (32, 64), (256, 320)):
        adj = adjust_block_mask(bm, nl, ns)
        ref = build_block_mask(mask, nl, ns, 32, 64, q_offset=off)
        for name in LISTS:
            assert np.array_equal(adj[name], ref[name]), (nl, ns, name)


def test_adjust_off_boundaries_is_conservative():
    rng = np.random.default_rng(4)
    doc = np.repeat(np.arange(6), [40, 70, 30, 90, 50, 40]).astype(np.int32)
    masks = [MaskMod("causal"), MaskMod("causal_window_sinks", window=45, sinks=3), MaskMod("doc_causal", doc_id=doc)]
    for mask in masks:
        bm = build_block_mask(mask, 300, 320, 32, 16)
        for _ in range(6):
            nl, ns = int(rng.integers(1, 301)), int(rng.integers(1, 321))
            adj, ref = tile_classes(adjust_block_mask(bm, nl, ns)), tile_classes(build_block_mask(mask, nl, ns, 32, 16))
            assert adj.shape == ref.shape
            # every tile with a visible cell is still computed, and no tile is
            # skipped its element mask unless every one of its cells is visible
            assert not ((ref != "0") & (adj == "0")).any()
            assert not ((adj == "F") & (ref != "F")).any()
            # the cropped edge row and column hold no full tile
            if nl % 32:
                assert not (adj[..., -1, :] == "F").any()
            if ns % 16:
                assert not (adj[..., :, -1] == "F").any()
            # and nothing beyond the crop changed class
            keep = tile_classes(bm)[:, :, :adj.shape[2], :adj.shape[3]]
            inner = keep[:, :, :adj.shape[2] - (1 if nl % 32 else 0), :adj.shape[3] - (1 if ns % 16 else 0)]
            assert np.array_equal(adj[:, :, :inner.shape[2], :inner.shape[3]], inner)


def test_dense_view_of_slice_and_adjust():
    bm = build_block_mask(MaskMod("causal"), 64, 64, 16, 16)
    assert to_dense(slice_block_mask(bm, rows=(2, 4)))[0, 0].tolist() == [[1, 1, 1, 0], [1, 1, 1, 1]]
    assert to_dense(adjust_block_mask(bm, 40, 20))[0, 0].tolist() == [[1, 0], [1, 1], [1, 1]]
