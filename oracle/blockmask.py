"""Block mask oracle: classify every Q_BLOCK x KV_BLOCK tile by counting cells.

Sources:
  * charlestar blog "FlexAttention score_mod / BlockMask", section on mask_mod
    and BlockMask: a tile with no visible cell is skipped, a tile whose cells are
    all visible runs without the element mask (score_mod still applies), any
    other tile runs with the element mask.
  * 2kiu "PyTorch Flex Attention complete guide", section 3.1: a block counts
    as sparse only when every element in it is; section 3.2: a row's dense form
    is rebuilt from the first num_blocks entries of its column-index list;
    section 4.1: create_block_mask pads lengths to a block multiple, aggregates
    per block and keeps full blocks in separate lists.
  * tensorcad "Attention expressions", What the engine does: the shading rule
    empty / full / in between.

Readings where the pages are silent: padding cells (beyond L or S) are not
visible, so an edge tile holding padding is never full; kv_num_blocks counts
partial tiles only and the full tiles sit in full_kv_*; each index row lists
its tiles in ascending order and is completed by the remaining tile indices,
ascending, so every row is a permutation of 0..nKB-1.
"""
from __future__ import annotations

import numpy as np

from .mods import MaskMod


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def visible_cells(mask: MaskMod, b: int, h: int, L: int, S: int, q_offset: int,
                  row0: int, nrows: int, col0: int, ncols: int) -> np.ndarray:
    """Boolean visibility of the cells [row0, row0+nrows) x [col0, col0+ncols).

    Cells outside [0, L) x [0, S) are not visible.
    """
    r = np.arange(row0, row0 + nrows, dtype=np.int64)
    c = np.arange(col0, col0 + ncols, dtype=np.int64)
    vis = mask(b, h, (r + q_offset)[:, None], c[None, :])
    vis &= (r < L)[:, None]
    vis &= (c < S)[None, :]
    return vis


def _ordered(flags: np.ndarray):
    """(count, indices): indices of set flags ascending, then the rest ascending."""
    idx = np.arange(flags.shape[0], dtype=np.int32)
    return int(flags.sum()), np.concatenate([idx[flags], idx[~flags]]).astype(np.int32)


def build_block_mask(mask: MaskMod, L: int, S: int, q_block: int, kv_block: int, *,
                     B: int = 1, H: int = 1, q_offset=0, kv_len=None) -> dict:
    """The four BlockMask arrays for a (B, H) grid of masks (1 = broadcast).

    ``q_offset`` and ``kv_len`` may be per-batch sequences (length B); keys at
    or past kv_len[b] are not visible (a cache of capacity S filled to
    kv_len[b], charlestar blog, decode section).

    Returns int32 arrays ``kv_num_blocks`` (B, H, nQB), ``kv_indices`` (B, H, nQB, nKB),
    ``full_kv_num_blocks``, ``full_kv_indices`` plus the per-tile cell counts.
    """
    nQB, nKB = _ceil_div(L, q_block), _ceil_div(S, kv_block)
    kv_num = np.zeros((B, H, nQB), dtype=np.int32)
    kv_idx = np.zeros((B, H, nQB, nKB), dtype=np.int32)
    fkv_num = np.zeros((B, H, nQB), dtype=np.int32)
    fkv_idx = np.zeros((B, H, nQB, nKB), dtype=np.int32)
    counts = np.zeros((B, H, nQB, nKB), dtype=np.int64)
    cells_per_tile = q_block * kv_block
    for b in range(B):
        for h in range(H):
            for qb in range(nQB):
                off = q_offset if np.isscalar(q_offset) else int(q_offset[b])
                S_b = S if kv_len is None else min(S, int(kv_len if np.isscalar(kv_len) else kv_len[b]))
                vis = visible_cells(mask, b, h, L, S_b, off, qb * q_block, q_block, 0, nKB * kv_block)
                cnt = vis.reshape(q_block, nKB, kv_block).sum(axis=(0, 2))
                counts[b, h, qb] = cnt
                full = cnt == cells_per_tile
                partial = (cnt > 0) & ~full
                kv_num[b, h, qb], kv_idx[b, h, qb] = _ordered(partial)
                fkv_num[b, h, qb], fkv_idx[b, h, qb] = _ordered(full)
    return {"kv_num_blocks": kv_num, "kv_indices": kv_idx,
            "full_kv_num_blocks": fkv_num, "full_kv_indices": fkv_idx,
            "counts": counts, "q_block": q_block, "kv_block": kv_block, "L": L, "S": S}


def to_dense(bm: dict) -> np.ndarray:
    """(B, H, nQB, nKB) 0/1 array: 1 where a tile is computed (partial or full).

    Rebuilds each row from the first num_blocks entries of its index list, as
    the 2kiu guide's section 3.2 describes, for both lists.
    """
    B, H, nQB, nKB = bm["kv_indices"].shape
    dense = np.zeros((B, H, nQB, nKB), dtype=np.int32)
    for num, ind in (("kv_num_blocks", "kv_indices"), ("full_kv_num_blocks", "full_kv_indices")):
        for b in range(B):
            for h in range(H):
                for r in range(nQB):
                    for t in range(bm[num][b, h, r]):
                        dense[b, h, r, bm[ind][b, h, r, t]] = 1
    return dense


def sparsity(bm: dict) -> float:
    """Percentage of tiles that are not computed (2kiu guide, section 3.3)."""
    d = to_dense(bm)
    return 100.0 * (1.0 - d.sum() / d.size)


def tile_classes(bm: dict) -> np.ndarray:
    """(B, H, nQB, nKB) array of 'F' / 'P' / '0' from the lists."""
    B, H, nQB, nKB = bm["kv_indices"].shape
    cls = np.full((B, H, nQB, nKB), "0", dtype="<U1")
    for num, ind, tag in (("kv_num_blocks", "kv_indices", "P"), ("full_kv_num_blocks", "full_kv_indices", "F")):
        for b in range(B):
            for h in range(H):
                for r in range(nQB):
                    for t in range(bm[num][b, h, r]):
                        cls[b, h, r, bm[ind][b, h, r, t]] = tag
    return cls


def transpose_block_mask(bm: dict) -> dict:
    """Q-side lists of a BlockMask: for every KV block, the Q blocks that list it.

    The 2kiu guide, section 3.3, says from_kv_blocks derives the Q-side block
    information from the KV-side lists by transposing them (for the backward
    pass).  Read here as: q_num_blocks[b, h, kb] counts the rows qb whose
    partial list holds kb, q_indices[b, h, kb] gives those qb ascending and then
    the remaining Q-block indices ascending; full_q_* do the same for the full
    lists.  Arrays are int32 of shapes (B, H, nKB) and (B, H, nKB, nQB).
    """
    B, H, nQB, nKB = bm["kv_indices"].shape
    out = {}
    for num, ind, tnum, tind in (("kv_num_blocks", "kv_indices", "q_num_blocks", "q_indices"),
                                 ("full_kv_num_blocks", "full_kv_indices", "full_q_num_blocks", "full_q_indices")):
        member = np.zeros((B, H, nKB, nQB), dtype=bool)
        for b in range(B):
            for h in range(H):
                for qb in range(nQB):
                    for t in range(bm[num][b, h, qb]):
                        member[b, h, bm[ind][b, h, qb, t], qb] = True
        cnt = np.zeros((B, H, nKB), dtype=np.int32)
        idx = np.zeros((B, H, nKB, nQB), dtype=np.int32)
        for b in range(B):
            for h in range(H):
                for kb in range(nKB):
                    cnt[b, h, kb], idx[b, h, kb] = _ordered(member[b, h, kb])
        out[tnum], out[tind] = cnt, idx
    return out


def slice_block_mask(bm: dict, batches=None, heads=None, rows=None) -> dict:
    """BlockMask restricted to batch range ``batches``, head range ``heads`` and
    Q-block rows ``rows`` (each a (start, stop) pair, default all).

    The 2kiu guide, section 3.3 (__getitem__): up to three indices select
    batch, head and Q-block row (a row of the tile grid, not a query token);
    integer indices become length-1 ranges so the dimensions stay.
    """
    B, H, nQB, nKB = bm["kv_indices"].shape
    b0, b1 = batches or (0, B)
    h0, h1 = heads or (0, H)
    r0, r1 = rows or (0, nQB)
    out = {name: np.array(bm[name][b0:b1, h0:h1, r0:r1], dtype=np.int32)
           for name in ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices")}
    out.update(q_block=bm["q_block"], kv_block=bm["kv_block"])
    return out


def adjust_block_mask(bm: dict, new_L: int, new_S: int) -> dict:
    """Crop a BlockMask to the top-left new lengths (2kiu guide, section 3.3, _adjust).

    Reading (the page gives the intent only, and warns it does not hold for
    every mask_mod): keep the first ceil(new_L / q_block) Q-block rows and,
    in each, the listed KV blocks below ceil(new_S / kv_block), in their
    order; a tile that now covers cells past new_L or new_S cannot be full
    (cells past the lengths are not visible), so such a full tile becomes
    partial.  Lists are then completed as the builder completes them.
    """
    qb, kb = bm["q_block"], bm["kv_block"]
    nq, nk = _ceil_div(new_L, qb), _ceil_div(new_S, kb)
    cls = tile_classes(bm)[:, :, :nq, :nk].copy()
    if new_L % qb:
        cls[:, :, nq - 1, :][cls[:, :, nq - 1, :] == "F"] = "P"
    if new_S % kb:
        cls[:, :, :, nk - 1][cls[:, :, :, nk - 1] == "F"] = "P"
    B, H = cls.shape[:2]
    out = {"kv_num_blocks": np.zeros((B, H, nq), np.int32), "kv_indices": np.zeros((B, H, nq, nk), np.int32),
           "full_kv_num_blocks": np.zeros((B, H, nq), np.int32),
           "full_kv_indices": np.zeros((B, H, nq, nk), np.int32), "q_block": qb, "kv_block": kb}
    for b in range(B):
        for h in range(H):
            for r in range(nq):
                out["kv_num_blocks"][b, h, r], out["kv_indices"][b, h, r] = _ordered(cls[b, h, r] == "P")
                out["full_kv_num_blocks"][b, h, r], out["full_kv_indices"][b, h, r] = _ordered(cls[b, h, r] == "F")
    return out


def grid_classes(bm: dict, grid_rows: int, grid_cols: int) -> np.ndarray:
    """Tile classes pooled into windows: 2 where every tile of the window is
    full, 0 where every tile is empty, 1 otherwise.

    Windows are ceil(nQB / grid_rows) x ceil(nKB / grid_cols) tiles (the last
    ones cut), so a grid no smaller than the tile grid is the tile grid
    itself.  This is the picture the 2kiu guide's to_string draws (section
    3.3: full, partial and empty blocks, grid_size bounding the picture); how
    it compresses a larger grid the page leaves open, and pooling by window is
    this oracle's reading.
    """
    cls = tile_classes(bm)
    B, H, nQB, nKB = cls.shape
    wr, wc = _ceil_div(nQB, grid_rows), _ceil_div(nKB, grid_cols)
    out = np.zeros((B, H, _ceil_div(nQB, wr), _ceil_div(nKB, wc)), dtype=np.int8)
    for i in range(out.shape[2]):
        for j in range(out.shape[3]):
            win = cls[:, :, i * wr:(i + 1) * wr, j * wc:(j + 1) * wc]
            all_full = (win == "F").all(axis=(2, 3))
            all_empty = (win == "0").all(axis=(2, 3))
            out[:, :, i, j] = np.where(all_full, 2, np.where(all_empty, 0, 1))
    return out


def to_string(bm: dict, grid_rows: int = 20, grid_cols: int = 20, limit: int = 4) -> str:
    """ASCII picture of the first ``limit`` (batch, head) grids: '█' full,
    '░' partial, ' ' empty (2kiu guide, section 3.3, to_string)."""
    g = grid_classes(bm, grid_rows, grid_cols)
    chars = {0: " ", 1: "░", 2: "█"}
    parts, shown = [], 0
    for b in range(g.shape[0]):
        for h in range(g.shape[1]):
            if shown == limit:
                break
            parts.append(f"b={b} h={h}")
            parts.extend("".join(chars[int(c)] for c in row) for row in g[b, h])
            shown += 1
    return "\n".join(parts)
