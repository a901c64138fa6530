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
                     B: int = 1, H: int = 1, q_offset: int = 0) -> dict:
    """The four BlockMask arrays for a (B, H) grid of masks (1 = broadcast).

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
                vis = visible_cells(mask, b, h, L, S, q_offset, qb * q_block, q_block, 0, nKB * kv_block)
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
