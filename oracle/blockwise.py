"""Second float64 oracle: walk only the block lists with an online softmax.

This is the tiled execution the pages describe, done slowly and in float64:
the charlestar blog "FlexAttention score_mod / BlockMask" (sections on
BlockMask and on the attention template) says empty tiles are skipped, full
tiles are computed without the element mask but still with score_mod, partial
tiles are computed and then masked, and the template keeps a running softmax
instead of a score matrix.  The quant67 causal-mask article (section 7,
FlashAttention block skipping) describes the same running statistics.

It exists to show that the block mask loses nothing: on any input its result
must equal the dense definition in ``attention`` up to float64 rounding.
It does not share the dense oracle's softmax code.
"""
from __future__ import annotations

import numpy as np

from .mods import MaskMod, ScoreMod


def blockwise_attention(q, k, v, bm: dict, *, scale: float, score: ScoreMod, mask: MaskMod,
                        q_offset: int):
    """out (B, Hq, L, Dv) and lse (B, Hq, L), float64, visiting only listed tiles."""
    B, Hq, L, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    group = Hq // Hkv
    QB, KB = bm["q_block"], bm["kv_block"]
    Bm, Hm, nQB, _ = bm["kv_indices"].shape
    out = np.zeros((B, Hq, L, v.shape[-1]), dtype=np.float64)
    lse = np.full((B, Hq, L), -np.inf, dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            bi, hi = (b if Bm > 1 else 0), (hq if Hm > 1 else 0)
            Qh = np.asarray(q[b, hq], dtype=np.float64)
            Kh = np.asarray(k[b, hq // group], dtype=np.float64)
            Vh = np.asarray(v[b, hq // group], dtype=np.float64)
            for qb in range(nQB):
                rows = np.arange(qb * QB, min((qb + 1) * QB, L), dtype=np.int64)
                qpos = rows + q_offset
                run_max = np.full(rows.size, -np.inf)
                denom = np.zeros(rows.size)
                acc = np.zeros((rows.size, Vh.shape[1]))
                work = [(int(t), False) for t in bm["full_kv_indices"][bi, hi, qb, :bm["full_kv_num_blocks"][bi, hi, qb]]]
                work += [(int(t), True) for t in bm["kv_indices"][bi, hi, qb, :bm["kv_num_blocks"][bi, hi, qb]]]
                for kb, needs_mask in work:
                    cols = np.arange(kb * KB, min((kb + 1) * KB, S), dtype=np.int64)
                    s = (Qh[rows] @ Kh[cols].T) * np.float64(scale)
                    t = score(s, b, hq, qpos[:, None], cols[None, :], Hq)
                    if needs_mask:
                        t = np.where(mask(b, hq, qpos[:, None], cols[None, :]), t, -np.inf)
                    new_max = np.maximum(run_max, t.max(axis=1))
                    ref = np.where(np.isfinite(new_max), new_max, 0.0)
                    decay = np.exp(run_max - ref)
                    w = np.exp(t - ref[:, None])
                    denom = denom * decay + w.sum(axis=1)
                    acc = acc * decay[:, None] + w @ Vh[cols]
                    run_max = new_max
                seen = denom > 0
                out[b, hq, rows[seen]] = acc[seen] / denom[seen, None]
                lse[b, hq, rows[seen]] = run_max[seen] + np.log(denom[seen])
    return out, lse
