"""Dense float64 definition of masked, score-modified attention.

Follows the charlestar blog "FlexAttention score_mod / BlockMask", section on
what one connection goes through: s_ij = scale * q_i . k_j; the score entering
the softmax is g(s_ij, b, h, i, j) where M_ij holds and -inf elsewhere; o_i is
the softmax-weighted sum of v_j over visible j.  The blog states this for rows
with at least one visible key; for a row with none (the quant67 causal-mask
article, section 7 on -inf numerics, shows the naive formula gives NaN) the
reading used here is out = 0 and lse = -inf.  lse is the natural log of the
softmax denominator (2kiu guide, section 2: auxiliary lse of shape (B, Hq, L));
the same section's other auxiliary output, max_scores, is read as the largest
score entering the softmax of each row (-inf for rows with no visible key).

Grouped-query attention (2kiu guide, section 6.1): query head hq reads K/V
head hq // (Hq / Hkv).  Query row i has logical position i + q_offset (blog,
decode section; quant67 article section 4 for the bottom-right alignment
q_offset = S - L).  The same decode section separates a cache's capacity from
its filled length: with ``kv_len`` a key at or past the valid length is not
visible whatever the mask says.  ``q_offset`` and ``kv_len`` may be given per
batch (a sequence indexed by b).

Nothing here is blocked or fused: each row chunk forms the full score row,
applies g, then the mask, then an ordinary softmax.  Chunking rows only bounds
memory; rows are independent.
"""
from __future__ import annotations

import numpy as np

from .mods import MaskMod, ScoreMod


def default_scale(D: int) -> float:
    """The default softmax scale 1/sqrt(D), D the head (embedding) dimension
    (2kiu guide, section 6.2: used when no scale is passed, applied to the
    scores before the softmax), as the float32 value a caller hands the
    kernel: 1/sqrt(D) evaluated in float64 and rounded once to float32."""
    return float(np.float32(1.0 / np.sqrt(np.float64(D))))


def _rows_softmax(z: np.ndarray, vis: np.ndarray, V: np.ndarray):
    """Row softmax of z (with -inf where not visible) applied to V; empty rows -> 0, -inf."""
    n_rows = z.shape[0]
    out = np.zeros((n_rows, V.shape[1]), dtype=np.float64)
    lse = np.full(n_rows, -np.inf, dtype=np.float64)
    live = vis.any(axis=1)
    if live.any():
        zl = z[live]
        m = zl.max(axis=1, keepdims=True)
        p = np.exp(zl - m)
        l = p.sum(axis=1, keepdims=True)
        out[live] = (p @ V) / l
        lse[live] = m[:, 0] + np.log(l[:, 0])
    return out, lse


def _at(value, b):
    """value[b] for a per-batch sequence, else value."""
    return value if value is None or np.isscalar(value) else value[b]


def attention_rows(q_rows, K, V, *, b: int, hq: int, Hq: int, row_ids, scale: float,
                   score: ScoreMod, mask: MaskMod, q_offset: int, with_max: bool = False, kv_len=None):
    """out (n, D) and lse (n,) for the given query rows of one (batch, query head),
    plus the row maxima of the masked scores when ``with_max``.

    q_rows: (n, D) query vectors of rows ``row_ids``; K, V: (S, D) of the matching
    K/V head.  ``scale`` is applied to q.k before g.
    """
    Q = np.asarray(q_rows, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    S = K.shape[0]
    s = (Q @ K.T) * np.float64(scale)
    q_pos = (np.asarray(row_ids, dtype=np.int64) + int(q_offset))[:, None]
    kv = np.arange(S, dtype=np.int64)[None, :]
    g = score(s, b, hq, q_pos, kv, Hq)
    vis = mask(b, hq, q_pos, kv)
    if kv_len is not None:
        vis = vis & (kv < int(kv_len))
    z = np.where(vis, g, -np.inf)
    out, lse = _rows_softmax(z, vis, V)
    if with_max:
        return out, lse, z.max(axis=1)
    return out, lse


def attention(q, k, v, *, scale: float, score: ScoreMod, mask: MaskMod, q_offset,
              rows=None, heads=None, batches=None, row_chunk: int = 512, with_max: bool = False, kv_len=None):
    """Dense oracle over (B, Hq, L, D) queries and (B, Hkv, S, D) keys/values.

    Returns ``out`` (nb, nh, nr, D) and ``lse`` (nb, nh, nr) in float64 for the selected
    batches / query heads / query rows (all of them by default), and the row
    maxima ``max_scores`` (nb, nh, nr) as a third value when ``with_max``.
    """
    B, Hq, L, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    batches = list(range(B)) if batches is None else list(batches)
    heads = list(range(Hq)) if heads is None else list(heads)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    Dv = v.shape[-1]
    out = np.zeros((len(batches), len(heads), len(rows), Dv), dtype=np.float64)
    lse = np.zeros((len(batches), len(heads), len(rows)), dtype=np.float64)
    mx = np.zeros((len(batches), len(heads), len(rows)), dtype=np.float64)
    for bi, b in enumerate(batches):
        for hi, hq in enumerate(heads):
            hkv = hq // group
            K = np.asarray(k[b, hkv], dtype=np.float64)
            V = np.asarray(v[b, hkv], dtype=np.float64)
            for c0 in range(0, len(rows), row_chunk):
                rid = rows[c0:c0 + row_chunk]
                o, ls, m = attention_rows(q[b, hq][rid], K, V, b=b, hq=hq, Hq=Hq, row_ids=rid,
                                          scale=scale, score=score, mask=mask, q_offset=_at(q_offset, b),
                                          with_max=True, kv_len=_at(kv_len, b))
                out[bi, hi, c0:c0 + len(rid)] = o
                lse[bi, hi, c0:c0 + len(rid)] = ls
                mx[bi, hi, c0:c0 + len(rid)] = m
    if with_max:
        return out, lse, mx
    return out, lse
