"""Dense float64 gradients of masked, score-modified attention (test oracle).

The forward is the definition the ``attention`` oracle follows: s = scale *
q.k, z = g(s) where the mask holds and -inf elsewhere, P = row softmax of z,
O = P V.  The pages say only that gradients flow through that same
definition: the charlestar blog "FlexAttention score_mod / BlockMask" runs its
windowed, soft-capped example and then calls backward on the summed output;
the 2kiu "PyTorch Flex Attention complete guide" (section 3.3) derives a
Q-side copy of the block lists for that pass, and its section 5.2 gives the
backward its own tile sizes.  The formulas below are the chain rule through
that definition, not anything printed on the pages:

  dV_j  = sum_i P_ij dO_i
  dP_ij = dO_i . V_j
  D_i   = sum_j P_ij dP_ij            (= dO_i . O_i)
  dZ_ij = P_ij (dP_ij - D_i)
  dS_ij = dZ_ij * g'(s_ij) * scale    (g' = 1 - tanh(s/c)^2 under a soft-cap,
                                       1 otherwise; the distance bias does not
                                       depend on s)
  dQ_i  = sum_j dS_ij K_j,   dK_j = sum_i dS_ij Q_i

Under GQA the K/V gradients of a K/V head sum over its query heads.  Rows
with no visible key have P = 0 and contribute nothing.  Nothing is blocked:
each (batch, head) forms the full score matrix.

As in the forward oracle, ``q_offset`` and the filled key length ``kv_len``
(the blog's decode section: keys at or past a cache's valid length are not
visible whatever the mask says) may be given per batch; a key that is not
visible to any row gets zero dK and dV.
"""
from __future__ import annotations

import numpy as np

from .attention import _at
from .mods import ScoreMod, MaskMod, SOFTCAP, SOFTCAP_ALIBI


def score_derivative(score: ScoreMod, s):
    """dg/ds for the menu (the bias term of the ALiBi kinds does not depend on s)."""
    s = np.asarray(s, dtype=np.float64)
    if score.kind in (SOFTCAP, SOFTCAP_ALIBI):
        t = np.tanh(s / float(score.cap))
        return 1.0 - t * t
    return np.ones_like(s)


def attention_backward(q, k, v, dout, *, scale: float, score: ScoreMod, mask: MaskMod, q_offset, pairs=None,
                       row_chunk: int = 0, kv_len=None):
    """(dq, dk, dv) in float64 for (B, Hq, L, D) queries and (B, Hkv, S, D) keys/values.

    ``q_offset``: logical position of query row 0, an int or one per batch.
    ``kv_len``: None (all S keys), or the valid key count, an int or one per batch.
    ``pairs``: optional list of (batch, query head) to include; the gradients
    then hold only those heads' terms (the others stay zero).  Default: all.
    ``row_chunk``: process that many query rows at a time (0: all); rows are
    independent, so this only bounds memory, and dk, dv add the chunks' terms.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, Hq, L, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    group = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    kv = np.arange(S, dtype=np.int64)[None, :]
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(Hq)]
    step = row_chunk or L
    for b, h in pairs:
        hk = h // group
        K, V = k[b, hk], v[b, hk]
        q_pos = (np.arange(L, dtype=np.int64) + int(_at(q_offset, b)))[:, None]
        kl = _at(kv_len, b)
        for r0 in range(0, L, step):
            rows = slice(r0, min(L, r0 + step))
            qp = q_pos[rows]
            s = (q[b, h, rows] @ K.T) * float(scale)
            vis = mask(b, h, qp, kv)
            if kl is not None:
                vis = vis & (kv < int(kl))
            z = np.where(vis, score(s, b, h, qp, kv, Hq), -np.inf)
            live = vis.any(axis=1)
            P = np.zeros_like(z)
            if live.any():
                zl = z[live]
                e = np.exp(zl - zl.max(axis=1, keepdims=True))
                P[live] = e / e.sum(axis=1, keepdims=True)
            O = P @ V
            dO = dout[b, h, rows]
            dP = dO @ V.T
            Dr = (dO * O).sum(axis=1, keepdims=True)
            dZ = P * (dP - Dr)
            dS = dZ * score_derivative(score, s) * float(scale)
            dq[b, h, rows] = dS @ K
            dk[b, hk] += dS.T @ q[b, h, rows]
            dv[b, hk] += P.T @ dO
    return dq, dk, dv
