"""score_mod and mask_mod menu of the oracle (float64 / int64 NumPy).

Sources (web pages on FlexAttention):
  * charlestar blog "FlexAttention score_mod / BlockMask", section on what one
    connection goes through: the score fed to score_mod is the already scaled
    q.k, the rule g(s, b, h, i, j) is applied to visible connections and the
    others become -inf.
  * same blog, section on score_mod ordering: the teaching rule
    g = c*tanh(s/c) + alpha_h*(p_j - p_i) caps first and adds the bias after.
  * same blog, section on the pinned-version example: a causal window of W
    keys includes the query itself (0 <= p_i - p_j < W).
  * same blog, section on packing: document masks require equal segment ids.
  * same blog, section on decode: the mods see the logical position
    q_idx + q_offset.
  * tensorcad "Attention expressions", Examples: sink window
    "q - kv < W or kv < 4" under causal, ALiBi slope 2**(-8*(h+1)/heads),
    Gemma-2 cap 50*tanh(score/50).
  * 2kiu "PyTorch Flex Attention complete guide" section 1.2: h is the query
    head; section 4.1: mask_mod returns True for connections that attend;
    section 4.3: and_masks is the AND of its masks folded from all-true,
    or_masks the OR folded from all-false.
  * tensorcad "Attention expressions", Examples: prefix-LM "kv <= q or
    kv < 16", chunked "floor(q / C) == floor(kv / C)", every fourth key
    "(q - kv) % 4 == 0" (the page's operators follow Python, so % and //
    floor), half the heads global "h < heads / 2 or q - kv < W", and the
    uncapped ALiBi row "score - 2 ** (-8 * (h + 1) / heads) * (q - kv)".
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

NONE, SOFTCAP, SOFTCAP_ALIBI, ALIBI = "none", "softcap", "softcap_alibi", "alibi"
NOOP, CAUSAL, CAUSAL_WINDOW_SINKS, DOC_CAUSAL = "noop", "causal", "causal_window_sinks", "doc_causal"
PROGRAM = "program"
PREDICATES = ("causal", "window", "kv_lt", "chunk", "stride", "doc", "head_lt")


def alibi_slope(h, heads: int, m: float = 8.0):
    """Per-query-head bias slope 2^(-m (h+1) / heads) (tensorcad Examples, ALiBi row)."""
    return np.power(2.0, -float(m) * (np.asarray(h, dtype=np.float64) + 1.0) / float(heads))


@dataclasses.dataclass(frozen=True)
class ScoreMod:
    """g(score, b, h, q_pos, kv): applied to the scaled score of every visible cell."""
    kind: str = NONE
    cap: float = 0.0
    alibi_m: float = 8.0

    def __call__(self, s, b, h, q_pos, kv, heads: int):
        s = np.asarray(s, dtype=np.float64)
        if self.kind == NONE:
            return s
        if self.kind == ALIBI:
            dist = np.asarray(kv, dtype=np.float64) - np.asarray(q_pos, dtype=np.float64)
            return s + alibi_slope(h, heads, self.alibi_m) * dist
        c = float(self.cap)
        capped = c * np.tanh(s / c)
        if self.kind == SOFTCAP:
            return capped
        if self.kind == SOFTCAP_ALIBI:
            dist = np.asarray(kv, dtype=np.float64) - np.asarray(q_pos, dtype=np.float64)
            return capped + alibi_slope(h, heads, self.alibi_m) * dist
        raise ValueError(f"unknown score kind {self.kind!r}")


@dataclasses.dataclass(frozen=True)
class MaskMod:
    """M(b, h, q_pos, kv) -> bool, True meaning the connection attends.

    kind "program": ``clauses`` is a tuple of clauses, each a tuple of
    (predicate, argument) pairs; the mask is the AND of the clauses and a
    clause the OR of its predicates (and_masks of or_masks)."""
    kind: str = NOOP
    window: int = 0
    sinks: int = 0
    doc_id: Optional[np.ndarray] = None
    clauses: tuple = ()

    def _doc_equal(self, q_pos, kv):
        doc = np.asarray(self.doc_id)
        n = doc.shape[0]
        # positions outside the id array belong to no document
        q_in = (q_pos >= 0) & (q_pos < n)
        kv_in = (kv >= 0) & (kv < n)
        dq = doc[np.clip(q_pos, 0, n - 1)]
        dk = doc[np.clip(kv, 0, n - 1)]
        return q_in & kv_in & (dq == dk)

    def _predicate(self, name, arg, h, q_pos, kv):
        if name == "causal":
            return kv <= q_pos
        if name == "window":
            return (q_pos - kv) < arg
        if name == "kv_lt":
            return kv < arg
        if name == "chunk":
            return np.floor_divide(q_pos, arg) == np.floor_divide(kv, arg)
        if name == "stride":
            return np.mod(q_pos - kv, arg) == 0
        if name == "doc":
            return self._doc_equal(q_pos, kv)
        if name == "head_lt":
            return np.asarray(h) < arg
        raise ValueError(f"unknown predicate {name!r}")

    def __call__(self, b, h, q_pos, kv):
        q_pos = np.asarray(q_pos, dtype=np.int64)
        kv = np.asarray(kv, dtype=np.int64)
        shape = np.broadcast_shapes(q_pos.shape, kv.shape)
        if self.kind == NOOP:
            return np.ones(shape, dtype=bool)
        causal = kv <= q_pos
        if self.kind == CAUSAL:
            return np.broadcast_to(causal, shape).copy()
        if self.kind == CAUSAL_WINDOW_SINKS:
            near = (q_pos - kv) < self.window
            sink = kv < self.sinks
            return np.broadcast_to(causal & (near | sink), shape).copy()
        if self.kind == DOC_CAUSAL:
            return np.broadcast_to(causal & self._doc_equal(q_pos, kv), shape).copy()
        if self.kind == PROGRAM:
            out = np.ones(shape, dtype=bool)                 # and_masks folds from true
            for clause in self.clauses:
                any_ = np.zeros(shape, dtype=bool)           # or_masks folds from false
                for name, arg in clause:
                    any_ = any_ | np.broadcast_to(self._predicate(name, int(arg), h, q_pos, kv), shape)
                out = out & any_
            return out
        raise ValueError(f"unknown mask kind {self.kind!r}")
