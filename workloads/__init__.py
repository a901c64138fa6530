"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle runs.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the HIP path and the CPU oracle are fed from here so
that they see exactly the same bytes.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per workload):
  1. for the packed-document workload only: document lengths, integers drawn
     uniformly from [256, 4096] one at a time until their sum reaches the total
     length; the last one is cut so the sum is exact;
  2. Q, then K, then V as float32 standard normals in C order, shapes
     (B, Hq, L, D), (B, Hkv, S, D), (B, Hkv, S, D);
  3. bfloat16 workloads round those float32 values to bfloat16 with
     round-to-nearest-even; the widened float32 copy is then exact.

The five workloads are the ones the block-sparse attention pages motivate:
plain causal (fp32), causal with soft-cap and an ALiBi-style bias, packed
documents, a sliding window with sink tokens under grouped-query attention,
and a 16-query verify step against a long KV cache with the causal mask
aligned to the bottom-right corner.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get_workload", "draw_doc_lengths", "doc_ids_from_lengths",
    "bf16_round", "bf16_bits_to_f32", "f32_to_bf16_bits", "make_inputs", "workload_doc_ids", "WORKLOAD_ORDER",
    "EXTRA_WORKLOADS", "make_upstream",
]


def f32_to_bf16_bits(x: np.ndarray, chunk: int = 1 << 24) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    Works in uint32 (no overflow for finite inputs: the largest finite pattern
    plus the rounding bias stays below 2^32) and in chunks to bound memory.
    Inputs here are finite by construction; NaN payloads are not handled.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1).view(np.uint32)
    out = np.empty(flat.shape, dtype=np.uint16)
    for i in range(0, flat.size, chunk):
        u = flat[i:i + chunk]
        r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        out[i:i + chunk] = (r >> np.uint32(16)).astype(np.uint16)
    return out.reshape(x.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exactly widened float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.uint32)
    np.left_shift(b, 16, out=out, dtype=np.uint32)
    return out.view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 and return them as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def draw_doc_lengths(rng: np.random.Generator, total: int, lo: int = 256, hi: int = 4096) -> list:
    """Document lengths uniform on [lo, hi], drawn until they cover ``total``; last one cut."""
    lengths, acc = [], 0
    while acc < total:
        n = int(rng.integers(lo, hi + 1))
        lengths.append(n)
        acc += n
    lengths[-1] -= acc - total
    return lengths


def doc_ids_from_lengths(lengths) -> np.ndarray:
    """Per-position document index (int32), documents laid end to end."""
    return np.repeat(np.arange(len(lengths), dtype=np.int32), np.asarray(lengths, dtype=np.int64))


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtype, mask and score rule, tile shape, seed."""
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    L: int
    S: int
    D: int
    dtype: str                  # "f32" or "bf16"
    mask: str                   # "noop" | "causal" | "causal_window_sinks" | "doc_causal" | "program"
    score: str                  # "none" | "softcap" | "softcap_alibi" | "alibi"
    q_block: int
    kv_block: int
    cap: float = 0.0
    alibi_m: float = 8.0
    window: int = 0
    sinks: int = 0
    docs: bool = False          # packed documents: draw lengths first
    clauses: tuple = ()         # "program" masks: AND of clauses, each an OR of (predicate, arg)

    @property
    def q_offset(self) -> int:
        # queries are the last L positions of the S-long sequence (bottom-right alignment)
        return self.S - self.L


WORKLOADS = {
    "causal_f32": Workload("causal_f32", 1, 1, 2, 2, 256, 256, 64, "f32", "causal", "none", 64, 64),
    "causal_softcap_alibi": Workload("causal_softcap_alibi", 2, 4, 16, 16, 2048, 2048, 64, "bf16",
                                     "causal", "softcap_alibi", 128, 64, cap=30.0, alibi_m=8.0),
    "doc_causal": Workload("doc_causal", 3, 1, 16, 16, 16384, 16384, 128, "bf16", "doc_causal", "none",
                           128, 64, docs=True),
    "window_sinks_gqa": Workload("window_sinks_gqa", 4, 2, 32, 8, 8192, 8192, 128, "bf16",
                                 "causal_window_sinks", "softcap", 128, 64, cap=50.0, window=1024, sinks=4),
    "decode_verify": Workload("decode_verify", 5, 16, 32, 8, 16, 32768, 128, "bf16", "causal", "softcap",
                              16, 64, cap=50.0),
    # mask programs from the tensorcad "Attention expressions" Examples table
    "prefix_lm_alibi": Workload("prefix_lm_alibi", 6, 4, 16, 16, 2048, 2048, 64, "bf16", "program", "alibi",
                                128, 64, clauses=((("causal", 0), ("kv_lt", 512)),)),
    "chunked_gqa": Workload("chunked_gqa", 7, 2, 32, 8, 8192, 8192, 128, "bf16", "program", "none", 128, 64,
                            clauses=((("causal", 0),), (("chunk", 2048),))),
}
WORKLOAD_ORDER = ["causal_f32", "causal_softcap_alibi", "doc_causal", "window_sinks_gqa", "decode_verify"]
# the same parity tests cover these; they are measured apart from the five above
EXTRA_WORKLOADS = ["prefix_lm_alibi", "chunked_gqa"]


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def workload_doc_ids(w: Workload):
    """The packed-document workload's doc_id array (same draw as make_inputs), or None."""
    if not w.docs:
        return None
    rng = np.random.Generator(np.random.PCG64(w.seed))
    return doc_ids_from_lengths(draw_doc_lengths(rng, w.S))


def make_inputs(w: Workload, *, B: Optional[int] = None, seed: Optional[int] = None) -> dict:
    """Draw the workload's inputs.

    Returns a dict with ``q``, ``k``, ``v`` as float32 arrays (for bf16 workloads these
    are the exactly widened bf16 values), ``q_bits``/``k_bits``/``v_bits`` as uint16 for
    bf16 workloads, ``doc_id`` (int32, or None) and ``doc_lengths``.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    B = w.B if B is None else B
    doc_lengths, doc_id = None, None
    if w.docs:
        doc_lengths = draw_doc_lengths(rng, w.S)
        doc_id = doc_ids_from_lengths(doc_lengths)
    out = {"doc_lengths": doc_lengths, "doc_id": doc_id}
    for name, shape in (("q", (B, w.Hq, w.L, w.D)), ("k", (B, w.Hkv, w.S, w.D)), ("v", (B, w.Hkv, w.S, w.D))):
        x = rng.standard_normal(shape, dtype=np.float32)
        if w.dtype == "bf16":
            bits = f32_to_bf16_bits(x)
            del x
            out[name + "_bits"] = bits
            out[name] = bf16_bits_to_f32(bits)
        else:
            out[name] = x
    return out


def make_upstream(w: Workload, *, B: Optional[int] = None, seed: Optional[int] = None) -> dict:
    """The gradient flowing into the attention output, for backward runs.

    Standard normals of shape (B, Hq, L, D) from their own generator
    (``PCG64(seed + 1_000_003)``) so the forward inputs stay as ``make_inputs``
    draws them; bf16 workloads round them as in step 3 of the recipe.  Returns
    ``dout`` (float32, exact widened values) and ``dout_bits`` for bf16.
    """
    rng = np.random.Generator(np.random.PCG64((w.seed if seed is None else seed) + 1_000_003))
    B = w.B if B is None else B
    x = rng.standard_normal((B, w.Hq, w.L, w.D), dtype=np.float32)
    if w.dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        return {"dout_bits": bits, "dout": bf16_bits_to_f32(bits)}
    return {"dout": x}
