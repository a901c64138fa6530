"""The seeded input generators shared by the tests, the benchmark and the
oracle runs: bfloat16 rounding bit-checks, determinism of the draws, and the
workload table.  CPU only."""
import numpy as np
import pytest
import torch

from oracle import MaskMod, build_block_mask
from workloads import (WORKLOADS, bf16_bits_to_f32, draw_doc_lengths, f32_to_bf16_bits, make_inputs, make_upstream,
                       workload_doc_ids)


def _bits(u32):
    return np.asarray(u32, dtype=np.uint32).view(np.float32)


def test_bf16_round_to_nearest_even_ties():
    cases = {
        0x3F800000: 0x3F80,   # 1.0 exactly
        0x3F808000: 0x3F80,   # halfway between 0x3F80 and 0x3F81: to the even one
        0x3F818000: 0x3F82,   # halfway between 0x3F81 and 0x3F82: to the even one
        0x3F808001: 0x3F81,   # just above halfway: up
        0x3F807FFF: 0x3F80,   # just below halfway: down
        0xBF808000: 0xBF80,   # the same ties for negative values
        0xBF818000: 0xBF82,
        0x00000000: 0x0000,
        0x80000000: 0x8000,   # -0 keeps its sign
        0x00008000: 0x0000,   # subnormal tie to even (zero)
        0x00018000: 0x0002,   # subnormal tie to even (up)
        0x7F7FFFFF: 0x7F80,   # the largest float rounds up to +inf, as round-to-nearest requires
        0x7F7F7FFF: 0x7F7F,   # the largest float below the bf16 rounding boundary stays finite
    }
    got = f32_to_bf16_bits(_bits(list(cases)))
    assert got.tolist() == list(cases.values())


def test_bf16_matches_torch_conversion():
    rng = np.random.default_rng(0)
    # every exponent of a finite float, random mantissas and signs
    u = (rng.integers(0, 2, 1 << 20, dtype=np.uint32) << 31) | \
        (rng.integers(0, 255, 1 << 20, dtype=np.uint32) << 23) | rng.integers(0, 1 << 23, 1 << 20, dtype=np.uint32)
    x = u.view(np.float32)
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # widening is exact: bits -> float32 -> bits round trip
    assert np.array_equal(f32_to_bf16_bits(bf16_bits_to_f32(ours)), ours)


def test_draws_are_deterministic_and_seeded():
    w = WORKLOADS["causal_softcap_alibi"]
    a = make_inputs(w, B=1)
    b = make_inputs(w, B=1)
    for name in ("q", "k", "v", "q_bits", "k_bits", "v_bits"):
        assert np.array_equal(a[name], b[name]), name
    c = make_inputs(w, B=1, seed=w.seed + 1)
    assert not np.array_equal(a["q_bits"], c["q_bits"])
    # Q, K and V come from one generator in that order: Q is its first draw
    rng = np.random.Generator(np.random.PCG64(w.seed))
    q = rng.standard_normal((1, w.Hq, w.L, w.D), dtype=np.float32)
    assert np.array_equal(a["q_bits"], f32_to_bf16_bits(q))
    # the widened float32 copy is exactly the bf16 value
    assert np.array_equal(f32_to_bf16_bits(a["k"]), a["k_bits"])
    # the upstream gradient has its own generator: the forward inputs do not move
    up = make_upstream(w, B=1)
    assert up["dout"].shape == (1, w.Hq, w.L, w.D)
    assert np.array_equal(make_inputs(w, B=1)["q"], a["q"])


def test_packed_document_draw():
    w = WORKLOADS["doc_causal"]
    rng = np.random.Generator(np.random.PCG64(w.seed))
    lengths = draw_doc_lengths(rng, w.S)
    # the draw the packed-document configuration is described with (seed 3)
    assert lengths == [3372, 584, 945, 1165, 952, 3333, 3594, 2439]
    doc = workload_doc_ids(w)
    assert doc.shape == (w.S,) and doc.dtype == np.int32
    assert np.array_equal(np.bincount(doc), lengths)
    assert np.all(np.diff(doc) >= 0)
    # every length but the cut last one is inside [256, 4096]
    assert all(256 <= n <= 4096 for n in lengths[:-1]) and 0 < lengths[-1] <= 4096


@pytest.mark.parametrize("name,shape,dtype", [
    ("causal_f32", (1, 2, 2, 256, 256, 64), "f32"),
    ("causal_softcap_alibi", (4, 16, 16, 2048, 2048, 64), "bf16"),
    ("doc_causal", (1, 16, 16, 16384, 16384, 128), "bf16"),
    ("window_sinks_gqa", (2, 32, 8, 8192, 8192, 128), "bf16"),
    ("decode_verify", (16, 32, 8, 16, 32768, 128), "bf16"),
])
def test_workload_table(name, shape, dtype):
    w = WORKLOADS[name]
    assert (w.B, w.Hq, w.Hkv, w.L, w.S, w.D) == shape
    assert w.dtype == dtype
    assert w.q_offset == w.S - w.L


def test_tile_classes_of_the_small_and_decode_workloads():
    # F / P / E tile counts of the configuration table, from the oracle's builder
    w = WORKLOADS["causal_f32"]
    bm = build_block_mask(MaskMod("causal"), w.L, w.S, w.q_block, w.kv_block, q_offset=w.q_offset)
    full, part = int(bm["full_kv_num_blocks"].sum()), int(bm["kv_num_blocks"].sum())
    assert (full, part, 16 - full - part) == (6, 4, 6)
    w = WORKLOADS["decode_verify"]
    bm = build_block_mask(MaskMod("causal"), w.L, w.S, w.q_block, w.kv_block, q_offset=w.q_offset)
    full, part = int(bm["full_kv_num_blocks"].sum()), int(bm["kv_num_blocks"].sum())
    assert (full, part) == (511, 1)
