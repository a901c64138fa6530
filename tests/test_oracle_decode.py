"""Pins for the oracle's decode extensions: a cache whose capacity exceeds its
filled length, and per-batch offsets and lengths."""
import numpy as np

from golden.fixtures import load
from oracle import MaskMod, ScoreMod, attention, build_block_mask
from oracle.blockmask import tile_classes


def test_capacity_is_not_the_filled_length():
    # the decode section's example: capacity 8, positions 0..5 filled, query
    # at logical position 5 with a 3-key window -> keys 3, 4, 5
    fx = load("decode_offset_window.txt")
    cap, n = fx["capacity"], fx["valid_length"]
    q = np.zeros((1, 1, 1, 4))
    k = np.random.default_rng(0).standard_normal((1, 1, cap, 4))
    v = np.eye(cap).reshape(1, 1, cap, cap)
    mask = MaskMod("causal_window_sinks", window=fx["window"], sinks=0)
    out, _ = attention(q, k, v, scale=1.0, score=ScoreMod(), mask=mask, q_offset=fx["q_offset"], kv_len=n)
    seen = np.nonzero(out[0, 0, 0])[0].tolist()
    assert seen == fx["visible"]
    # checking only the capacity would let a no-op mask read the unfilled slots
    out, _ = attention(q, k, v, scale=1.0, score=ScoreMod(), mask=MaskMod("noop"), q_offset=fx["q_offset"],
                       kv_len=n)
    assert np.allclose(out[0, 0, 0], np.r_[np.full(n, 1.0 / n), np.zeros(cap - n)])


def test_per_batch_offsets_and_lengths_equal_separate_calls():
    rng = np.random.default_rng(1)
    B, H, L, S, D = 3, 2, 5, 40, 8
    q, k, v = (rng.standard_normal(s) for s in ((B, H, L, D), (B, H, S, D), (B, H, S, D)))
    offs, lens = [35, 0, 12], [40, 7, 17]
    mask, score = MaskMod("causal"), ScoreMod("softcap", cap=3.0)
    out, lse = attention(q, k, v, scale=0.4, score=score, mask=mask, q_offset=offs, kv_len=lens)
    for b in range(B):
        o1, l1 = attention(q[b:b + 1], k[b:b + 1, :, :lens[b]], v[b:b + 1, :, :lens[b]], scale=0.4, score=score,
                           mask=mask, q_offset=offs[b])
        assert np.allclose(out[b], o1[0], atol=1e-14) and np.allclose(lse[b], l1[0], atol=1e-14)


def test_block_mask_with_lengths_equals_shorter_build():
    offs, lens = [50, 3], [70, 21]
    bm = build_block_mask(MaskMod("causal_window_sinks", window=9, sinks=2), 30, 100, 8, 8, B=2, q_offset=offs,
                          kv_len=lens)
    cls = tile_classes(bm)
    for b in range(2):
        ref = tile_classes(build_block_mask(MaskMod("causal_window_sinks", window=9, sinks=2), 30, lens[b], 8, 8,
                                            q_offset=offs[b]))
        nk = ref.shape[3]
        assert np.array_equal(cls[b, :, :, :nk], ref[0])
        assert (cls[b, :, :, nk:] == "0").all()          # tiles past the filled length are empty
