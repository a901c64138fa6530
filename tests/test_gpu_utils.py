"""GPU parity of the BlockMask utilities (to_dense, the pooled grid and its
picture, sparsity, slicing, cropping) against the oracle, bit for bit."""
import numpy as np
import pytest
import torch

import programmable_block_sparse_amd as pbs
from gpu_common import require_gpu
from oracle import (MaskMod, adjust_block_mask, build_block_mask, grid_classes, slice_block_mask, sparsity, to_dense,
                    to_string)

pytestmark = pytest.mark.gpu

LISTS = ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices")


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _masks(dev, rng):
    doc = np.repeat(np.arange(7), [5, 40, 3, 70, 1, 60, 121]).astype(np.int32)
    doc_t = torch.from_numpy(doc).to(dev)
    return [
        (pbs.MaskSpec("causal", q_offset=0), MaskMod("causal"), 0),
        (pbs.MaskSpec("causal_window_sinks", window=40, sinks=3, q_offset=20), MaskMod("causal_window_sinks", window=40, sinks=3), 20),
        (pbs.MaskSpec("doc_causal", q_offset=0, doc_id=doc_t), MaskMod("doc_causal", doc_id=doc), 0),
        (pbs.MaskSpec("program", q_offset=5, clauses=((("causal", 0),), (("head_lt", 1), ("chunk", 24)))),
         MaskMod("program", clauses=((("causal", 0),), (("head_lt", 1), ("chunk", 24)))), 5),
    ]


def _cases(dev):
    rng = np.random.default_rng(8)
    for i, (spec, mod, off) in enumerate(_masks(dev, rng)):
        for L, S, qb, kb in ((300, 300, 32, 16), (250, 280, 64, 32), (97, 130, 16, 8)):
            B, H = (2, 3) if i % 2 else (1, 1)
            gpu = pbs.flex_blockmask_build(spec, L, S, qb, kb, B=B, H=H, device=dev)
            ref = build_block_mask(mod, L, S, qb, kb, B=B, H=H, q_offset=off)
            yield f"mask{i} {L}x{S} {qb}x{kb}", gpu, ref, L, S


def test_to_dense_grid_sparsity(dev):
    for what, gpu, ref, L, S in _cases(dev):
        assert np.array_equal(gpu.to_dense().cpu().numpy(), to_dense(ref)), what
        for gr, gc in ((1, 1), (3, 5), (7, 20), (1000, 1000)):
            assert np.array_equal(gpu.grid(gr, gc).cpu().numpy(), grid_classes(ref, gr, gc)), (what, gr, gc)
        assert gpu.to_string() == to_string(ref)
        assert gpu.sparsity() == pytest.approx(sparsity(ref), abs=1e-12), what


def test_slices(dev):
    rng = np.random.default_rng(9)
    for what, gpu, ref, L, S in _cases(dev):
        B, H, nqb, _ = ref["kv_indices"].shape
        for _ in range(4):
            b0 = int(rng.integers(0, B)); b1 = int(rng.integers(b0 + 1, B + 1))
            h0 = int(rng.integers(0, H)); h1 = int(rng.integers(h0 + 1, H + 1))
            r0 = int(rng.integers(0, nqb)); r1 = int(rng.integers(r0 + 1, nqb + 1))
            got = gpu[b0:b1, h0:h1, r0:r1]
            want = slice_block_mask(ref, (b0, b1), (h0, h1), (r0, r1))
            for name in LISTS:
                assert np.array_equal(getattr(got, name).cpu().numpy(), want[name]), (what, name)
        one = gpu[0, 0, nqb - 1]
        assert one.kv_indices.shape[:3] == (1, 1, 1)


def test_adjust(dev):
    rng = np.random.default_rng(10)
    for what, gpu, ref, L, S in _cases(dev):
        for _ in range(4):
            nl, ns = int(rng.integers(1, L + 1)), int(rng.integers(1, S + 1))
            got = gpu.adjust(nl, ns)
            want = adjust_block_mask(ref, nl, ns)
            for name in LISTS:
                assert np.array_equal(getattr(got, name).cpu().numpy(), want[name]), (what, nl, ns, name)


def test_adjusted_mask_runs_attention(dev):
    """A cropped causal mask drives the forward over the cropped lengths."""
    L = S = 512
    spec = pbs.MaskSpec("causal", q_offset=0)
    bm = pbs.flex_blockmask_build(spec, L, S, 128, 64, device=dev)
    small = bm.adjust(300, 300)
    rebuilt = pbs.flex_blockmask_build(spec, 300, 300, 128, 64, device=dev)
    g = torch.Generator().manual_seed(3)
    q, k, v = (torch.randn(1, 2, 300, 64, generator=g).to(dev).to(torch.bfloat16) for _ in range(3))
    out_a, lse_a = pbs.flex_attn_fwd(q, k, v, block_mask=small, mask=spec)
    out_b, lse_b = pbs.flex_attn_fwd(q, k, v, block_mask=rebuilt, mask=spec)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)
