"""The forward entry point that allocates nothing (flex_attn_fwd_noalloc):
its output equals flex_attn_fwd's on the same inputs, bit for bit, on two
calls in a row, the second with a smaller input, on the split-KV decode path
(which keeps its partials in the library's scratch array) and on the prefill
path (which needs none).  Also checked against the CPU oracle."""
import numpy as np
import pytest
import torch

import programmable_block_sparse_amd as pbs
from gpu_common import assert_attention_close, require_gpu
from oracle import MaskMod, ScoreMod, attention
from oracle import default_scale as oracle_default_scale
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _inputs(rng, B, Hq, Hkv, L, S, D, dev):
    bits = [f32_to_bf16_bits(rng.standard_normal(s, dtype=np.float32))
            for s in ((B, Hq, L, D), (B, Hkv, S, D), (B, Hkv, S, D))]
    ts = [torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16) for b in bits]
    return ts, [bf16_bits_to_f32(b) for b in bits]


def _case(dev, rng, B, Hq, Hkv, L, S, D, qb, expect_scratch):
    (q, k, v), (qf, kf, vf) = _inputs(rng, B, Hq, Hkv, L, S, D, dev)
    mspec = pbs.MaskSpec(kind="causal")                  # bottom-right: q_offset = S - L
    sspec = pbs.ScoreSpec(kind="softcap", cap=50.0)
    bm = pbs.flex_blockmask_build(mspec, L, S, qb, 64, device=dev)
    need = pbs.flex_attn_fwd_workspace_bytes(torch.bfloat16, B, Hq, Hkv, L, S, D, bm)
    assert (need > 0) == expect_scratch, need
    out_ref, lse_ref = pbs.flex_attn_fwd(q, k, v, block_mask=bm, score=sspec, mask=mspec)
    out = torch.full_like(out_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    pbs.flex_attn_fwd_noalloc(q, k, v, block_mask=bm, out=out, lse=lse, score=sspec, mask=mspec)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref), "noalloc out differs from flex_attn_fwd"
    assert torch.equal(lse, lse_ref), "noalloc lse differs from flex_attn_fwd"
    o_or, l_or = attention(qf, kf, vf, scale=oracle_default_scale(D), score=ScoreMod("softcap", cap=50.0),
                           mask=MaskMod("causal"), q_offset=S - L)
    assert_attention_close(out, lse, o_or, l_or, "bf16", f"noalloc B={B} Hq={Hq} L={L} S={S} D={D}")
    return need


def test_noalloc_matches_fwd_decode_then_smaller(dev=None):
    dev = require_gpu()
    rng = np.random.default_rng(4242)
    need1 = _case(dev, rng, B=4, Hq=32, Hkv=8, L=16, S=8192, D=128, qb=16, expect_scratch=True)
    need2 = _case(dev, rng, B=2, Hq=8, Hkv=2, L=16, S=3000, D=128, qb=16, expect_scratch=True)
    assert 0 < need2 < need1 <= 32 << 20


def test_noalloc_matches_fwd_prefill_then_smaller(dev=None):
    dev = require_gpu()
    rng = np.random.default_rng(4343)
    _case(dev, rng, B=2, Hq=8, Hkv=2, L=700, S=700, D=64, qb=128, expect_scratch=False)
    _case(dev, rng, B=1, Hq=4, Hkv=1, L=200, S=260, D=64, qb=128, expect_scratch=False)
