"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

BlockMask arrays must match bit for bit; out within 2e-2 (bf16 inputs) or
1e-5 (fp32) max-abs; lse within 1e-3 and -inf exactly where the oracle has it.
Small cases compare every output; the five full-size workloads compare sampled
rows (edges of every Q block plus random rows) that the oracle computes one by
one.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import programmable_block_sparse_amd as pbs
from gpu_common import TOL_LSE, assert_attention_close, assert_block_mask_equal, oracle_mods, require_gpu
from oracle import MaskMod, ScoreMod, attention, build_block_mask
from oracle import default_scale as oracle_default_scale
from workloads import (EXTRA_WORKLOADS, WORKLOAD_ORDER, WORKLOADS, Workload, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs,
                       workload_doc_ids)
from workloads.torch_io import specs, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _mask_pair(kind, window=0, sinks=0, q_offset=0, doc_np=None, doc_t=None, clauses=()):
    clauses = tuple(tuple(c) for c in clauses)
    return (pbs.MaskSpec(kind=kind, window=window, sinks=sinks, q_offset=q_offset, doc_id=doc_t, clauses=clauses),
            MaskMod(kind, window=window, sinks=sinks, doc_id=doc_np, clauses=clauses))


def _uses_doc(kind, clauses):
    return kind == "doc_causal" or any(name == "doc" for c in clauses for name, _ in c)


def _rand_doc(rng, n):
    cuts = np.sort(rng.choice(np.arange(1, n), size=min(n - 1, int(rng.integers(0, 5))), replace=False)) if n > 1 else []
    lens = np.diff(np.concatenate([[0], cuts, [n]])).astype(np.int64)
    return np.repeat(np.arange(len(lens), dtype=np.int32), lens)


# ------------------------------------------------------------ BlockMask builder
def test_blockmask_fuzz_bit_exact(dev):
    rng = np.random.default_rng(1234)
    kinds = ["noop", "causal", "causal_window_sinks", "doc_causal"]
    n_cases = 0
    for trial in range(160):
        L, S = int(rng.integers(1, 300)), int(rng.integers(1, 300))
        QB = int(rng.choice([1, 2, 3, 4, 7, 16, 32, 64, 128]))
        KB = int(rng.choice([1, 2, 5, 16, 64, 128]))
        kind = kinds[trial % 4]
        offs = [S - L, 0, int(rng.integers(-40, 40))]
        for off in offs:
            doc_np = doc_t = None
            if kind == "doc_causal":
                if off < 0:
                    continue
                doc_np = _rand_doc(rng, max(S, off + L) + int(rng.integers(0, 3)))
                doc_t = torch.from_numpy(doc_np).to(dev)
            window, sinks = int(rng.integers(1, 40)), int(rng.integers(0, 6))
            spec, mod = _mask_pair(kind, window, sinks, off, doc_np, doc_t)
            Bm, Hm = (1, 1) if trial % 3 else (2, 3)
            gpu = pbs.flex_blockmask_build(spec, L, S, QB, KB, B=Bm, H=Hm, device=dev)
            ref = build_block_mask(mod, L, S, QB, KB, B=Bm, H=Hm, q_offset=off)
            assert_block_mask_equal(gpu, ref)
            n_cases += 1
    assert n_cases > 300


def test_blockmask_extreme_parameters(dev):
    """Windows up to INT32_MAX, sinks past S, 1024-wide tiles and document ids
    that are not sorted (a run of equal ids per cell, or ids repeating far
    apart), all against the oracle's cell-by-cell count."""
    rng = np.random.default_rng(99)
    cases = []
    for window in (1, 2, 1000, 2**31 - 1):
        for sinks in (0, 1, 5000):
            cases.append(("causal_window_sinks", window, sinks, None))
    for pattern in ("alternating", "random3", "reversed_runs"):
        cases.append(("doc_causal", 0, 0, pattern))
    n = 0
    for kind, window, sinks, pattern in cases:
        for L, S, QB, KB, off in ((1500, 2100, 1024, 1024, 600), (700, 700, 128, 64, 0), (33, 2000, 16, 1000, 1967)):
            doc_np = doc_t = None
            if kind == "doc_causal":
                m = max(S, off + L)
                if pattern == "alternating":
                    doc_np = (np.arange(m) % 2).astype(np.int32)
                elif pattern == "random3":
                    doc_np = rng.integers(0, 3, size=m).astype(np.int32)
                else:
                    doc_np = _rand_doc(rng, m)[::-1].copy()
                doc_t = torch.from_numpy(doc_np).to(dev)
            spec, mod = _mask_pair(kind, window, sinks, off, doc_np, doc_t)
            print(f"[blockmask] {kind} window={window} sinks={sinks} doc={pattern} L={L} S={S} "
                  f"tiles={QB}x{KB} q_offset={off}", flush=True)
            gpu = pbs.flex_blockmask_build(spec, L, S, QB, KB, device=dev)
            ref = build_block_mask(mod, L, S, QB, KB, q_offset=off)
            assert_block_mask_equal(gpu, ref)
            n += 1
    assert n == 45


@pytest.mark.parametrize("name", WORKLOAD_ORDER + EXTRA_WORKLOADS)
def test_blockmask_workloads_bit_exact(dev, name):
    w = WORKLOADS[name]
    doc_np = workload_doc_ids(w)
    doc_t = torch.from_numpy(doc_np).to(dev) if doc_np is not None else None
    spec, _ = specs(w, doc_t)
    mod = MaskMod(w.mask, window=w.window, sinks=w.sinks, doc_id=doc_np, clauses=w.clauses)
    gpu = pbs.flex_blockmask_build(spec, w.L, w.S, w.q_block, w.kv_block, device=dev)
    ref = build_block_mask(mod, w.L, w.S, w.q_block, w.kv_block, q_offset=w.q_offset)
    assert_block_mask_equal(gpu, ref)


# ------------------------------------------------------- attention, small cases
def _tensor(x_f32, dtype, dev):
    if dtype == "bf16":
        return torch.from_numpy(f32_to_bf16_bits(x_f32).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(dev)


def _widen(x_f32, dtype):
    return bf16_bits_to_f32(f32_to_bf16_bits(x_f32)) if dtype == "bf16" else x_f32


def run_case(dev, *, seed, dtype, B, Hq, Hkv, L, S, D, qb, kb, score, mask_kind, window=0, sinks=0,
             q_offset=None, value_scale=1.0, scale=None, with_lse=True, what="", clauses=(), bm_heads=1,
             with_max=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, L, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, S, D), dtype=np.float32) * np.float32(value_scale)
    off = S - L if q_offset is None else q_offset
    doc_np = doc_t = None
    if _uses_doc(mask_kind, clauses):
        doc_np = _rand_doc(rng, max(S, off + L))
        doc_t = torch.from_numpy(doc_np).to(dev)
    mspec, mmod = _mask_pair(mask_kind, window, sinks, off, doc_np, doc_t, clauses)
    sspec = pbs.ScoreSpec(**score)
    smod = ScoreMod(**score)
    bm = pbs.flex_blockmask_build(mspec, L, S, qb, kb, H=bm_heads, device=dev)
    qt, kt, vt = _tensor(q, dtype, dev), _tensor(k, dtype, dev), _tensor(v, dtype, dev)
    if with_max:
        out, lse, mx = pbs.flex_attn_fwd_aux(qt, kt, vt, block_mask=bm, score=sspec, mask=mspec, scale=scale,
                                             return_lse=with_lse)
    else:
        out, lse = pbs.flex_attn_fwd(qt, kt, vt, block_mask=bm, score=sspec, mask=mspec, scale=scale,
                                     return_lse=with_lse)
    torch.cuda.synchronize()
    sc = oracle_default_scale(D) if scale is None else float(np.float32(scale))
    out_ref, lse_ref, mx_ref = attention(_widen(q, dtype), _widen(k, dtype), _widen(v, dtype), scale=sc,
                                         score=smod, mask=mmod, q_offset=off, with_max=True)
    err = assert_attention_close(out, lse, out_ref, lse_ref, dtype, what)
    if with_max:
        # the row maximum is a score like lse: same error sources, same bound
        m = mx.cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isneginf(m), np.isneginf(mx_ref)), f"{what}: -inf pattern of max_scores"
        fin = ~np.isneginf(mx_ref)
        merr = np.abs(m[fin] - mx_ref[fin]).max() if fin.any() else 0.0
        print(f"[parity] {what}: max_scores max-abs {merr:.3e}")
        assert merr <= TOL_LSE, f"{what}: max_scores max-abs {merr:.3e}"
    return err


SCORES = [dict(kind="none"), dict(kind="softcap", cap=5.0), dict(kind="softcap_alibi", cap=30.0, alibi_m=8.0)]
MASKS = [dict(mask_kind="noop"), dict(mask_kind="causal"),
         dict(mask_kind="causal_window_sinks", window=70, sinks=3), dict(mask_kind="doc_causal")]


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("f32", 64), ("f32", 128)])
def test_attention_menu_small(dev, dtype, D):
    """Every score x mask pair on ragged lengths that span several tiles."""
    for i, (score, mask) in enumerate(itertools.product(SCORES, MASKS)):
        L, S = (300, 300) if i % 2 == 0 else (173, 389)
        run_case(dev, seed=100 + i, dtype=dtype, B=2, Hq=4, Hkv=2, L=L, S=S, D=D, qb=128, kb=64, score=score,
                 what=f"{dtype} D={D} {score} {mask}", **mask)


@pytest.mark.parametrize("qb,kb", [(16, 64), (32, 64), (64, 64), (64, 128), (128, 128), (128, 192)])
def test_attention_tile_shapes(dev, qb, kb):
    for dtype in ("bf16", "f32"):
        run_case(dev, seed=7 + qb + kb, dtype=dtype, B=1, Hq=2, Hkv=1, L=211, S=333, D=64, qb=qb, kb=kb,
                 score=dict(kind="softcap_alibi", cap=20.0), mask_kind="causal", what=f"{dtype} {qb}x{kb}")


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_attention_gqa_ratios(dev, G):
    run_case(dev, seed=40 + G, dtype="bf16", B=2, Hq=8, Hkv=8 // G, L=150, S=150, D=128, qb=128, kb=64,
             score=dict(kind="softcap", cap=50.0), mask_kind="causal_window_sinks", window=40, sinks=4,
             what=f"G={G}")


def _many_docs(rng, n, hi):
    """Document ids of n positions cut into documents of 1..hi tokens."""
    lens = []
    while sum(lens) < n:
        lens.append(int(rng.integers(1, hi + 1)))
    lens[-1] -= sum(lens) - n
    return np.repeat(np.arange(len(lens), dtype=np.int32), lens)


@pytest.mark.parametrize("D,qb,L", [(64, 128, 3000), (128, 128, 2100), (64, 64, 4200)])
def test_packed_documents_launch_order(dev, D, qb, L):
    """Many short documents whose boundaries fall inside Q blocks, so tile
    counts rise and fall along the sequence.  The prefill launches the Q blocks
    longest document first; every block must still be computed exactly once.
    Covers 128-row workgroups (D 64 and 128) and 64-row key-split ones (qb=64,
    66 blocks)."""
    rng = np.random.default_rng(900 + D + qb)
    Hq, Hkv = 2, 1
    q = rng.standard_normal((1, Hq, L, D), dtype=np.float32)
    k = rng.standard_normal((1, Hkv, L, D), dtype=np.float32)
    v = rng.standard_normal((1, Hkv, L, D), dtype=np.float32)
    doc_np = _many_docs(rng, L, 400)
    doc_t = torch.from_numpy(doc_np).to(dev)
    mspec, mmod = _mask_pair("doc_causal", 0, 0, 0, doc_np, doc_t)
    bm = pbs.flex_blockmask_build(mspec, L, L, qb, 64, device=dev)
    print(f"[parity] packed documents D={D} qb={qb} L={L}: {int(doc_np[-1]) + 1} documents, "
          f"{bm.kv_num_blocks.shape[-1]} Q blocks", flush=True)
    out, lse = pbs.flex_attn_fwd(_tensor(q, "bf16", dev), _tensor(k, "bf16", dev), _tensor(v, "bf16", dev),
                                 block_mask=bm, mask=mspec)
    torch.cuda.synchronize()
    out_ref, lse_ref, _ = attention(_widen(q, "bf16"), _widen(k, "bf16"), _widen(v, "bf16"),
                                    scale=oracle_default_scale(D), score=ScoreMod("none"), mask=mmod, q_offset=0,
                                    with_max=True)
    assert_attention_close(out, lse, out_ref, lse_ref, "bf16", f"packed documents D={D} qb={qb}")


def test_attention_empty_rows_and_offsets(dev):
    # L > S bottom-right: the first L - S rows see no key -> out 0, lse -inf
    run_case(dev, seed=3, dtype="bf16", B=1, Hq=2, Hkv=2, L=200, S=70, D=64, qb=64, kb=64,
             score=dict(kind="softcap", cap=10.0), mask_kind="causal", what="L>S")
    run_case(dev, seed=4, dtype="f32", B=1, Hq=2, Hkv=1, L=100, S=30, D=128, qb=32, kb=64,
             score=dict(kind="none"), mask_kind="causal", what="L>S f32")
    # negative and top-left offsets
    for off in (0, -17, 45):
        run_case(dev, seed=5, dtype="bf16", B=1, Hq=2, Hkv=1, L=90, S=260, D=64, qb=32, kb=64,
                 score=dict(kind="softcap_alibi", cap=30.0), mask_kind="causal", q_offset=off, what=f"off={off}")
    # window 1 (only self) and sinks only
    run_case(dev, seed=6, dtype="bf16", B=1, Hq=1, Hkv=1, L=130, S=130, D=64, qb=128, kb=64,
             score=dict(kind="none"), mask_kind="causal_window_sinks", window=1, sinks=0, what="w=1")
    run_case(dev, seed=6, dtype="bf16", B=1, Hq=1, Hkv=1, L=130, S=130, D=64, qb=128, kb=64,
             score=dict(kind="none"), mask_kind="causal_window_sinks", window=1, sinks=64, what="sinks")


def test_attention_minimum_sizes(dev):
    for L, S in ((1, 1), (1, 65), (17, 1), (2, 3)):
        for dtype in ("bf16", "f32"):
            run_case(dev, seed=L * 100 + S, dtype=dtype, B=1, Hq=1, Hkv=1, L=L, S=S, D=64, qb=16, kb=64,
                     score=dict(kind="softcap", cap=5.0), mask_kind="causal", what=f"L={L} S={S}")


def test_attention_large_scores_and_values(dev):
    # sharper softmax (scale 1) and large values exercise the rescale path and the bf16 budget
    run_case(dev, seed=9, dtype="f32", B=1, Hq=2, Hkv=2, L=256, S=256, D=64, qb=64, kb=64,
             score=dict(kind="none"), mask_kind="causal", scale=1.0, what="scale 1 f32")
    run_case(dev, seed=9, dtype="bf16", B=1, Hq=2, Hkv=2, L=256, S=256, D=64, qb=128, kb=64,
             score=dict(kind="softcap", cap=50.0), mask_kind="noop", scale=2.0, what="scale 2 bf16")
    run_case(dev, seed=10, dtype="bf16", B=1, Hq=2, Hkv=2, L=256, S=256, D=128, qb=128, kb=64,
             score=dict(kind="none"), mask_kind="causal", value_scale=0.5, what="values")


@pytest.mark.parametrize("mask_kind", ["causal", "noop"])
@pytest.mark.parametrize("score", [dict(kind="softcap", cap=30.0), dict(kind="softcap_alibi", cap=30.0),
                                   dict(kind="softcap", cap=50.0)])
def test_softcap_tiers_by_score_magnitude(dev, mask_kind, score):
    """Rows scaled so that different waves take the cubic, quintic and exact tanh paths."""
    rng = np.random.default_rng(21)
    B, H, L, S, D = 1, 2, 256, 256, 64
    q = rng.standard_normal((B, H, L, D), dtype=np.float32)
    q *= np.repeat(np.array([0.3, 1.0, 2.5, 6.0], dtype=np.float32), L // 4)[None, None, :, None]
    k = rng.standard_normal((B, H, S, D), dtype=np.float32)
    v = rng.standard_normal((B, H, S, D), dtype=np.float32)
    mspec, mmod = _mask_pair(mask_kind, q_offset=0)
    bm = pbs.flex_blockmask_build(mspec, L, S, 128, 64, device=dev)
    out, lse = pbs.flex_attn_fwd(_tensor(q, "bf16", dev), _tensor(k, "bf16", dev), _tensor(v, "bf16", dev),
                                 block_mask=bm, score=pbs.ScoreSpec(**score), mask=mspec)
    torch.cuda.synchronize()
    out_ref, lse_ref = attention(_widen(q, "bf16"), _widen(k, "bf16"), _widen(v, "bf16"), scale=oracle_default_scale(D),
                                 score=ScoreMod(**score), mask=mmod, q_offset=0)
    assert_attention_close(out, lse, out_ref, lse_ref, "bf16", f"tiers {score} {mask_kind}")


# Short query blocks against long key ranges take the GQA-packed split-KV
# decode kernel (query heads of one K/V head packed into the rows, key range
# split across workgroups, partials merged by the combine kernel).  Rows with
# only a few visible tiles give split ranges of zero, one or two tiles.
DECODE_CASES = [
    # G, q_block, L, S, mask, score
    (4, 16, 16, 4100, dict(mask_kind="causal"), dict(kind="softcap", cap=50.0)),
    (2, 16, 21, 3000, dict(mask_kind="causal_window_sinks", window=70, sinks=3),
     dict(kind="softcap_alibi", cap=30.0, alibi_m=8.0)),
    (2, 32, 40, 2600, dict(mask_kind="doc_causal"), dict(kind="none")),
    (1, 32, 7, 2100, dict(mask_kind="noop"), dict(kind="softcap", cap=5.0)),
    (4, 16, 33, 2500, dict(mask_kind="causal_window_sinks", window=300, sinks=0), dict(kind="none")),
]


@pytest.mark.parametrize("D", [64, 128])
def test_decode_split_kv_paths(dev, D):
    for i, (G, qb, L, S, mask, score) in enumerate(DECODE_CASES):
        B, Hkv = 2, 2
        probe = pbs.flex_blockmask_build(pbs.MaskSpec(kind="causal", q_offset=S - L), L, S, qb, 64, device=dev)
        assert pbs.flex_attn_fwd_workspace_bytes(torch.bfloat16, B, G * Hkv, Hkv, L, S, D, probe) > 0, \
            "case does not take the split-KV decode path"
        run_case(dev, seed=300 + i + D, dtype="bf16", B=B, Hq=G * Hkv, Hkv=Hkv, L=L, S=S, D=D, qb=qb, kb=64,
                 score=score, what=f"decode D={D} G={G} qb={qb} L={L} S={S} {mask} {score}", **mask)


def test_lse_optional_and_strided_inputs(dev):
    rng = np.random.default_rng(11)
    B, H, L, S, D = 2, 4, 190, 190, 64
    qkv = rng.standard_normal((3, B, L, H, D), dtype=np.float32)       # (B, L, H, D) storage
    t = _tensor(qkv, "bf16", dev)
    q, k, v = (t[i].permute(0, 2, 1, 3) for i in range(3))              # (B, H, L, D) views, strided
    mspec = pbs.MaskSpec(kind="causal")
    sspec = pbs.ScoreSpec(kind="softcap_alibi", cap=30.0)
    bm = pbs.flex_blockmask_build(mspec, L, S, 128, 64, device=dev)
    out_s, lse_s = pbs.flex_attn_fwd(q, k, v, block_mask=bm, score=sspec, mask=mspec)
    out_c, lse_c = pbs.flex_attn_fwd(q.contiguous(), k.contiguous(), v.contiguous(), block_mask=bm, score=sspec,
                                     mask=mspec)
    out_n, lse_n = pbs.flex_attn_fwd(q, k, v, block_mask=bm, score=sspec, mask=mspec, return_lse=False)
    torch.cuda.synchronize()
    assert lse_n is None
    assert torch.equal(out_s, out_c) and torch.equal(lse_s, lse_c) and torch.equal(out_s, out_n)


# ------------------------------------------------- the five full-size workloads
def _sample_rows(w: Workload, rng, n_random=48):
    edges = set()
    for qb in range(-(-w.L // w.q_block)):
        for r in (qb * w.q_block, qb * w.q_block + w.q_block - 1):
            if 0 <= r < w.L:
                edges.add(r)
    rows = sorted(edges | set(rng.integers(0, w.L, size=min(n_random, w.L)).tolist()) | {0, w.L - 1})
    if len(rows) > 96:
        rows = sorted(set(rng.choice(rows, size=96, replace=False).tolist()) | {0, w.L - 1})
    return np.array(rows, dtype=np.int64)


@pytest.mark.parametrize("name", WORKLOAD_ORDER + EXTRA_WORKLOADS)
def test_workload_parity_sampled(dev, name):
    w = WORKLOADS[name]
    inp = make_inputs(w)
    q, k, v, doc_t = to_device(w, inp, dev)
    mspec, sspec = specs(w, doc_t)
    bm = pbs.flex_blockmask_build(mspec, w.L, w.S, w.q_block, w.kv_block, device=dev)
    out, lse = pbs.flex_attn_fwd(q, k, v, block_mask=bm, score=sspec, mask=mspec)
    torch.cuda.synchronize()
    out_np = out.float().cpu().numpy()
    lse_np = lse.cpu().numpy()
    mmod, smod = oracle_mods(w, inp["doc_id"])
    rng = np.random.default_rng(w.seed)
    if w.B * w.Hq * w.L <= 1024:            # small workload: every output
        bs, hs, rows = range(w.B), range(w.Hq), np.arange(w.L)
    else:
        bs = sorted({0, w.B - 1})
        hs = sorted({0, w.Hq - 1, int(rng.integers(0, w.Hq))})
        rows = _sample_rows(w, rng)
    out_ref, lse_ref = attention(inp["q"], inp["k"], inp["v"], scale=oracle_default_scale(w.D), score=smod,
                                 mask=mmod, q_offset=w.q_offset, rows=rows, heads=hs, batches=bs)
    got_o = out_np[np.ix_(list(bs), list(hs), rows)]
    got_l = lse_np[np.ix_(list(bs), list(hs), rows)]
    assert_attention_close(got_o, got_l, out_ref, lse_ref, w.dtype, name)
    # properties that hold at any size: finite everywhere rows see keys, no NaN
    assert not np.isnan(out_np).any() and not np.isnan(lse_np).any()


# Whole (batch, head) slices at full size: every row of the first slice and
# of the last batch's last query head (plus one slice between them), so the
# launch orders that only change behaviour at full size (longest document
# first, the XCD-grouped GQA head order, the highest Q block first) are
# checked end to end on every row they touch.  The decode / verify workload
# is small enough per row to check every output.
FULL_SLICE_WORKLOADS = ["causal_softcap_alibi", "doc_causal", "window_sinks_gqa", "decode_verify",
                        "prefix_lm_alibi", "chunked_gqa"]


@pytest.mark.parametrize("name", FULL_SLICE_WORKLOADS)
def test_workload_parity_full_slices(dev, name):
    w = WORKLOADS[name]
    inp = make_inputs(w)
    q, k, v, doc_t = to_device(w, inp, dev)
    mspec, sspec = specs(w, doc_t)
    bm = pbs.flex_blockmask_build(mspec, w.L, w.S, w.q_block, w.kv_block, device=dev)
    out, lse = pbs.flex_attn_fwd(q, k, v, block_mask=bm, score=sspec, mask=mspec)
    torch.cuda.synchronize()
    out_np = out.float().cpu().numpy()
    lse_np = lse.cpu().numpy()
    del q, k, v, out, lse
    mmod, smod = oracle_mods(w, inp["doc_id"])
    if w.L * w.S <= 1 << 20:
        slices = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    else:
        mid = (w.B // 2, (w.Hq // 2) + 1 if w.Hq > 2 else 0)
        slices = sorted({(0, 0), mid, (w.B - 1, w.Hq - 1)})
    worst_o = worst_l = 0.0
    for b, h in slices:
        out_ref, lse_ref = attention(inp["q"], inp["k"], inp["v"], scale=oracle_default_scale(w.D), score=smod,
                                     mask=mmod, q_offset=w.q_offset, heads=[h], batches=[b])
        err_o = assert_attention_close(out_np[b:b + 1, h:h + 1], lse_np[b:b + 1, h:h + 1], out_ref, lse_ref,
                                       w.dtype, f"{name} full slice b={b} h={h}")
        fin = np.isfinite(lse_ref)
        err_l = float(np.abs(lse_np[b:b + 1, h:h + 1][fin] - lse_ref[fin]).max()) if fin.any() else 0.0
        worst_o, worst_l = max(worst_o, err_o), max(worst_l, err_l)
    print(f"[parity] {name}: {len(slices)} full (batch, head) slices of {w.L} rows, worst out max-abs "
          f"{worst_o:.3e}, worst lse max-abs {worst_l:.3e}", flush=True)


@pytest.mark.parametrize("dtype,D,L,S,qb", [("bf16", 64, 300, 300, 128), ("bf16", 128, 300, 300, 128),
                                            ("f32", 64, 300, 300, 64), ("f32", 128, 200, 200, 64),
                                            ("bf16", 128, 16, 3000, 16)])
def test_default_scale_is_the_pages_value(dev, dtype, D, L, S, qb):
    """scale=None (the library's default, scale <= 0 at the C ABI) gives
    bit-for-bit the result of passing the pages' default 1/sqrt(D), computed
    here in float64 and rounded once to float32 (2kiu guide, section 6.2),
    on the prefill and the split-KV decode paths."""
    rng = np.random.default_rng(77 + D + L)
    Hq, Hkv = 4, 2
    x = [rng.standard_normal(s, dtype=np.float32) for s in ((1, Hq, L, D), (1, Hkv, S, D), (1, Hkv, S, D))]
    q, k, v = (_tensor(t, dtype, dev) for t in x)
    mspec = pbs.MaskSpec(kind="causal")
    sspec = pbs.ScoreSpec(kind="softcap", cap=30.0)
    bm = pbs.flex_blockmask_build(mspec, L, S, qb, 64, device=dev)
    o_def, l_def = pbs.flex_attn_fwd(q, k, v, block_mask=bm, score=sspec, mask=mspec)
    o_exp, l_exp = pbs.flex_attn_fwd(q, k, v, block_mask=bm, score=sspec, mask=mspec, scale=oracle_default_scale(D))
    torch.cuda.synchronize()
    assert torch.equal(o_def, o_exp) and torch.equal(l_def, l_exp), \
        f"default scale differs from float32(1/sqrt({D})) = {oracle_default_scale(D)!r}"
    # and a different scale does change the result (the argument is not ignored)
    o_oth, _ = pbs.flex_attn_fwd(q, k, v, block_mask=bm, score=sspec, mask=mspec,
                                 scale=oracle_default_scale(D) * 1.25)
    torch.cuda.synchronize()
    assert not torch.equal(o_def, o_oth)


def test_run_to_run_bitwise_determinism(dev):
    w = WORKLOADS["causal_softcap_alibi"]
    inp = make_inputs(w)
    q, k, v, _ = to_device(w, inp, dev)
    mspec, sspec = specs(w)
    bm = pbs.flex_blockmask_build(mspec, w.L, w.S, w.q_block, w.kv_block, device=dev)
    o1, l1 = pbs.flex_attn_fwd(q, k, v, block_mask=bm, score=sspec, mask=mspec)
    o2, l2 = pbs.flex_attn_fwd(q, k, v, block_mask=bm, score=sspec, mask=mspec)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------ program masks, plain ALiBi, max_scores
# The tensorcad "Attention expressions" Examples (mask column) as programs:
# an AND of clauses, each an OR of predicates (2kiu guide, section 4.3).
PROGRAMS = {
    "prefix_lm": ((("causal", 0), ("kv_lt", 16)),),
    "sink_window": ((("causal", 0),), (("window", 40), ("kv_lt", 4))),
    "chunked": ((("causal", 0),), (("chunk", 48),)),
    "every_4th": ((("causal", 0),), (("stride", 4),)),
    "half_heads_global": ((("causal", 0),), (("head_lt", 2), ("window", 30))),
    "doc_window": ((("causal", 0),), (("doc", 0),), (("window", 90), ("kv_lt", 2))),
}


def _random_program(rng, with_head, with_doc):
    names = ["causal", "window", "kv_lt", "chunk", "stride"] + (["head_lt"] if with_head else []) + \
            (["doc"] if with_doc else [])
    clauses = []
    for _ in range(int(rng.integers(1, 5))):
        lits = []
        for _ in range(int(rng.integers(1, 3))):
            n = str(rng.choice(names))
            arg = {"causal": 0, "doc": 0, "window": int(rng.integers(1, 60)), "kv_lt": int(rng.integers(0, 40)),
                   "chunk": int(rng.integers(1, 70)), "stride": int(rng.integers(1, 7)),
                   "head_lt": int(rng.integers(0, 4))}[n]
            lits.append((n, arg))
        clauses.append(tuple(lits))
    return tuple(clauses)


def test_blockmask_program_fuzz_bit_exact(dev):
    rng = np.random.default_rng(4321)
    n = 0
    for trial in range(90):
        L, S = int(rng.integers(1, 260)), int(rng.integers(1, 260))
        QB = int(rng.choice([1, 3, 16, 64, 128]))
        KB = int(rng.choice([1, 5, 64, 128]))
        with_doc = trial % 3 == 0
        Hm = 3 if trial % 4 == 1 else 1
        off = int(rng.integers(0, 30)) if with_doc else int(rng.integers(-40, 40))
        clauses = _random_program(rng, Hm > 1, with_doc)
        doc_np = doc_t = None
        if with_doc:
            doc_np = _rand_doc(rng, max(S, off + L) + int(rng.integers(0, 3)))
            doc_t = torch.from_numpy(doc_np).to(dev)
        spec, mod = _mask_pair("program", q_offset=off, doc_np=doc_np, doc_t=doc_t, clauses=clauses)
        print(f"[blockmask] program {clauses} L={L} S={S} tiles={QB}x{KB} off={off} H={Hm}", flush=True)
        gpu = pbs.flex_blockmask_build(spec, L, S, QB, KB, H=Hm, device=dev)
        ref = build_block_mask(mod, L, S, QB, KB, H=Hm, q_offset=off)
        assert_block_mask_equal(gpu, ref)
        n += 1
    assert n == 90


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_attention_program_masks(dev, dtype, D):
    scores = [dict(kind="none"), dict(kind="softcap", cap=20.0), dict(kind="alibi", alibi_m=8.0)]
    for i, (name, clauses) in enumerate(PROGRAMS.items()):
        score = scores[i % len(scores)]
        Hq, Hkv = 4, 2
        bm_heads = Hq if any(n == "head_lt" for c in clauses for n, _ in c) else 1
        L, S = (211, 211) if i % 2 == 0 else (150, 333)
        run_case(dev, seed=500 + i, dtype=dtype, B=2, Hq=Hq, Hkv=Hkv, L=L, S=S, D=D, qb=128, kb=64, score=score,
                 mask_kind="program", clauses=clauses, bm_heads=bm_heads,
                 what=f"{dtype} D={D} {name} {score}")


def test_attention_fuzz_small(dev):
    """Random small cases over the whole menu: ragged L and S (L > S too),
    offsets, tile shapes, GQA ratios, head dims, dtypes, every mask kind (with
    random windows, sinks, documents and programs) and every score kind."""
    rng = np.random.default_rng(2468)
    kinds = ["noop", "causal", "causal_window_sinks", "doc_causal", "program"]
    scores = [dict(kind="none"), dict(kind="alibi", alibi_m=8.0)] + \
        [dict(kind=k, cap=float(c)) for k in ("softcap", "softcap_alibi") for c in (3.0, 20.0, 50.0)]
    for trial in range(40):
        dtype = "bf16" if trial % 3 else "f32"
        D = int(rng.choice([64, 128]))
        G = int(rng.choice([1, 2, 4]))
        Hkv = int(rng.integers(1, 3))
        L, S = int(rng.integers(1, 300)), int(rng.integers(1, 300))
        qb = int(rng.choice([16, 32, 64, 128]))
        kb = int(rng.choice([64, 128]))
        kind = kinds[trial % len(kinds)]
        score = scores[int(rng.integers(0, len(scores)))]
        off = None if trial % 4 else int(rng.integers(-40, 60))
        clauses = _random_program(rng, True, True) if kind == "program" else ()
        eff = S - L if off is None else off
        if eff < 0 and _uses_doc(kind, clauses):
            off = -eff   # document masks take q_offset >= 0 (a documented argument check)
        bm_heads = Hkv * G if any(n == "head_lt" for c in clauses for n, _ in c) else 1
        window, sinks = (int(rng.integers(1, 120)), int(rng.integers(0, 8))) if kind == "causal_window_sinks" else (0, 0)
        what = (f"fuzz {trial}: {dtype} D={D} G={G} Hkv={Hkv} L={L} S={S} tiles {qb}x{kb} {kind} {score} "
                f"off={off} w={window} s={sinks} {clauses}")
        print(f"[parity] {what}", flush=True)
        run_case(dev, seed=3000 + trial, dtype=dtype, B=2, Hq=Hkv * G, Hkv=Hkv, L=L, S=S, D=D, qb=qb, kb=kb,
                 score=score, mask_kind=kind, window=window, sinks=sinks, q_offset=off, clauses=clauses,
                 bm_heads=bm_heads, what=what)


@pytest.mark.parametrize("D", [64, 128])
def test_softcap_alibi_programs_that_hide_the_diagonal(dev, D):
    """Soft-cap plus distance bias under mask programs with a causal clause
    and a clause that can hide a row's own key, (causal) AND (kv < 4) and
    (causal) AND (h < 8 OR kv < 4): rows far down see only distant keys whose
    biased scores sit far below the cap, so their weights must not underflow
    (each such row has a finite lse).  Long enough rows that the bias of the
    nearest visible key reaches hundreds (base 2) in the first heads."""
    programs = {"causal_and_kv_lt": ((("causal", 0),), (("kv_lt", 4),)),
                "causal_and_head_or_kv": ((("causal", 0),), (("head_lt", 8), ("kv_lt", 4)))}
    for i, (name, clauses) in enumerate(programs.items()):
        bm_heads = 16 if name == "causal_and_head_or_kv" else 1
        run_case(dev, seed=820 + i + D, dtype="bf16", B=1, Hq=16, Hkv=16 if D == 64 else 4, L=1024, S=1024, D=D,
                 qb=128, kb=64, score=dict(kind="softcap_alibi", cap=30.0, alibi_m=8.0), mask_kind="program",
                 clauses=clauses, bm_heads=bm_heads, what=f"softcap_alibi D={D} {name}")


@pytest.mark.parametrize("case", ["softcap_alibi_causal", "none_noop", "softcap_doc", "alibi_program", "max_window"])
def test_attention_128_row_workgroups_d64(dev, case):
    """bf16 at head dim 64 with B*Hq*ceil(L/128) >= 768 row blocks, enough
    that the prefill takes 128-row workgroups in which each wave computes
    both key halves of a tile (QK^T of the second half overlapping the first
    half's softmax).  Ragged L and S, GQA 4, every output checked."""
    score, mask = {
        "softcap_alibi_causal": (dict(kind="softcap_alibi", cap=30.0, alibi_m=8.0), dict(mask_kind="causal")),
        "none_noop": (dict(kind="none"), dict(mask_kind="noop")),
        "softcap_doc": (dict(kind="softcap", cap=5.0), dict(mask_kind="doc_causal")),
        "alibi_program": (dict(kind="alibi", alibi_m=8.0), dict(mask_kind="program", clauses=PROGRAMS["prefix_lm"])),
        "max_window": (dict(kind="softcap", cap=20.0), dict(mask_kind="causal_window_sinks", window=90, sinks=2)),
    }[case]
    run_case(dev, seed=700 + len(case), dtype="bf16", B=2, Hq=128, Hkv=32, L=300, S=333, D=64, qb=128, kb=64,
             score=score, with_max=case == "max_window", what=f"128-row workgroups D=64 {case}", **mask)


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("f32", 128)])
def test_plain_alibi_score(dev, dtype, D):
    for i, mask in enumerate(MASKS):
        run_case(dev, seed=600 + i, dtype=dtype, B=1, Hq=8, Hkv=4, L=190, S=260, D=D, qb=64, kb=64,
                 score=dict(kind="alibi", alibi_m=8.0), what=f"{dtype} D={D} alibi {mask}", **mask)


def test_max_scores_output(dev):
    cases = [
        dict(dtype="bf16", D=64, score=dict(kind="softcap_alibi", cap=30.0), mask_kind="causal"),
        dict(dtype="bf16", D=128, score=dict(kind="softcap", cap=50.0), mask_kind="causal_window_sinks",
             window=40, sinks=3),
        dict(dtype="bf16", D=64, score=dict(kind="none"), mask_kind="program", clauses=PROGRAMS["every_4th"]),
        dict(dtype="f32", D=64, score=dict(kind="alibi"), mask_kind="doc_causal"),
    ]
    for i, c in enumerate(cases):
        c = dict(c)
        run_case(dev, seed=700 + i, B=2, Hq=4, Hkv=2, L=170, S=230, qb=128, kb=64, with_max=True,
                 what=f"max_scores {c}", **c)
    # rows with no visible key (L > S, bottom-right): max_scores = -inf there
    run_case(dev, seed=710, dtype="bf16", B=1, Hq=2, Hkv=1, L=200, S=90, D=64, qb=64, kb=64,
             score=dict(kind="softcap", cap=10.0), mask_kind="causal", with_max=True, what="max_scores empty rows")


def test_decode_path_programs_alibi_and_max(dev):
    cases = [
        (dict(mask_kind="program", clauses=PROGRAMS["chunked"]), dict(kind="softcap", cap=50.0), False),
        (dict(mask_kind="program", clauses=PROGRAMS["prefix_lm"]), dict(kind="alibi"), False),
        (dict(mask_kind="causal"), dict(kind="softcap", cap=50.0), True),
        (dict(mask_kind="program", clauses=PROGRAMS["doc_window"]), dict(kind="none"), True),
    ]
    for i, (mask, score, with_max) in enumerate(cases):
        for D in (64, 128):
            B, Hkv, G, qb, L, S = 2, 2, 4, 16, 16, 3100
            probe = pbs.flex_blockmask_build(pbs.MaskSpec(kind="causal"), L, S, qb, 64, device=dev)
            assert pbs.flex_attn_fwd_workspace_bytes(torch.bfloat16, B, G * Hkv, Hkv, L, S, D, probe) > 0
            run_case(dev, seed=800 + i + D, dtype="bf16", B=B, Hq=G * Hkv, Hkv=Hkv, L=L, S=S, D=D, qb=qb, kb=64,
                     score=score, with_max=with_max, what=f"decode D={D} {mask} {score} max={with_max}", **mask)


def test_binding_rejects_wrong_buffers(dev):
    """Every tensor handed to the binding is checked (device, dtype, exact
    shape, contiguity) before any pointer is marshalled: each wrong buffer is
    a ValueError and the output the call would have written is untouched."""
    rng = np.random.default_rng(5)
    B, H, L, D = 1, 2, 130, 64
    x = [_tensor(rng.standard_normal((B, H, L, D), dtype=np.float32), "bf16", dev) for _ in range(3)]
    q, k, v = x
    mspec = pbs.MaskSpec(kind="causal")
    bm = pbs.flex_blockmask_build(mspec, L, L, 128, 64, device=dev)
    good_out = torch.full((B, H, L, D), 7.0, dtype=torch.bfloat16, device=dev)
    cases = {
        "out too small": dict(out=torch.empty((B, H, L - 1, D), dtype=torch.bfloat16, device=dev)),
        "out wrong dtype": dict(out=torch.empty((B, H, L, D), dtype=torch.float32, device=dev)),
        "out strided": dict(out=torch.empty((B, H, D, L), dtype=torch.bfloat16, device=dev).transpose(2, 3)),
        "out on host": dict(out=torch.empty((B, H, L, D), dtype=torch.bfloat16)),
        "lse wrong dtype": dict(out=good_out, lse=torch.empty((B, H, L), dtype=torch.bfloat16, device=dev)),
        "lse too small": dict(out=good_out, lse=torch.empty((B, H, L - 5), dtype=torch.float32, device=dev)),
    }
    for what, kw in cases.items():
        with pytest.raises(ValueError):
            pbs.flex_attn_fwd(q, k, v, block_mask=bm, mask=mspec, **kw)
    with pytest.raises(ValueError, match="GPU tensor"):
        pbs.flex_attn_fwd(q, k.cpu(), v, block_mask=bm, mask=mspec, out=good_out)
    bm64 = pbs.BlockMask(bm.kv_num_blocks.long(), bm.kv_indices, bm.full_kv_num_blocks, bm.full_kv_indices,
                         bm.q_block, bm.kv_block, bm.L, bm.S)
    with pytest.raises(ValueError):
        pbs.flex_attn_fwd(q, k, v, block_mask=bm64, mask=mspec, out=good_out)
    short = pbs.BlockMask(bm.kv_num_blocks, bm.kv_indices[..., :1].contiguous(), bm.full_kv_num_blocks,
                          bm.full_kv_indices, bm.q_block, bm.kv_block, bm.L, bm.S)
    with pytest.raises(ValueError):
        pbs.flex_attn_fwd(q, k, v, block_mask=short, mask=mspec, out=good_out)
    # the split-KV path's workspace: a too-small one is refused, not replaced
    Lq, S = 16, 3000
    qd = _tensor(rng.standard_normal((1, 4, Lq, D), dtype=np.float32), "bf16", dev)
    kd = _tensor(rng.standard_normal((1, 1, S, D), dtype=np.float32), "bf16", dev)
    mdec = pbs.MaskSpec(kind="causal")
    bmd = pbs.flex_blockmask_build(mdec, Lq, S, 16, 64, device=dev)
    need = pbs.flex_attn_fwd_workspace_bytes(torch.bfloat16, 1, 4, 1, Lq, S, D, bmd)
    assert need > 0
    with pytest.raises(ValueError, match="workspace"):
        pbs.flex_attn_fwd(qd, kd, kd, block_mask=bmd, mask=mdec,
                          workspace=torch.empty(need - 16, dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()
    assert bool((good_out == 7.0).all()), "a rejected call wrote its output"
