"""GPU parity of the backward pass: dq, dk, dv from the HIP path (through the C
ABI) against the CPU oracle's float64 gradients, and the Q-side block lists bit
for bit against the oracle's transpose.

The HIP backward takes the HIP forward's out and lse, as a caller would; the
oracle differentiates the exact definition.  Tolerance per gradient tensor g
with oracle value r, elementwise:

  |g - r| <= TOL_ABS * max(max|r|, 1) + TOL_REL * |r|

(the floor of 1 is the magnitude of gradients of unit-normal inputs; it keeps
the bound meaningful where the exact gradient vanishes, e.g. dq when every
row sees one key).  bf16 (TOL_ABS 1e-2, TOL_REL 2e-2): the inputs are exact;
the largest error source is D_i, formed from the forward's bf16 output: its
error, about 2^-9 |dout_i| |out_i|, is common to a whole row of dS and reaches
dq_i as that times scale * |sum_j P_ij k_j| (about 1e-2 at unit-normal inputs
and head dim 64); next come the bf16 roundings of P and dS before their
products and of the gradients themselves (2^-9 relative each).  fp32 (TOL_ABS
1e-5, TOL_REL 1e-4): products in fp32 MFMA, exp2 and the soft-cap tanh in fp32,
so errors of a few fp32 ulps of the largest score propagate (about 1e-6 of
the largest gradient).
"""
import itertools

import numpy as np
import pytest
import torch

import programmable_block_sparse_amd as pbs
from gpu_common import assert_attention_close, assert_block_mask_equal, require_gpu
from oracle import MaskMod, ScoreMod, attention, attention_backward, build_block_mask, transpose_block_mask
from oracle import default_scale as oracle_default_scale
from workloads import WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs, make_upstream
from workloads.torch_io import specs, to_device

pytestmark = pytest.mark.gpu

TOL = {"bf16": (1e-2, 2e-2), "f32": (1e-5, 1e-4)}


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _tensor(x_f32, dtype, dev):
    if dtype == "bf16":
        return torch.from_numpy(f32_to_bf16_bits(x_f32).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(dev)


def _widen(x_f32, dtype):
    return bf16_bits_to_f32(f32_to_bf16_bits(x_f32)) if dtype == "bf16" else x_f32


def _rand_doc(rng, n):
    cuts = np.sort(rng.choice(np.arange(1, n), size=min(n - 1, int(rng.integers(0, 5))), replace=False)) if n > 1 else []
    lens = np.diff(np.concatenate([[0], cuts, [n]])).astype(np.int64)
    return np.repeat(np.arange(len(lens), dtype=np.int32), lens)


def assert_grads_close(got, ref, dtype, what):
    ta, tr = TOL[dtype]
    worst = []
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = g.float().cpu().numpy().astype(np.float64) if isinstance(g, torch.Tensor) else g
        assert not np.isnan(g).any(), f"{what}: NaN in {name}"
        scale = max(np.abs(r).max(), 1.0) if r.size else 1.0
        err = np.abs(g - r)
        bound = ta * scale + tr * np.abs(r)
        ratio = (err / np.maximum(bound, 1e-30)).max() if r.size else 0.0
        worst.append(f"{name} max-abs {err.max():.2e} (max|ref| {scale:.2e}, {ratio:.2f} of bound)")
        assert (err <= bound).all(), f"{what}: {name} exceeds tolerance at {np.argwhere(err > bound)[:4].tolist()}: " \
                                     f"{worst[-1]}"
    print(f"[bwd parity] {what}: " + "; ".join(worst))


def _many_docs(rng, n, hi):
    """Document ids of n positions cut into documents of 1..hi tokens."""
    lens = []
    while sum(lens) < n:
        lens.append(int(rng.integers(1, hi + 1)))
    lens[-1] -= sum(lens) - n
    return np.repeat(np.arange(len(lens), dtype=np.int32), lens)


def run_bwd_case(dev, *, seed, dtype, B, Hq, Hkv, L, S, D, qb, kb, score, mask_kind, window=0, sinks=0,
                 q_offset=None, clauses=(), bm_heads=1, scale=None, what="", doc_max=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, L, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    do = rng.standard_normal((B, Hq, L, D), dtype=np.float32)
    off = S - L if q_offset is None else q_offset
    clauses = tuple(tuple(c) for c in clauses)
    doc_np = doc_t = None
    if mask_kind == "doc_causal" or any(n == "doc" for c in clauses for n, _ in c):
        n = max(S, off + L)
        doc_np = _many_docs(rng, n, doc_max) if doc_max else _rand_doc(rng, n)
        doc_t = torch.from_numpy(doc_np).to(dev)
    mspec = pbs.MaskSpec(kind=mask_kind, window=window, sinks=sinks, q_offset=off, doc_id=doc_t, clauses=clauses)
    mmod = MaskMod(mask_kind, window=window, sinks=sinks, doc_id=doc_np, clauses=clauses)
    sspec, smod = pbs.ScoreSpec(**score), ScoreMod(**score)
    bm = pbs.flex_blockmask_build(mspec, L, S, qb, kb, H=bm_heads, device=dev)
    bmq = pbs.flex_blockmask_transpose(bm)
    qt, kt, vt, dot = (_tensor(x, dtype, dev) for x in (q, k, v, do))
    out, lse = pbs.flex_attn_fwd(qt, kt, vt, block_mask=bm, score=sspec, mask=mspec, scale=scale)
    grads = pbs.flex_attn_bwd(qt, kt, vt, out, dot, lse, block_mask=bm, block_mask_q=bmq, score=sspec, mask=mspec,
                              scale=scale)
    torch.cuda.synchronize()
    sc = oracle_default_scale(D) if scale is None else float(np.float32(scale))
    ref = attention_backward(_widen(q, dtype), _widen(k, dtype), _widen(v, dtype), _widen(do, dtype), scale=sc,
                             score=smod, mask=mmod, q_offset=off)
    assert_grads_close(grads, ref, dtype, what)
    return grads


SCORES = [dict(kind="none"), dict(kind="softcap", cap=5.0), dict(kind="softcap_alibi", cap=30.0, alibi_m=8.0),
          dict(kind="alibi", alibi_m=4.0)]
MASKS = [dict(mask_kind="noop"), dict(mask_kind="causal"),
         dict(mask_kind="causal_window_sinks", window=70, sinks=3), dict(mask_kind="doc_causal")]


# ------------------------------------------------------------ Q-side lists
def test_transpose_bit_exact(dev):
    rng = np.random.default_rng(321)
    kinds = ["noop", "causal", "causal_window_sinks", "doc_causal"]
    for trial in range(60):
        L, S = int(rng.integers(1, 400)), int(rng.integers(1, 400))
        QB = int(rng.choice([1, 3, 16, 64, 128]))
        KB = int(rng.choice([1, 2, 16, 64, 128]))
        kind = kinds[trial % 4]
        off = int(rng.integers(0, 40)) if kind == "doc_causal" else int(rng.integers(-40, 40))
        doc_np = doc_t = None
        if kind == "doc_causal":
            doc_np = _rand_doc(rng, max(S, off + L))
            doc_t = torch.from_numpy(doc_np).to(dev)
        window, sinks = int(rng.integers(1, 60)), int(rng.integers(0, 6))
        spec = pbs.MaskSpec(kind=kind, window=window, sinks=sinks, q_offset=off, doc_id=doc_t)
        mod = MaskMod(kind, window=window, sinks=sinks, doc_id=doc_np)
        Bm, Hm = (1, 1) if trial % 3 else (2, 3)
        bm = pbs.flex_blockmask_build(spec, L, S, QB, KB, B=Bm, H=Hm, device=dev)
        got = pbs.flex_blockmask_transpose(bm)
        want = transpose_block_mask(build_block_mask(mod, L, S, QB, KB, B=Bm, H=Hm, q_offset=off))
        for name in ("q_num_blocks", "q_indices", "full_q_num_blocks", "full_q_indices"):
            arr = getattr(got, name).cpu().numpy()
            assert np.array_equal(arr, want[name]), f"trial {trial} {name} differs"


# ------------------------------------------------------------- gradients
@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("f32", 64), ("f32", 128)])
def test_bwd_menu_small(dev, dtype, D):
    """Every score x mask pair on ragged lengths that span several tiles."""
    for i, (score, mask) in enumerate(itertools.product(SCORES, MASKS)):
        L, S = (300, 300) if i % 2 == 0 else (173, 389)
        run_bwd_case(dev, seed=500 + i, dtype=dtype, B=2, Hq=4, Hkv=2, L=L, S=S, D=D, qb=128, kb=64, score=score,
                     what=f"{dtype} D={D} {score['kind']} {mask['mask_kind']} L={L} S={S}", **mask)


@pytest.mark.parametrize("qb,kb", [(64, 64), (64, 128), (128, 128), (128, 192)])
def test_bwd_tile_shapes(dev, qb, kb):
    for dtype in ("bf16", "f32"):
        run_bwd_case(dev, seed=70 + qb + kb, dtype=dtype, B=1, Hq=2, Hkv=1, L=211, S=333, D=64, qb=qb, kb=kb,
                     score=dict(kind="softcap_alibi", cap=20.0), mask_kind="causal", what=f"{dtype} {qb}x{kb}")


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_bwd_gqa_ratios(dev, G):
    run_bwd_case(dev, seed=80 + G, dtype="bf16", B=2, Hq=8, Hkv=8 // G, L=150, S=150, D=128, qb=128, kb=64,
                 score=dict(kind="softcap", cap=50.0), mask_kind="causal_window_sinks", window=40, sinks=4,
                 what=f"G={G}")


def test_bwd_empty_rows_and_offsets(dev):
    # L > S bottom-right: the first L - S rows see no key and get dq = 0
    g = run_bwd_case(dev, seed=13, dtype="bf16", B=1, Hq=2, Hkv=2, L=200, S=70, D=64, qb=64, kb=64,
                     score=dict(kind="softcap", cap=10.0), mask_kind="causal", what="L>S")
    assert not g[0][:, :, :130].float().abs().max().item()
    run_bwd_case(dev, seed=14, dtype="f32", B=1, Hq=2, Hkv=1, L=100, S=30, D=128, qb=64, kb=64,
                 score=dict(kind="none"), mask_kind="causal", what="L>S f32")
    for off in (0, -17, 45):
        run_bwd_case(dev, seed=15, dtype="bf16", B=1, Hq=2, Hkv=1, L=90, S=260, D=64, qb=64, kb=64,
                     score=dict(kind="softcap_alibi", cap=30.0), mask_kind="causal", q_offset=off,
                     what=f"off={off}")
    # window 1 (only self): P = 1, so dq = dk = 0 and dv = dout of the one row
    run_bwd_case(dev, seed=16, dtype="bf16", B=1, Hq=1, Hkv=1, L=130, S=130, D=64, qb=128, kb=64,
                 score=dict(kind="none"), mask_kind="causal_window_sinks", window=1, sinks=0, what="w=1")
    # one query row, one key
    run_bwd_case(dev, seed=17, dtype="f32", B=1, Hq=1, Hkv=1, L=1, S=1, D=64, qb=64, kb=64,
                 score=dict(kind="softcap", cap=3.0), mask_kind="noop", what="1x1")
    # an explicit scale
    run_bwd_case(dev, seed=18, dtype="bf16", B=1, Hq=2, Hkv=2, L=129, S=257, D=128, qb=128, kb=128,
                 score=dict(kind="softcap", cap=8.0), mask_kind="noop", scale=0.3, what="scale=0.3")


PROGRAMS = [
    ((("causal", 0), ("kv_lt", 40)),),                               # prefix-LM
    ((("causal", 0),), (("chunk", 48),)),                           # chunked causal
    ((("causal", 0),), (("stride", 4),)),                           # every fourth key
    ((("causal", 0),), (("head_lt", 2), ("window", 24))),           # half the heads global
    ((("doc", 0),), (("window", 100), ("kv_lt", 2))),               # documents, windowed, with sinks
]


@pytest.mark.parametrize("pi", range(len(PROGRAMS)))
def test_bwd_programs(dev, pi):
    clauses = PROGRAMS[pi]
    heads = 4 if any(n == "head_lt" for c in clauses for n, _ in c) else 1
    for dtype, D in (("bf16", 64), ("f32", 128)):
        run_bwd_case(dev, seed=90 + pi, dtype=dtype, B=1, Hq=4, Hkv=2, L=230, S=230, D=D, qb=64, kb=64,
                     score=dict(kind="softcap_alibi", cap=20.0), mask_kind="program", clauses=clauses,
                     bm_heads=heads, what=f"program {pi} {dtype}")


def _i32(x, dev):
    return torch.tensor(np.asarray(x, dtype=np.int32), device=dev)


def run_bwd_per_batch(dev, *, seed, dtype, B, Hq, Hkv, L, S, D, qb, kb, score, mask_kind, offs, lens, window=0,
                      sinks=0, clauses=(), doc_max=0, split_cols=False, what=""):
    """Backward with per-batch query offsets and filled key lengths (the
    blog's decode section: a cache's capacity S is not its filled length).
    The GPU BlockMask and forward are checked against the oracle first, so a
    failure names the stage; then the gradients, including zero dk, dv rows
    for keys at or past each batch's length."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, L, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    do = rng.standard_normal((B, Hq, L, D), dtype=np.float32)
    clauses = tuple(tuple(c) for c in clauses)
    doc_np = doc_t = None
    if mask_kind == "doc_causal" or any(n == "doc" for c in clauses for n, _ in c):
        # ids for positions [0, max(S, L)); query positions outside have no document
        doc_np = _many_docs(rng, max(S, L), doc_max)
        doc_t = torch.from_numpy(doc_np).to(dev)
    spec = pbs.MaskSpec(kind=mask_kind, window=window, sinks=sinks, q_offset=0, doc_id=doc_t, clauses=clauses,
                        q_offsets=_i32(offs, dev), kv_lens=_i32(lens, dev))
    mod = MaskMod(mask_kind, window=window, sinks=sinks, doc_id=doc_np, clauses=clauses)
    heads = Hq if any(n == "head_lt" for c in clauses for n, _ in c) else 1
    bm = pbs.flex_blockmask_build(spec, L, S, qb, kb, B=B, H=heads, device=dev)
    assert_block_mask_equal(bm, build_block_mask(mod, L, S, qb, kb, B=B, H=heads, q_offset=offs, kv_len=lens))
    bmq = pbs.flex_blockmask_transpose(bm)
    sspec, smod = pbs.ScoreSpec(**score), ScoreMod(**score)
    qt, kt, vt, dot = (_tensor(x, dtype, dev) for x in (q, k, v, do))
    out, lse = pbs.flex_attn_fwd(qt, kt, vt, block_mask=bm, score=sspec, mask=spec)
    grads = pbs.flex_attn_bwd(qt, kt, vt, out, dot, lse, block_mask=bm, block_mask_q=bmq, score=sspec, mask=spec)
    if split_cols:
        ws = pbs.flex_attn_bwd_workspace_bytes(qt.dtype, B, Hq, Hkv, L, S, D, bm)
        assert ws > 2 * B * Hq * ((L + 127) // 128 * 128) * 4, "case does not split long columns"
    torch.cuda.synchronize()
    sc = oracle_default_scale(D)
    qw, kw, vw, dw = (_widen(x, dtype) for x in (q, k, v, do))
    out_ref, lse_ref = attention(qw, kw, vw, scale=sc, score=smod, mask=mod, q_offset=offs, kv_len=lens)
    assert_attention_close(out, lse, out_ref, lse_ref, dtype, f"{what} forward")
    ref = attention_backward(qw, kw, vw, dw, scale=sc, score=smod, mask=mod, q_offset=offs, kv_len=lens)
    assert_grads_close(grads, ref, dtype, what)
    for b, n in enumerate(lens):
        if n < S:
            assert grads[1][b, :, n:].float().abs().max().item() == 0, f"{what}: dk of batch {b} past its length"
            assert grads[2][b, :, n:].float().abs().max().item() == 0, f"{what}: dv of batch {b} past its length"


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("f32", 64), ("f32", 128)])
def test_bwd_per_batch_offsets_and_lengths(dev, dtype, D):
    run_bwd_per_batch(dev, seed=400 + D, dtype=dtype, B=3, Hq=4, Hkv=2, L=150, S=400, D=D, qb=64, kb=64,
                      score=dict(kind="softcap_alibi", cap=20.0, alibi_m=8.0), mask_kind="causal",
                      offs=[250, 0, 40], lens=[400, 130, 230], what=f"per-batch causal {dtype} D={D}")
    run_bwd_per_batch(dev, seed=410 + D, dtype=dtype, B=2, Hq=2, Hkv=1, L=130, S=300, D=D, qb=128, kb=64,
                      score=dict(kind="softcap", cap=5.0), mask_kind="causal_window_sinks", window=60, sinks=3,
                      offs=[170, -20], lens=[300, 77], what=f"per-batch window {dtype} D={D}")
    run_bwd_per_batch(dev, seed=420 + D, dtype=dtype, B=2, Hq=4, Hkv=4, L=100, S=260, D=D, qb=64, kb=128,
                      score=dict(kind="alibi", alibi_m=4.0), mask_kind="noop", offs=[0, 0], lens=[260, 1],
                      what=f"per-batch lengths noop {dtype} D={D}")


def test_bwd_per_batch_documents_and_programs(dev):
    # query positions before 0 or past the id array have no document
    run_bwd_per_batch(dev, seed=430, dtype="bf16", B=3, Hq=2, Hkv=1, L=200, S=500, D=64, qb=64, kb=64,
                      score=dict(kind="none"), mask_kind="doc_causal", offs=[-30, 120, 400], lens=[500, 330, 500],
                      doc_max=90, what="per-batch documents")
    run_bwd_per_batch(dev, seed=431, dtype="f32", B=2, Hq=2, Hkv=2, L=120, S=300, D=64, qb=64, kb=64,
                      score=dict(kind="softcap", cap=10.0), mask_kind="doc_causal", offs=[250, -60], lens=[300, 200],
                      doc_max=70, what="per-batch documents f32")
    for pi, clauses in enumerate(PROGRAMS):
        run_bwd_per_batch(dev, seed=440 + pi, dtype="bf16", B=2, Hq=4, Hkv=2, L=160, S=330, D=64, qb=64, kb=64,
                          score=dict(kind="softcap_alibi", cap=20.0), mask_kind="program", clauses=clauses,
                          offs=[170, -7], lens=[330, 150], doc_max=80, what=f"per-batch program {pi}")


def test_bwd_per_batch_long_columns(dev):
    # columns long enough to be split across workgroups, with lengths
    run_bwd_per_batch(dev, seed=450, dtype="bf16", B=2, Hq=8, Hkv=1, L=1100, S=1100, D=64, qb=128, kb=64,
                      score=dict(kind="softcap", cap=20.0), mask_kind="noop", offs=[0, 0], lens=[1100, 700],
                      split_cols=True, what="per-batch split columns")


@pytest.mark.parametrize("dtype,D,page,kb", [("bf16", 64, 64, 64), ("bf16", 128, 128, 64), ("f32", 64, 64, 64),
                                             ("f32", 128, 256, 64), ("bf16", 64, 64, 128)])
def test_bwd_paged_cache(dev, dtype, D, page, kb):
    """Backward over a paged cache: K/V scattered into a shuffled pool whose
    unfilled rows hold finite junk.  Fed the same out and lse, the paged
    backward must give the contiguous backward's gradients bit for bit (same
    arithmetic, other addresses), and both match the oracle.  With 128-key
    blocks over 700 keys the last block's second tile starts past the last
    page."""
    B, Hq, Hkv, L, S = 3, 4, 2, 150, 700
    offs, lens = [S - L, 300, 40], [S, 300 + L, 190]
    rng = np.random.default_rng(500 + D + page)
    q = rng.standard_normal((B, Hq, L, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    do = rng.standard_normal((B, Hq, L, D), dtype=np.float32)
    score = dict(kind="softcap_alibi", cap=20.0, alibi_m=8.0)
    spec = pbs.MaskSpec(kind="causal", q_offset=0, q_offsets=_i32(offs, dev), kv_lens=_i32(lens, dev))
    bm = pbs.flex_blockmask_build(spec, L, S, 64, kb, B=B, device=dev)
    bmq = pbs.flex_blockmask_transpose(bm)
    sspec = pbs.ScoreSpec(**score)
    n_log = -(-S // page)
    n_phys = B * n_log + 3
    table = rng.permutation(n_phys)[:B * n_log].reshape(B, n_log).astype(np.int32)
    pool_k = rng.uniform(-50, 50, (n_phys, Hkv, page, D)).astype(np.float32)   # junk where nothing was written
    pool_v = rng.uniform(-50, 50, (n_phys, Hkv, page, D)).astype(np.float32)
    for b in range(B):
        for p in range(-(-lens[b] // page)):
            n = min(page, lens[b] - p * page)
            pool_k[table[b, p], :, :n] = k[b, :, p * page:p * page + n]
            pool_v[table[b, p], :, :n] = v[b, :, p * page:p * page + n]
    qt, kt, vt, dot = (_tensor(x, dtype, dev) for x in (q, k, v, do))
    pk, pv = _tensor(pool_k, dtype, dev), _tensor(pool_v, dtype, dev)
    tt = torch.from_numpy(table).to(dev)
    out, lse = pbs.flex_attn_fwd(qt, kt, vt, block_mask=bm, score=sspec, mask=spec)
    out_p, lse_p, _ = pbs.flex_attn_fwd_paged(qt, pk, pv, tt, S=S, block_mask=bm, score=sspec, mask=spec)
    g_c = pbs.flex_attn_bwd(qt, kt, vt, out, dot, lse, block_mask=bm, block_mask_q=bmq, score=sspec, mask=spec)
    g_p = pbs.flex_attn_bwd_paged(qt, pk, pv, tt, out, dot, lse, S=S, block_mask=bm, block_mask_q=bmq, score=sspec,
                                  mask=spec)
    torch.cuda.synchronize()
    what = f"paged bwd {dtype} D={D} page={page} kv_block={kb}"
    assert torch.equal(out_p, out) and torch.equal(lse_p, lse), f"{what}: paged forward differs from contiguous"
    for name, a_, c_ in zip(("dq", "dk", "dv"), g_p, g_c):
        assert torch.equal(a_, c_), f"{what}: {name} differs from the contiguous backward"
    sc = oracle_default_scale(D)
    ref = attention_backward(_widen(q, dtype), _widen(k, dtype), _widen(v, dtype), _widen(do, dtype), scale=sc,
                             score=ScoreMod(**score), mask=MaskMod("causal"), q_offset=offs, kv_len=lens)
    assert_grads_close(g_p, ref, dtype, what)


@pytest.mark.parametrize("D,L,sinks", [(64, 300, 0), (128, 300, 0), (128, 1100, 4)])
def test_bwd_deterministic(dev, D, L, sinks):
    """Two runs give bitwise equal gradients: every dq row and every dk, dv
    key is written by one workgroup and split sums are added in a fixed order.
    Head dim 128 under GQA takes the single shared launch; L = 1100 with sinks
    under GQA 8 adds long Q-side columns cut into shares."""
    kw = dict(seed=5, dtype="bf16", B=2, Hq=8, Hkv=1 if sinks else 2, L=L, S=L, D=D, qb=128, kb=64,
              score=dict(kind="softcap_alibi", cap=30.0),
              mask_kind="causal_window_sinks" if sinks else "causal", window=128, sinks=sinks,
              what=f"det D={D} L={L} sinks={sinks}")
    a = run_bwd_case(dev, **kw)
    b = run_bwd_case(dev, **kw)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_full_size_sampled(dev):
    """The soft-capped causal workload at full size (B=4, H=16, L=S=2048, D=64,
    bf16, 128x64 tiles), checked on two (batch, head) slices against the
    dense oracle, and every other slice against the same bound being finite."""
    w = WORKLOADS["causal_softcap_alibi"]
    inp = make_inputs(w)
    up = make_upstream(w)
    q, k, v, _ = to_device(w, inp, dev)
    dout = torch.from_numpy(up["dout_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
    mspec, sspec = specs(w)
    bm = pbs.flex_blockmask_build(mspec, w.L, w.S, w.q_block, w.kv_block, device=dev)
    bmq = pbs.flex_blockmask_transpose(bm)
    out, lse = pbs.flex_attn_fwd(q, k, v, block_mask=bm, score=sspec, mask=mspec)
    dq, dk, dv = pbs.flex_attn_bwd(q, k, v, out, dout, lse, block_mask=bm, block_mask_q=bmq, score=sspec,
                                   mask=mspec)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    mmod = MaskMod(w.mask)
    smod = ScoreMod(w.score, cap=w.cap, alibi_m=w.alibi_m)
    for b, h in ((0, 0), (3, 15)):
        sl = lambda x: x[b:b + 1, h:h + 1]
        ref = attention_backward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(up["dout"]),
                                 scale=oracle_default_scale(w.D), score=ScoreModAt(smod, h, w.Hq), mask=mmod,
                                 q_offset=w.q_offset)
        got = tuple(x[b:b + 1, h:h + 1] for x in (dq, dk, dv))
        assert_grads_close(got, ref, "bf16", f"full size b={b} h={h}")


class ScoreModAt:
    """A score rule evaluated for query head h of `heads` on a one-head slice."""

    def __init__(self, mod, h, heads):
        self.mod, self.h, self.heads = mod, h, heads
        self.kind, self.cap = mod.kind, mod.cap

    def __call__(self, s, b, h, q_pos, kv, heads):
        return self.mod(s, b, self.h, q_pos, kv, self.heads)


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_bwd_long_columns_split(dev, dtype, D):
    """Columns longer than one workgroup's share: eight query heads per K/V
    head and nine 128-row Q blocks give up to 144 Q-side tiles per 64-key
    column, so the key-major pass splits columns and adds the partial sums
    (every column under the no-op mask, the sink column under the window)."""
    for mask in (dict(mask_kind="noop"), dict(mask_kind="causal_window_sinks", window=100, sinks=4)):
        run_bwd_case(dev, seed=60 + D, dtype=dtype, B=1, Hq=8, Hkv=1, L=1100, S=1100, D=D, qb=128, kb=64,
                     score=dict(kind="softcap", cap=20.0), what=f"split {dtype} D={D} {mask['mask_kind']}", **mask)


@pytest.mark.parametrize("D", [64, 128])
def test_bwd_packed_documents(dev, D):
    """Many short documents whose boundaries fall inside Q blocks and key
    tiles, so the Q-side and KV-side lists rise and fall along the sequence."""
    run_bwd_case(dev, seed=950 + D, dtype="bf16", B=1, Hq=2, Hkv=1, L=1500, S=1500, D=D, qb=128, kb=64,
                 score=dict(kind="none"), mask_kind="doc_causal", q_offset=0, doc_max=300,
                 what=f"packed documents D={D}")


@pytest.mark.parametrize("name,pairs", [("window_sinks_gqa", [(1, 20), (1, 21), (1, 22), (1, 23)]),
                                        ("doc_causal", [(0, 7)])])
def test_bwd_full_size_d128(dev, name, pairs):
    """The head-dim-128 workloads at full size (window + sinks under GQA 4;
    packed documents, 16K tokens), 128x64 tiles as bench.py runs them, checked
    on sampled slices: for GQA every query head of one K/V head, so that K/V
    head's dk, dv are complete."""
    w = WORKLOADS[name]
    inp = make_inputs(w)
    up = make_upstream(w)
    q, k, v, doc_t = to_device(w, inp, dev)
    dout = torch.from_numpy(up["dout_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
    mspec, sspec = specs(w, doc_t)
    bm = pbs.flex_blockmask_build(mspec, w.L, w.S, w.q_block, w.kv_block, device=dev)
    bmq = pbs.flex_blockmask_transpose(bm)
    out, lse = pbs.flex_attn_fwd(q, k, v, block_mask=bm, score=sspec, mask=mspec)
    dq, dk, dv = pbs.flex_attn_bwd(q, k, v, out, dout, lse, block_mask=bm, block_mask_q=bmq, score=sspec,
                                   mask=mspec)
    torch.cuda.synchronize()
    mmod = MaskMod(w.mask, window=w.window, sinks=w.sinks, doc_id=inp["doc_id"])
    smod = ScoreMod(w.score, cap=w.cap, alibi_m=w.alibi_m)
    print(f"[bwd parity] {name}: oracle over {len(pairs)} head(s)", flush=True)
    ref_q, ref_k, ref_v = attention_backward(inp["q"], inp["k"], inp["v"], up["dout"], scale=oracle_default_scale(w.D),
                                             score=smod, mask=mmod, q_offset=w.q_offset, pairs=pairs, row_chunk=512)
    b = pairs[0][0]
    heads = [h for _, h in pairs]
    hk = heads[0] // (w.Hq // w.Hkv)
    got = (dq[b, heads].float().cpu().numpy(), dk[b, hk].float().cpu().numpy(), dv[b, hk].float().cpu().numpy())
    ref = (ref_q[b, heads], ref_k[b, hk], ref_v[b, hk])
    assert_grads_close(got, ref, "bf16", f"full size {name}")
