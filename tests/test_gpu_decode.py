"""GPU parity of the decode extensions: per-batch query offsets and filled
lengths of a cache, paged K/V pools (and a circular buffer expressed as a
page table), through the C ABI against the CPU oracle on the logical K/V."""
import numpy as np
import pytest
import torch

import programmable_block_sparse_amd as pbs
from gpu_common import TOL_LSE, assert_attention_close, assert_block_mask_equal, require_gpu
from oracle import MaskMod, ScoreMod, attention, build_block_mask
from oracle import default_scale as oracle_default_scale
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _t(x, dtype, dev):
    if dtype == "bf16":
        return torch.from_numpy(f32_to_bf16_bits(x).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


def _w(x, dtype):
    return bf16_bits_to_f32(f32_to_bf16_bits(x)) if dtype == "bf16" else x


def _i32(x, dev):
    return torch.tensor(np.asarray(x, dtype=np.int32), device=dev)


def run(dev, *, seed, dtype, B, Hq, Hkv, L, S, D, qb, kb, score, kind, window=0, sinks=0, offs, lens,
        page_size=0, ring_pages=0, clauses=(), with_max=False, what=""):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, L, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    spec = pbs.MaskSpec(kind, window=window, sinks=sinks, q_offset=0, q_offsets=_i32(offs, dev), kv_lens=_i32(lens, dev),
                        clauses=clauses)
    mod = MaskMod(kind, window=window, sinks=sinks, clauses=clauses)
    bm = pbs.flex_blockmask_build(spec, L, S, qb, kb, B=B, device=dev)
    assert_block_mask_equal(bm, build_block_mask(mod, L, S, qb, kb, B=B, q_offset=offs, kv_len=lens))
    sspec, smod = pbs.ScoreSpec(**score), ScoreMod(**score)
    qt = _t(q, dtype, dev)
    if page_size:
        n_log = -(-S // page_size)
        if ring_pages:
            # a rolling buffer: logical page p of every batch in ring slot p mod ring_pages
            n_phys = B * ring_pages
            table = np.array([[b * ring_pages + p % ring_pages for p in range(n_log)] for b in range(B)], np.int32)
        else:
            n_phys = B * n_log + 3
            perm = rng.permutation(n_phys)[:B * n_log]
            table = perm.reshape(B, n_log).astype(np.int32)
        pool_k = np.zeros((n_phys, Hkv, page_size, D), np.float32)
        pool_v = np.zeros_like(pool_k)
        kp = np.zeros((B, Hkv, n_log * page_size, D), np.float32)
        vp = np.zeros_like(kp)
        kp[:, :, :S], vp[:, :, :S] = k, v
        for b in range(B):
            # the pages a cache filled to lens[b] has written, in order (later
            # pages overwrite earlier ones in a ring)
            for p in range(-(-lens[b] // page_size)):
                pool_k[table[b, p]] = kp[b, :, p * page_size:(p + 1) * page_size]
                pool_v[table[b, p]] = vp[b, :, p * page_size:(p + 1) * page_size]
        out, lse, mx = pbs.flex_attn_fwd_paged(qt, _t(pool_k, dtype, dev), _t(pool_v, dtype, dev),
                                               torch.from_numpy(table).to(dev), S=S, block_mask=bm, score=sspec,
                                               mask=spec, return_max_scores=with_max)
    elif with_max:
        out, lse, mx = pbs.flex_attn_fwd_aux(qt, _t(k, dtype, dev), _t(v, dtype, dev), block_mask=bm, score=sspec,
                                             mask=spec)
    else:
        out, lse = pbs.flex_attn_fwd(qt, _t(k, dtype, dev), _t(v, dtype, dev), block_mask=bm, score=sspec, mask=spec)
    torch.cuda.synchronize()
    sc = oracle_default_scale(D)
    out_ref, lse_ref, mx_ref = attention(_w(q, dtype), _w(k, dtype), _w(v, dtype), scale=sc, score=smod, mask=mod,
                                         q_offset=offs, kv_len=lens, with_max=True)
    assert_attention_close(out, lse, out_ref, lse_ref, dtype, what)
    if with_max:
        # the row maximum is a score like lse: same error sources, same bound
        m = mx.cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isneginf(m), np.isneginf(mx_ref)), f"{what}: -inf pattern of max_scores"
        fin = ~np.isneginf(mx_ref)
        merr = np.abs(m[fin] - mx_ref[fin]).max() if fin.any() else 0.0
        print(f"[decode] {what}: max_scores max-abs {merr:.3e}")
        assert merr <= TOL_LSE, f"{what}: max_scores max-abs {merr:.3e}"


def test_per_batch_offsets_and_lengths_prefill(dev):
    for dtype, D in (("bf16", 64), ("bf16", 128), ("f32", 64)):
        run(dev, seed=1, dtype=dtype, B=3, Hq=4, Hkv=2, L=150, S=400, D=D, qb=64, kb=64,
            score=dict(kind="softcap_alibi", cap=20.0), kind="causal", offs=[250, 0, 40], lens=[400, 130, 230],
            what=f"prefill {dtype} D={D}")
    run(dev, seed=2, dtype="bf16", B=2, Hq=2, Hkv=2, L=100, S=300, D=64, qb=128, kb=64, score=dict(kind="none"),
        kind="noop", offs=[0, 0], lens=[300, 77], what="noop lengths")


def test_decode_capacity_example(dev):
    # the decode section's example scaled to one query per batch: capacity
    # 8, filled 6, logical position 5, window 3
    run(dev, seed=3, dtype="bf16", B=2, Hq=4, Hkv=4, L=1, S=8, D=64, qb=16, kb=64, score=dict(kind="none"),
        kind="causal_window_sinks", window=3, offs=[5, 2], lens=[6, 3], what="capacity 8 filled 6")


def test_decode_kernel_per_batch(dev):
    # 16-query verify steps under GQA: the split-KV decode kernel
    run(dev, seed=4, dtype="bf16", B=4, Hq=16, Hkv=4, L=16, S=4096, D=128, qb=16, kb=64,
        score=dict(kind="softcap", cap=50.0), kind="causal", offs=[4080, 1000, 2047, 16], lens=[4096, 1016, 2063, 32],
        what="decode per batch")


@pytest.mark.parametrize("dtype,D,L,page", [("bf16", 128, 16, 64), ("bf16", 64, 200, 128), ("f32", 64, 70, 64)])
def test_paged_cache(dev, dtype, D, L, page):
    run(dev, seed=5 + D + L, dtype=dtype, B=3, Hq=8, Hkv=2, L=L, S=1000, D=D, qb=16 if L == 16 else 64, kb=64,
        score=dict(kind="softcap_alibi", cap=30.0), kind="causal", offs=[1000 - L, 500, 300],
        lens=[1000, 500 + L, 300 + L], page_size=page, what=f"paged {dtype} D={D} L={L} page={page}")


def test_paged_cache_128_row_workgroups(dev):
    """A paged prefill large enough (B*Hq*ceil(L/128) = 768 row blocks) for
    the 128-row workgroups at head dim 64, with per-batch offsets and lengths."""
    run(dev, seed=31, dtype="bf16", B=3, Hq=128, Hkv=32, L=200, S=700, D=64, qb=128, kb=64,
        score=dict(kind="softcap_alibi", cap=30.0), kind="causal", offs=[500, 120, 0], lens=[700, 320, 200],
        page_size=128, what="paged bf16 D=64 128-row workgroups")


def test_per_batch_128_row_workgroups(dev):
    """The contiguous counterpart of the paged case above: per-batch offsets
    and lengths over contiguous caches in 128-row workgroups."""
    run(dev, seed=32, dtype="bf16", B=3, Hq=128, Hkv=32, L=200, S=700, D=64, qb=128, kb=64,
        score=dict(kind="softcap_alibi", cap=30.0), kind="causal", offs=[500, 120, 0], lens=[700, 320, 200],
        what="per-batch bf16 D=64 128-row workgroups")


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_extended_kernels_per_batch(dev, paged, dtype, D):
    """Mask programs and the row maxima with per-batch offsets and lengths,
    contiguous and paged: the extended kernels of both cache layouts."""
    clauses = (("causal", 0),), (("window", 90), ("kv_lt", 8))
    run(dev, seed=40 + D, dtype=dtype, B=3, Hq=4, Hkv=2, L=150, S=520, D=D, qb=64, kb=64,
        score=dict(kind="softcap", cap=20.0), kind="program", clauses=clauses, offs=[370, 0, 60],
        lens=[520, 140, 250], page_size=128 if paged else 0, with_max=True,
        what=f"program per batch {dtype} D={D} paged={paged}")
    # 16-query verify steps under GQA with the row maxima: the extended decode kernel
    run(dev, seed=50 + D, dtype=dtype, B=2, Hq=8, Hkv=2, L=16, S=1200, D=D, qb=16, kb=64,
        score=dict(kind="softcap", cap=50.0), kind="causal", offs=[1184, 400], lens=[1200, 416],
        page_size=64 if paged else 0, with_max=True, what=f"decode max_scores {dtype} D={D} paged={paged}")


def test_circular_buffer(dev):
    # a ring of four 64-key pages per batch; the window keeps every visible key
    # inside the last four pages, whose slots hold the latest writes
    run(dev, seed=9, dtype="bf16", B=2, Hq=8, Hkv=2, L=16, S=1000, D=128, qb=16, kb=64,
        score=dict(kind="softcap", cap=50.0), kind="causal_window_sinks", window=150, sinks=0,
        offs=[984, 700], lens=[1000, 716], page_size=64, ring_pages=4, what="ring of 4 pages")


def test_paged_cache_wide_kv_blocks(dev):
    # 128-key blocks over a 900-key cache of 64-key pages: the last block's
    # second tile starts past the last page (its rows read as zeros)
    run(dev, seed=77, dtype="bf16", B=2, Hq=4, Hkv=2, L=120, S=900, D=64, qb=64, kb=128,
        score=dict(kind="softcap", cap=30.0), kind="causal", offs=[780, 300], lens=[900, 420], page_size=64,
        what="paged kv_block 128")


@pytest.mark.parametrize("paged", [False, True])
def test_unfilled_cache_rows_are_never_read(dev, paged):
    """Cache rows at or past a batch's filled length hold NaN: the forward and
    the backward must give the same bits as with zeros there (those rows load
    as zeros, so no 0 * NaN reaches a product), on the split-KV decode path and
    the prefill path, contiguous and paged."""
    B, Hq, Hkv, S, D, page = 2, 8, 2, 1000, 64, 64
    lens = [700, 333]
    rng = np.random.default_rng(91)
    n_log = -(-S // page)
    table = rng.permutation(B * n_log + 2)[:B * n_log].reshape(B, n_log).astype(np.int32)
    tt = torch.from_numpy(table).to(dev)
    k = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)

    def caches(fill):
        kc, vc = k.copy(), v.copy()
        for b, n in enumerate(lens):
            kc[b, :, n:] = fill
            vc[b, :, n:] = fill
        if not paged:
            return _t(kc, "bf16", dev), _t(vc, "bf16", dev)
        pk = np.full((B * n_log + 2, Hkv, page, D), fill, np.float32)
        pv = np.full_like(pk, fill)
        kp = np.full((B, Hkv, n_log * page, D), fill, np.float32)
        vp = np.full_like(kp, fill)
        kp[:, :, :S], vp[:, :, :S] = kc, vc
        for b in range(B):
            for p in range(n_log):
                pk[table[b, p]] = kp[b, :, p * page:(p + 1) * page]
                pv[table[b, p]] = vp[b, :, p * page:(p + 1) * page]
        return _t(pk, "bf16", dev), _t(pv, "bf16", dev)

    for L, qb in ((16, 16), (130, 64)):
        offs = [n - L for n in lens]
        q = _t(rng.standard_normal((B, Hq, L, D), dtype=np.float32), "bf16", dev)
        do = _t(rng.standard_normal((B, Hq, L, D), dtype=np.float32), "bf16", dev)
        spec = pbs.MaskSpec("causal", q_offset=0, q_offsets=_i32(offs, dev), kv_lens=_i32(lens, dev))
        score = pbs.ScoreSpec(kind="softcap", cap=30.0)
        bm = pbs.flex_blockmask_build(spec, L, S, qb, 64, B=B, device=dev)
        res = []
        for fill in (0.0, np.nan):
            kc, vc = caches(fill)
            if paged:
                out, lse, _ = pbs.flex_attn_fwd_paged(q, kc, vc, tt, S=S, block_mask=bm, score=score, mask=spec)
            else:
                out, lse = pbs.flex_attn_fwd(q, kc, vc, block_mask=bm, score=score, mask=spec)
            grads = ()
            if qb == 64:
                bmq = pbs.flex_blockmask_transpose(bm)
                if paged:
                    grads = pbs.flex_attn_bwd_paged(q, kc, vc, tt, out, do, lse, S=S, block_mask=bm, block_mask_q=bmq,
                                                    score=score, mask=spec)
                else:
                    grads = pbs.flex_attn_bwd(q, kc, vc, out, do, lse, block_mask=bm, block_mask_q=bmq, score=score,
                                              mask=spec)
            torch.cuda.synchronize()
            res.append((out, lse) + tuple(grads))
        for name, a, b in zip(("out", "lse", "dq", "dk", "dv"), res[0], res[1]):
            assert not torch.isnan(b).any(), f"L={L} paged={paged}: NaN in {name}"
            assert torch.equal(a, b), f"L={L} paged={paged}: {name} depends on the unfilled rows"
