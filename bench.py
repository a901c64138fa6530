"""Benchmark of the block-sparse attention forward hot path on one MI355X.

One step = one pass of the hot path over one batch of seeded synthetic input
already resident in HBM: the BlockMask build from the mask_mod, then the fused
forward (QK^T, scale, score_mod, partial-tile mask, online softmax, PV, out and
lse).  The default workload is causal attention with a soft-cap plus ALiBi-
slope score_mod at B=4, H=16, L=S=2048, D=64, bf16, 128x64 tiles.

Throughput is counted over visited-block FLOPs: 4*D per cell of every full or
partial tile (clipped to the sequence bounds), times B*Hq.  The roofline entry
times the forward kernel alone with HIP events on the stream it runs on.  The
CPU baseline times the float64 oracle on a bounded sample of the same workload
and checks the GPU output on those rows.

With --pass bwd a step is one training pass of the attention: BlockMask
build, its Q-side transpose, the forward and the backward (dq, dk, dv).  Its
throughput counts visited-block FLOPs of both directions: 4*D per cell forward
and 10*D per cell backward (dV, dP, dK, dQ and the recomputed scores S: five
products of 2*D each; the query-major pass recomputes S and dP, which is not
counted).  The roofline entry then times the backward call (row pass,
key-major and query-major passes) against its 10*D per cell.

With --paged PAGE_SIZE the K/V caches are first scattered into a pool of
pages in a seeded random order and the forward reads them through the page
table (flex_attn_fwd_paged; with --pass bwd also the backward,
flex_attn_bwd_paged); everything else is the same.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--pass fwd|bwd] [--paged N]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3      # MI355X fp32 matrix
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="causal_softcap_alibi")
    p.add_argument("--pass", dest="direction", choices=("fwd", "bwd"), default="fwd",
                   help="fwd: the forward hot path (default); bwd: forward + backward training pass")
    p.add_argument("--paged", type=int, default=0, metavar="PAGE_SIZE",
                   help="keep K/V in a paged pool of PAGE_SIZE-key pages (seeded random page order) and run the "
                        "paged forward (and, with --pass bwd, the paged backward)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--eager", action="store_true", help="launch from Python each step instead of replaying a HIP graph")
    p.add_argument("--cpu-sample-heads", type=int, default=0, help="0 = automatic (about 10 s of oracle work)")
    p.add_argument("--quick", action="store_true",
                   help="profiling runs: no time-based warm-up and one timing window of --steps calls per unit")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run device-to-device copies of MIB MiB (HBM counter calibration) and exit")
    return p.parse_args()


# Kernel sources whose code the HBM traffic figures under profiles/ were taken
# on; a figure is reported only while these files are unchanged.
KERNEL_SOURCES = ("programmable_block_sparse_amd/csrc/attn_fwd.hip",
                  "programmable_block_sparse_amd/csrc/attn_fwd_impl.hpp",
                  "programmable_block_sparse_amd/csrc/attn_fwd_bf16_d64.hip",
                  "programmable_block_sparse_amd/csrc/attn_fwd_bf16_d128.hip",
                  "programmable_block_sparse_amd/csrc/attn_fwd_f32_d64.hip",
                  "programmable_block_sparse_amd/csrc/attn_fwd_f32_d128.hip",
                  "programmable_block_sparse_amd/csrc/device_common.hpp",
                  "programmable_block_sparse_amd/csrc/internal.hpp")
# the backward kernels include the forward's device code
KERNEL_SOURCES_BWD = KERNEL_SOURCES + ("programmable_block_sparse_amd/csrc/attn_bwd.hip",
                                       "programmable_block_sparse_amd/csrc/attn_bwd_impl.hpp",
                                       "programmable_block_sparse_amd/csrc/attn_bwd_bf16_d64.hip",
                                       "programmable_block_sparse_amd/csrc/attn_bwd_bf16_d128.hip",
                                       "programmable_block_sparse_amd/csrc/attn_bwd_f32_d64.hip",
                                       "programmable_block_sparse_amd/csrc/attn_bwd_f32_d128.hip")


def kernel_source_hash(sources=KERNEL_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, backward=False):
    """HBM bytes per forward launch (per backward call with backward=True)
    from the rocprofv3 FETCH_SIZE / WRITE_SIZE summary of this workload, or
    None when there is none or the kernel sources changed since it was taken."""
    name = f"hbm_traffic_bwd_{workload}.txt" if backward else f"hbm_traffic_{workload}.txt"
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash(KERNEL_SOURCES_BWD if backward else KERNEL_SOURCES):
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(mib):
    """Device-to-device copies of a known size: what FETCH_SIZE and WRITE_SIZE
    read for them scales the counters of the attention kernels to bytes."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for i in range(3):
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"bench: copy {i} of {mib} MiB done", file=sys.stderr, flush=True)
    print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)


def visited_flops_per_head(bm_np, w):
    """4*D * cells of every listed tile (clipped to L, S), per (batch, head) of mask row (0, 0)."""
    total = 0
    nqb = bm_np["kv_num_blocks"].shape[2]
    for qb in range(nqb):
        rows = min(w.q_block, w.L - qb * w.q_block)
        for num, idx in (("kv_num_blocks", "kv_indices"), ("full_kv_num_blocks", "full_kv_indices")):
            n = int(bm_np[num][0, 0, qb])
            for kb in bm_np[idx][0, 0, qb, :n]:
                total += rows * min(w.kv_block, w.S - int(kb) * w.kv_block)
    return 4 * w.D * total


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1"}))
        print("bench.py: multi-GPU runs are not part of this build (one GPU per box); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.direction == "bwd":
        main_bwd(args)
        return

    import torch
    import programmable_block_sparse_amd as pbs
    from workloads import WORKLOADS, make_inputs
    from workloads.torch_io import specs, to_device

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    inp = make_inputs(w)
    q, k, v, doc_t = to_device(w, inp, dev)
    mspec, sspec = specs(w, doc_t)
    print(f"bench: workload {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} L={w.L} S={w.S} D={w.D} {w.dtype} "
          f"mask={w.mask} score={w.score} tiles {w.q_block}x{w.kv_block}", file=sys.stderr, flush=True)

    bm = pbs.flex_blockmask_build(mspec, w.L, w.S, w.q_block, w.kv_block, device=dev)
    torch.cuda.synchronize()
    bm_np = {n: getattr(bm, n).cpu().numpy() for n in
             ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices")}
    flops = visited_flops_per_head(bm_np, w) * w.B * w.Hq
    elem = 2 if w.dtype == "bf16" else 4
    alg_bytes = (w.B * w.Hq * w.L * w.D + 2 * w.B * w.Hkv * w.S * w.D + w.B * w.Hq * w.L * w.D) * elem \
        + w.B * w.Hq * w.L * 4
    out = torch.empty((w.B, w.Hq, w.L, w.D), dtype=q.dtype, device=dev)
    lse = torch.empty((w.B, w.Hq, w.L), dtype=torch.float32, device=dev)
    ws_bytes = pbs.flex_attn_fwd_workspace_bytes(q.dtype, w.B, w.Hq, w.Hkv, w.L, w.S, w.D, bm)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    bm_step = pbs.flex_blockmask_build(mspec, w.L, w.S, w.q_block, w.kv_block, device=dev)

    def attend(block_mask):
        pbs.flex_attn_fwd(q, k, v, block_mask=block_mask, score=sspec, mask=mspec, out=out, lse=lse, workspace=ws)

    if args.paged:
        k_pool, v_pool, table = paged_pools(w, k, v, args.paged, dev)
        del k, v

        def attend(block_mask):
            pbs.flex_attn_fwd_paged(q, k_pool, v_pool, table, S=w.S, block_mask=block_mask, score=sspec, mask=mspec,
                                    out=out, lse=lse, workspace=ws)

    def fwd():
        attend(bm)

    def build_only():
        pbs.flex_blockmask_build(mspec, w.L, w.S, w.q_block, w.kv_block, out=bm_step)

    def step():
        build_only()
        attend(bm_step)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"bench: warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)
    runners = {"step": step, "fwd": fwd, "mask": build_only}
    mode = "eager"
    if not args.eager:
        runners = graph_runners(runners, dev, ([out, lse], step))
        mode = "hip_graph"
    tm = time_units(runners, args, dev, **QUICK) if args.quick else time_units(runners, args, dev)
    ms_step, ms_fwd, ms_mask = tm["ms_per_step"], tm["fwd"]["median_ms"], tm["mask"]["median_ms"]
    print(f"bench: step {ms_step * 1e3:.1f} us ({args.steps} steps; windows median "
          f"{tm['step']['median_ms'] * 1e3:.1f} us), fwd {ms_fwd * 1e3:.1f} us "
          f"[{tm['fwd']['min_ms'] * 1e3:.1f}, {tm['fwd']['max_ms'] * 1e3:.1f}], "
          f"block mask {ms_mask * 1e3:.1f} us ({mode}, {tm['calls_per_window']} calls per window, "
          f"{tm['windows']} windows)", file=sys.stderr, flush=True)

    # a step holds the forward plus the BlockMask build, so it cannot be faster
    tm["step_ge_fwd"] = bool(tm["step"]["median_ms"] >= ms_fwd)
    if not tm["step_ge_fwd"]:
        print(f"bench: WARNING step median {tm['step']['median_ms'] * 1e3:.1f} us below fwd median "
              f"{ms_fwd * 1e3:.1f} us: timing unreliable on this run", file=sys.stderr, flush=True)
    value = flops / (ms_step * 1e-3) / 1e12
    fwd_tflops = flops / (ms_fwd * 1e-3) / 1e12
    if w.name == "decode_verify":
        roof = {"bound": "hbm", "achieved": alg_bytes / (ms_fwd * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
        roof = {"bound": "mfma", "achieved": fwd_tflops, "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(w.name)
    roof["kernel"] = "attn_fwd_decode + attn_fwd_combine" if ws_bytes else "attn_fwd_prefill"
    if args.paged:
        roof["traffic"] = None          # counters are taken on the contiguous layout
    roof["algorithmic_per_launch"] = flops if roof["unit"] == "TFLOP/s" else alg_bytes

    result = {
        "metric": "flex fwd TFLOP/s (visited-block FLOPs) and % of MI355X bf16 MFMA peak",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded N(0,1) inputs, PCG64 seed %d)" % w.seed,
        "config": {"workload": w.name + (f"_paged{args.paged}" if args.paged else ""), "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "L": w.L, "S": w.S, "D": w.D,
                   "mask": w.mask, "score": w.score, "cap": w.cap, "window": w.window, "sinks": w.sinks,
                   "q_block": w.q_block, "kv_block": w.kv_block, "q_offset": w.q_offset,
                   "doc_lengths": inp["doc_lengths"], "page_size": args.paged or None},
        "roofline": roof,
        "fwd_ms": ms_fwd, "blockmask_ms": ms_mask, "launch_mode": mode, "timing": tm,
        "fwd_tflops_visited": fwd_tflops, "pct_bf16_peak_fwd": 100.0 * fwd_tflops / BF16_PEAK_TFLOPS,
        "visited_block_flops": flops, "algorithmic_bytes": alg_bytes,
        "hbm_gbs_fwd": alg_bytes / (ms_fwd * 1e-3) / 1e9,
    }
    if not args.no_cpu_baseline and not args.paged:
        result.update(cpu_baseline(args, w, inp, out, lse, flops))
    print(json.dumps(result), flush=True)


# Calls of one unit captured back to back in one HIP graph: a replay then
# costs one graph launch per GRAPH_CALLS calls, so the launch overhead of a
# replay (about 10 us on this stack, as long as a BlockMask build) does not
# count as kernel time.
GRAPH_CALLS = 10


class GraphUnit:
    """A unit of work replayed from HIP graphs: ``run(n)`` enqueues n calls
    (n // GRAPH_CALLS replays of the multi-call graph, then single-call ones)."""

    def __init__(self, g1, gn):
        self.g1, self.gn = g1, gn

    def run(self, n):
        for _ in range(n // GRAPH_CALLS):
            self.gn.replay()
        for _ in range(n % GRAPH_CALLS):
            self.g1.replay()


class EagerUnit:
    def __init__(self, fn):
        self.fn = fn

    def run(self, n):
        for _ in range(n):
            self.fn()


def graph_runners(runners, dev, check):
    """Capture each runner in HIP graphs of one call and of GRAPH_CALLS calls
    (on a side stream) and check three replays of ``check``'s one-call graph,
    then three of its multi-call graph, against the eager result, with eager
    work between them.  Returns name -> GraphUnit."""
    import torch
    graphs = {}
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for name, fn in runners.items():
            pair = []
            for calls in (1, GRAPH_CALLS):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    for _ in range(calls):
                        fn()
                pair.append(g)
            graphs[name] = GraphUnit(*pair)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    bufs, eager = check
    ref = [b.clone() for b in bufs]
    first = graphs[next(iter(graphs))]
    for i, g in enumerate([first.g1] * 3 + [first.gn] * 3):
        for b in bufs:
            b.zero_()
        g.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(b, r) for b, r in zip(bufs, ref)):
            raise RuntimeError(f"graph replay {i} differs from the eager result")
        eager()
        torch.cuda.synchronize()
    return graphs


# --quick: for runs under a profiler, where every call is recorded
QUICK = {"windows": 1, "min_calls": 1, "warm_ms": 0.0}


def time_units(units, args, dev, windows=5, min_calls=50, warm_ms=100.0):
    """Time every unit on the stream its kernels run on (HIP events).

    First the step unit runs until at least ``warm_ms`` of GPU time has passed
    (clocks and caches settle).  Then ``ms_per_step`` is the time of exactly
    ``args.steps`` steps, and each unit is timed in ``windows`` interleaved
    windows of max(min_calls, args.steps) calls: median, min and max per call.
    Units are GraphUnit or EagerUnit (name -> unit); plain callables are
    wrapped as eager units."""
    import torch
    units = {n: (u if hasattr(u, "run") else EagerUnit(u)) for n, u in units.items()}
    stream = torch.cuda.current_stream(dev)

    def window(unit, n):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        unit.run(n)
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end)

    warm, warm_calls = 0.0, 0
    while warm_calls == 0 or warm < warm_ms:
        warm += window(units["step"], 20)
        warm_calls += 20
    ms_per_step = window(units["step"], args.steps) / args.steps
    n = max(min_calls, args.steps)
    per = {name: [] for name in units}
    for _ in range(windows):
        for name, unit in units.items():
            per[name].append(window(unit, n) / n)
    out = {"ms_per_step": ms_per_step, "warmup_ms": warm, "warmup_calls": warm_calls, "windows": windows,
           "calls_per_window": n, "graph_calls": GRAPH_CALLS}
    for name, xs in per.items():
        out[name] = {"median_ms": float(np.median(xs)), "min_ms": float(min(xs)), "max_ms": float(max(xs))}
    return out


def paged_pools(w, k, v, ps, dev):
    """K/V scattered into pools of ps-key pages in a seeded random page order:
    logical page p of batch b sits in pool page table[b, p].  Returns the two
    pools and the int32 page table."""
    import torch
    n_log = -(-w.S // ps)
    perm = torch.from_numpy(np.random.Generator(np.random.PCG64(w.seed + 77)).permutation(w.B * n_log)
                            .astype(np.int64)).to(dev)
    table = perm.view(w.B, n_log).to(torch.int32).contiguous()

    def to_pool(x):
        xp = torch.zeros((w.B, w.Hkv, n_log * ps, w.D), dtype=x.dtype, device=dev)
        xp[:, :, :w.S] = x
        pages = xp.view(w.B, w.Hkv, n_log, ps, w.D).permute(0, 2, 1, 3, 4).reshape(w.B * n_log, w.Hkv, ps, w.D)
        pool = torch.empty_like(pages)
        pool[perm] = pages
        return pool
    pools = to_pool(k), to_pool(v)
    torch.cuda.synchronize()
    print(f"bench: paged K/V, {w.B * n_log} pages of {ps} keys", file=sys.stderr, flush=True)
    return pools[0], pools[1], table


def bwd_kernel_names(w) -> str:
    """Kernels of one backward call: the two major passes share one launch
    under GQA at head dim 128 (bf16, element-rule masks); long Q-side columns
    add the split-sum kernel."""
    fused = w.dtype == "bf16" and w.D == 128 and w.Hq > w.Hkv and w.mask != "program"
    names = "attn_bwd_rows + " + ("attn_bwd_fused" if fused else "attn_bwd_dkdv + attn_bwd_dq")
    group, n_qb = w.Hq // w.Hkv, -(-w.L // w.q_block)
    if group * n_qb * (w.q_block // 64) > 128:
        names += " + attn_bwd_dkdv_reduce"
    return names


def main_bwd(args):
    import torch
    import programmable_block_sparse_amd as pbs
    from workloads import WORKLOADS, make_inputs, make_upstream
    from workloads.torch_io import specs, to_device

    w = WORKLOADS[args.workload]
    if w.q_block not in (64, 128):
        print(json.dumps({"error": f"the backward pass needs 64- or 128-row Q blocks ({w.name} has {w.q_block})"}))
        sys.exit(2)
    dev = torch.device("cuda:0")
    inp = make_inputs(w)
    up = make_upstream(w)
    q, k, v, doc_t = to_device(w, inp, dev)
    if w.dtype == "bf16":
        dout = torch.from_numpy(up["dout_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        dout = torch.from_numpy(up["dout"]).to(dev)
    mspec, sspec = specs(w, doc_t)
    print(f"bench: backward, workload {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} L={w.L} S={w.S} D={w.D} {w.dtype} "
          f"mask={w.mask} score={w.score} tiles {w.q_block}x{w.kv_block}", file=sys.stderr, flush=True)
    bm = pbs.flex_blockmask_build(mspec, w.L, w.S, w.q_block, w.kv_block, device=dev)
    bmq = pbs.flex_blockmask_transpose(bm)
    torch.cuda.synchronize()
    bm_np = {n: getattr(bm, n).cpu().numpy() for n in
             ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices")}
    fwd_flops = visited_flops_per_head(bm_np, w) * w.B * w.Hq        # 4*D per visited cell
    bwd_flops = fwd_flops * 10 // 4                                    # 10*D per visited cell
    out = torch.empty((w.B, w.Hq, w.L, w.D), dtype=q.dtype, device=dev)
    lse = torch.empty((w.B, w.Hq, w.L), dtype=torch.float32, device=dev)
    dq = torch.empty_like(out)
    dk = torch.empty((w.B, w.Hkv, w.S, w.D), dtype=q.dtype, device=dev)
    dv = torch.empty_like(dk)
    ws_f = torch.empty(max(pbs.flex_attn_fwd_workspace_bytes(q.dtype, w.B, w.Hq, w.Hkv, w.L, w.S, w.D, bm), 1),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(pbs.flex_attn_bwd_workspace_bytes(q.dtype, w.B, w.Hq, w.Hkv, w.L, w.S, w.D, bm),
                       dtype=torch.uint8, device=dev)
    bm_step = pbs.flex_blockmask_build(mspec, w.L, w.S, w.q_block, w.kv_block, device=dev)
    bmq_step = pbs.flex_blockmask_transpose(bm_step)

    def fwd_call(block_mask):
        pbs.flex_attn_fwd(q, k, v, block_mask=block_mask, score=sspec, mask=mspec, out=out, lse=lse, workspace=ws_f)

    def bwd_call(block_mask, block_mask_q):
        pbs.flex_attn_bwd(q, k, v, out, dout, lse, block_mask=block_mask, block_mask_q=block_mask_q, score=sspec,
                          mask=mspec, dq=dq, dk=dk, dv=dv, workspace=ws_b)

    if args.paged:
        k_pool, v_pool, table = paged_pools(w, k, v, args.paged, dev)
        del k, v

        def fwd_call(block_mask):
            pbs.flex_attn_fwd_paged(q, k_pool, v_pool, table, S=w.S, block_mask=block_mask, score=sspec, mask=mspec,
                                    out=out, lse=lse, workspace=ws_f)

        def bwd_call(block_mask, block_mask_q):
            pbs.flex_attn_bwd_paged(q, k_pool, v_pool, table, out, dout, lse, S=w.S, block_mask=block_mask,
                                    block_mask_q=block_mask_q, score=sspec, mask=mspec, dq=dq, dk=dk, dv=dv,
                                    workspace=ws_b)

    def bwd():
        bwd_call(bm, bmq)

    def step():
        pbs.flex_blockmask_build(mspec, w.L, w.S, w.q_block, w.kv_block, out=bm_step)
        pbs.flex_blockmask_transpose(bm_step, out=bmq_step)
        fwd_call(bm_step)
        bwd_call(bm_step, bmq_step)

    def transpose_only():
        pbs.flex_blockmask_transpose(bm_step, out=bmq_step)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"bench: warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)
    runners = {"step": step, "bwd": bwd, "transpose": transpose_only}
    mode = "eager"
    if not args.eager:
        runners = graph_runners(runners, dev, ([out, lse, dq, dk, dv], step))
        mode = "hip_graph"
    tm = time_units(runners, args, dev, **QUICK) if args.quick else time_units(runners, args, dev)
    ms_step, ms_bwd, ms_tr = tm["ms_per_step"], tm["bwd"]["median_ms"], tm["transpose"]["median_ms"]
    print(f"bench: step {ms_step * 1e3:.1f} us, bwd {ms_bwd * 1e3:.1f} us "
          f"[{tm['bwd']['min_ms'] * 1e3:.1f}, {tm['bwd']['max_ms'] * 1e3:.1f}], transpose {ms_tr * 1e3:.1f} us "
          f"({mode})", file=sys.stderr, flush=True)
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
    bwd_tflops = bwd_flops / (ms_bwd * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": bwd_tflops, "peak": peak, "unit": "TFLOP/s", "frac": bwd_tflops / peak,
            "traffic": None if args.paged else measured_traffic(w.name, backward=True), "kernel": bwd_kernel_names(w),
            "algorithmic_per_launch": bwd_flops}
    result = {
        "metric": "flex fwd+bwd TFLOP/s (visited-block FLOPs: 4*D fwd + 10*D bwd per cell)",
        "value": (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs and upstream gradient, PCG64 seed %d)" % w.seed,
        "config": {"workload": w.name + "_train" + (f"_paged{args.paged}" if args.paged else ""), "B": w.B,
                   "Hq": w.Hq, "Hkv": w.Hkv, "L": w.L, "S": w.S, "D": w.D, "mask": w.mask, "score": w.score,
                   "cap": w.cap, "window": w.window, "sinks": w.sinks, "q_block": w.q_block,
                   "kv_block": w.kv_block, "q_offset": w.q_offset, "page_size": args.paged or None},
        "roofline": roof, "bwd_ms": ms_bwd, "transpose_ms": ms_tr, "launch_mode": mode, "timing": tm,
        "bwd_tflops_visited": bwd_tflops, "fwd_visited_flops": fwd_flops, "bwd_visited_flops": bwd_flops,
    }
    if not args.no_cpu_baseline and not args.paged:
        result.update(cpu_baseline_bwd(args, w, inp, up, (dq, dk, dv), bwd_flops))
    print(json.dumps(result), flush=True)


def cpu_baseline_bwd(args, w, inp, up, grads, flops):
    """Time the float64 backward oracle on (batch, head) slices of the workload
    (about 10 s) and compare the GPU gradients of those slices."""
    from oracle import MaskMod, ScoreMod, attention_backward
    from oracle import default_scale as oracle_default_scale

    cores, cpu_model, blas_threads = host_info()
    mmod = MaskMod(w.mask, window=w.window, sinks=w.sinks, doc_id=inp["doc_id"], clauses=w.clauses)
    smod = ScoreMod(w.score, cap=w.cap, alibi_m=w.alibi_m)
    pairs = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    sample, t_total, refs = [], 0.0, {}
    for (b, h) in pairs:
        t0 = time.perf_counter()
        refs[(b, h)] = attention_backward(inp["q"], inp["k"], inp["v"], up["dout"], scale=oracle_default_scale(w.D),
                                          score=smod, mask=mmod, q_offset=w.q_offset, pairs=[(b, h)])
        t_total += time.perf_counter() - t0
        sample.append((b, h))
        if (args.cpu_sample_heads and len(sample) >= args.cpu_sample_heads) or \
                (not args.cpu_sample_heads and t_total >= 10.0):
            break
    dq = grads[0].float().cpu().numpy()
    # dq of a sampled head is complete; dk, dv of a K/V head need all its query heads
    err_dq = max(float(np.abs(dq[b, h] - refs[(b, h)][0][b, h]).max()) for (b, h) in sample)
    dense_per_head = 12 * w.D * w.L * w.S      # S, O = PV, dP, dV, dK, dQ over every (row, key) pair
    return {
        "cpu_baseline": {"value": dense_per_head * len(sample) / t_total / 1e12, "unit": "TFLOP/s",
                         "cores": blas_threads or cores, "kind": "oracle",
                         "flops_counted": "dense: 12*D*L*S per (batch, head) slice, as the oracle computes",
                         "sample": f"{len(sample)} of {w.B * w.Hq} (batch, head) slices, all rows; float64 dense "
                                   f"backward oracle, {t_total:.1f} s; host cores {cores}, BLAS threads "
                                   f"{blas_threads}, CPU {cpu_model}",
                         "host_cores": cores, "blas_threads": blas_threads, "cpu_model": cpu_model},
        "parity_on_bench_buffers": {"dq_max_abs": err_dq, "heads_checked": len(sample)},
    }


def host_info():
    """Cores this process may run on, the CPU model and the BLAS thread count."""
    cores = len(os.sched_getaffinity(0))
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas = None
    return cores, model, blas


def cpu_baseline(args, w, inp, out, lse, flops):
    """Time the float64 oracle on whole (batch, head) slices of the workload and
    compare the GPU output on those rows.  The oracle forms every score of a
    row (dense), so its rate is counted on the dense FLOPs it performs:
    4*D*L*S per (batch, head) slice (QK^T and PV)."""
    from oracle import MaskMod, ScoreMod, attention, build_block_mask
    from oracle import default_scale as oracle_default_scale

    cores, cpu_model, blas_threads = host_info()
    mmod = MaskMod(w.mask, window=w.window, sinks=w.sinks, doc_id=inp["doc_id"], clauses=w.clauses)
    smod = ScoreMod(w.score, cap=w.cap, alibi_m=w.alibi_m)
    t0 = time.perf_counter()
    ref_bm = build_block_mask(mmod, w.L, w.S, w.q_block, w.kv_block, q_offset=w.q_offset)
    visible = int(ref_bm["counts"].sum())
    t_bm = time.perf_counter() - t0
    heads_total = w.B * w.Hq
    dense_per_head = 4 * w.D * w.L * w.S
    # about 10 s of work: calibrate on one head, then run the rest of the sample;
    # the last batch's last head is always in the sample
    pairs = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    t0 = time.perf_counter()
    o1, l1 = attention(inp["q"], inp["k"], inp["v"], scale=oracle_default_scale(w.D), score=smod, mask=mmod,
                       q_offset=w.q_offset, heads=[0], batches=[0])
    t_one = time.perf_counter() - t0
    n = args.cpu_sample_heads or int(max(2, min(len(pairs), 10.0 // max(t_one, 1e-3))))
    sample = pairs[:max(1, n - 1)]
    if pairs[-1] not in sample:
        sample.append(pairs[-1])
    outs = {(0, 0): (o1, l1)}
    t0 = time.perf_counter()
    for (b, h) in sample[1:]:
        outs[(b, h)] = attention(inp["q"], inp["k"], inp["v"], scale=oracle_default_scale(w.D), score=smod,
                                 mask=mmod, q_offset=w.q_offset, heads=[h], batches=[b])
    t_rest = time.perf_counter() - t0
    t_total = t_one + t_rest
    out_np = out.float().cpu().numpy()
    lse_np = lse.cpu().numpy()
    err_o = max(float(np.abs(out_np[b, h] - outs[(b, h)][0][0, 0]).max()) for (b, h) in sample)
    fin = [np.isfinite(outs[(b, h)][1][0, 0]) for (b, h) in sample]
    err_l = max(float(np.abs(lse_np[b, h][f] - outs[(b, h)][1][0, 0][f]).max()) if f.any() else 0.0
                for (b, h), f in zip(sample, fin))
    inf_ok = all(np.array_equal(np.isneginf(lse_np[b, h]), ~f) for (b, h), f in zip(sample, fin))
    tol_out = 2e-2 if w.dtype == "bf16" else 1e-5
    within = bool(err_o <= tol_out and err_l <= 1e-3 and inf_ok)
    if not within:
        print(f"bench: PARITY FAILURE on the bench buffers: out {err_o:.3e} (tol {tol_out}), lse {err_l:.3e} "
              f"(tol 1e-3), -inf pattern {'ok' if inf_ok else 'differs'}", file=sys.stderr, flush=True)
    return {
        "cpu_baseline": {"value": dense_per_head * len(sample) / t_total / 1e12, "unit": "TFLOP/s",
                         "cores": blas_threads or cores, "kind": "oracle",
                         "flops_counted": "dense: 4*D*L*S per (batch, head) slice, as the oracle computes",
                         "sample": f"{len(sample)} of {heads_total} (batch, head) slices, all {w.L} rows each; "
                                   f"float64 dense oracle, {t_total:.1f} s; host cores {cores}, "
                                   f"BLAS threads {blas_threads}, CPU {cpu_model}",
                         "host_cores": cores, "blas_threads": blas_threads, "cpu_model": cpu_model,
                         "seconds": t_total},
        "cpu_blockmask_oracle_s": t_bm,
        "visible_element_flops": 4 * w.D * visible * w.B * w.Hq,
        "parity_on_bench_buffers": {"out_max_abs": err_o, "lse_max_abs": err_l, "neg_inf_pattern_equal": inf_ok,
                                    "rows_checked": len(sample) * w.L, "slices_checked": len(sample),
                                    "last_slice": list(sample[-1]),
                                    "tolerance": {"out": tol_out, "lse": 1e-3}, "within_tolerance": within},
    }


if __name__ == "__main__":
    main()
