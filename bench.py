#!/usr/bin/env python3
"""Benchmark of one tree-verify MLA attention step on one MI355X.

A step is one verify call (verify_attn_run + verify_attn_reduce) over the
long-prefix tensor-parallel-rank workload: 1 request, H=8 heads, T=16 draft
nodes in a random tree, prefix L=65536, a 262144-slot bf16 pool whose slot
table is half contiguous runs (length 1..64) and half scattered slots.

Timing: the steps are captured in a HIP graph and replayed on the current
stream between two HIP events.  Each step reads a different copy of the pool
(8 copies, 2.4 GB), so consecutive calls do not hit the 256 MB Infinity
Cache with the previous call's 75.5 MB of KV rows; a warm variant (one pool)
is reported beside it.  The partial-pass kernel is also timed alone (a graph
of run-only launches) for the roofline line.

Metric: effective KV GB/s = (L + T) * 1152 bytes (each 576-wide bf16 latent
row read once per call, shared by every head) / time per call.

CPU baseline: the fp64 oracle (tests' reference) on the same workload, on
the host cores, full verify calls repeated for a bounded ~10-30 s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_DENSE_PEAK_TFLOPS = 2500.0
WORKLOAD = 3                   # 1 request, H=8, T=16, L=65536
N_POOLS = 8


# The partial pass counts as held back by HBM only when the same launches
# with the pool resident in the 256 MB Infinity Cache (warm) run clearly
# faster than with the pool rotated out of it (cold).
HBM_LIMITED_WARM_RATIO = 0.9


def roofline_bound(flops, nbytes):
    """Which roofline bounds a kernel of this arithmetic intensity: below
    the ridge (peak flops / peak bytes per second) the HBM one."""
    ridge = BF16_DENSE_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    return "hbm" if flops / nbytes < ridge else "mfma"


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


KERNEL_SRC = os.path.join(ROOT, "speculative_tree_verify_mla_amd", "csrc", "verify_attn.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_va_partial_kernel_tp_rank_h8_t16_l65536.txt")


def kernel_source_hash():
    """SHA-256 of the kernel source's code: line comments, trailing blanks and
    empty lines removed, so a comment edit keeps a measurement valid while
    any code change voids it (the source has no block comments and no "//"
    inside string literals)."""
    with open(KERNEL_SRC, encoding="utf-8") as f:
        lines = [ln.split("//", 1)[0].rstrip() for ln in f]
    return hashlib.sha256("\n".join(ln for ln in lines if ln).encode()).hexdigest()


def traffic_from_profile():
    """HBM bytes per partial-kernel launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy calibration), or None
    when there is no summary or it was taken on another version of the kernel
    source."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    sha = re.search(r"^kernel_source_sha256:\s*([0-9a-f]{64})", text, re.M)
    val = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not sha or not val or sha.group(1) != kernel_source_hash():
        return None
    return float(val.group(1))


def capture_timer(torch, stream):
    """Returns time_graph(fn, n): ms per call of fn(i), i < n, captured in one
    HIP graph and replayed between two events on `stream`."""
    def time_graph(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for i in range(n):
                    fn(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n
    return time_graph


def capture_timer_interleaved(torch, stream):
    """Returns time_graphs(fns, n, rounds): for each fn, the median over
    `rounds` of ms per call of fn(i), i < n, each fn captured in its own HIP
    graph; the graphs' timed replays alternate round by round, so a clock
    that drifts under sustained load affects every fn alike."""
    def time_graphs(fns, n, rounds):
        graphs = []
        for fn in fns:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                with torch.cuda.graph(g, stream=stream):
                    for i in range(n):
                        fn(i)
            torch.cuda.synchronize()
            g.replay()
            graphs.append(g)
        torch.cuda.synchronize()
        times = [[] for _ in fns]
        for r in range(rounds):
            order = range(len(fns)) if r % 2 == 0 else reversed(range(len(fns)))
            for k in order:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                with torch.cuda.stream(stream):
                    e0.record(stream)
                    graphs[k].replay()
                    e1.record(stream)
                torch.cuda.synchronize()
                times[k].append(e0.elapsed_time(e1) / n)
        return [float(np.median(t)) for t in times]
    return time_graphs


def measure_defrag(torch, va, wl, pools, table, indptr, prefix, parent, q, H, K, stream,
                   time_graph):
    """Tier 1 defrag on the bench request: the compaction kernel's time, and
    verify on the fragmented table against the compacted one.  Each pool copy
    gets a free run of n slots appended; the compacted rows land there."""
    n = int(table.numel())
    base = pools[0].shape[0]
    ext = [torch.cat([p, torch.zeros((n, p.shape[1]), dtype=p.dtype, device=p.device)])
           for p in pools]
    frag = table.clone()
    work = table.clone()
    lib = va.load_library()
    ws = torch.empty(int(lib.verify_attn_compact_workspace_bytes(n, n)), dtype=torch.uint8,
                     device=table.device)
    copied = torch.empty(1, dtype=torch.int32, device=table.device)

    def restore(i):
        work.copy_(frag)

    def restore_and_compact(i):
        work.copy_(frag)
        va.verify_attn_compact(ext[i % len(ext)], work, base, n, workspace=ws, copied=copied,
                               stream=stream)

    reps = max(8, min(K, 64))
    ms_restore = time_graph(restore, reps)
    ms_compact = time_graph(restore_and_compact, reps) - ms_restore
    assert int(copied.item()) == n
    compacted = work.clone()                      # base .. base + n - 1
    with torch.cuda.stream(stream):               # every pool copy holds the compacted rows
        for p in ext:
            work.copy_(frag)
            va.verify_attn_compact(p, work, base, n, workspace=ws, copied=copied, stream=stream)
    torch.cuda.synchronize()
    plan = va.verify_attn_plan(H, wl.prefix_len, wl.num_tree)
    vws = va.workspace_for(plan, table.device)
    out = torch.empty((int(plan.total_tree), H, 512), dtype=torch.bfloat16, device=table.device)
    lse = torch.empty((int(plan.total_tree), H), dtype=torch.float32, device=table.device)

    def verify_with(tab):
        def fn(i):
            va.verify_attn_run(plan, q, ext[i % len(ext)], tab, indptr, prefix, parent,
                               wl.sm_scale, vws, stream)
            va.verify_attn_reduce(plan, vws, out, lse, stream)
        return fn

    ms_frag = time_graph(verify_with(frag), K)
    o_frag = out.clone()
    ms_comp = time_graph(verify_with(compacted), K)
    same = bool(torch.equal(o_frag.view(torch.int16), out.view(torch.int16)))
    kv_bytes = wl.kv_bytes()

    def runs(t):   # maximal runs of consecutive slots
        t = t.cpu().numpy().astype(np.int64)
        return 1 + int(np.count_nonzero(t[1:] != t[:-1] + 1)) if len(t) else 0

    return {
        "policy": "rows moved to a reserved free run in logical order, budget = all rows",
        "rows": n,
        "runs_before": runs(frag),
        "runs_after": runs(compacted),
        "compact_us": round(ms_compact * 1e3, 3),
        "compact_copy_gbs": round(2 * n * 1152 / (ms_compact * 1e-3) / 1e9, 1),
        "verify_fragmented_us": round(ms_frag * 1e3, 3),
        "verify_compacted_us": round(ms_comp * 1e3, 3),
        "verify_fragmented_gbs": round(kv_bytes / (ms_frag * 1e-3) / 1e9, 2),
        "verify_compacted_gbs": round(kv_bytes / (ms_comp * 1e-3) / 1e9, 2),
        "outputs_bitwise_equal": same,
    }


def measure_marshal(torch, va, inputs, dev, time_graph):
    """Device draft-tree marshaling (verify order, parent array, ancestor
    masks, draft slot entries) for the bench request's shape and for a batch
    of four 64-node trees; also with the queries gathered into verify order,
    as two launches and as one."""
    res = {}
    for name, num_tree, prefix in (("1x16", [16], [65536]), ("4x64", [64] * 4, [4096] * 4)):
        wl = inputs.make_workload("marshal", 8, num_tree, prefix, 1 << 18, seed=7,
                                  table="interleaved" if len(num_tree) > 1 else "scattered")
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        plan = va.verify_attn_plan(8, wl.prefix_len, wl.num_tree)
        rp, rs = t(wl.parent), t(wl.slot_table[:int(plan.total_tree)])
        pre, ind, tab = t(wl.prefix_len), t(wl.slot_indptr), t(wl.slot_table)
        ms = time_graph(lambda i: va.verify_attn_build_tree(plan, rp, rs, pre, ind, tab), 200)
        res[f"us_{name}"] = round(ms * 1e3, 3)
        # with the queries gathered into verify order by the library as well
        q_raw = torch.zeros((int(plan.total_tree), 8, 576), dtype=torch.bfloat16, device=dev)
        q_v = torch.empty_like(q_raw)

        def marshal_q(i):
            perm = va.verify_attn_build_tree(plan, rp, rs, pre, ind, tab)[0]
            va.verify_attn_permute_rows(plan, perm, q_raw, q_v)

        ms = time_graph(marshal_q, 200)
        res[f"us_{name}_with_q"] = round(ms * 1e3, 3)
        # the same in one launch
        ms = time_graph(lambda i: va.verify_attn_build_tree_rows(plan, rp, rs, pre, ind, tab,
                                                                 q_raw, q_v), 200)
        res[f"us_{name}_with_q_one_launch"] = round(ms * 1e3, 3)
    res["pages_host_tree_and_mask_ms"] = 1.98
    return res


def measure_restart(torch, va, inputs, wl, pool, table, indptr, prefix, parent, H, stream,
                    time_graph, us_plain_warm):
    """The fixed-reference softmax's slow path at the bench shape.  The rope
    columns of tile j (0..7) of every 512-key split get j*c added, with q =
    0.5 + 0.1 N(0, 1) so that every row's score climbs by about 24 log2 units
    per 64-key tile.  Tile 3 of each split then beats the split's first-tile
    reference by more than the 64-unit slack: every work item stops its first
    pass, sweeps its split for the exact row maxima, and computes the split
    again, the three-pass worst case.  One pool copy (warm), against the warm
    plain call."""
    import math
    dev = pool.device
    T = int(wl.num_tree.sum())
    L = int(wl.prefix_len[0])
    rng = np.random.default_rng(5)
    q_r = torch.from_numpy(inputs.bf16_bits(
        (0.5 + 0.1 * rng.standard_normal((T, H, 576))).astype(np.float32)).view(np.int16)).to(dev)
    q_r = q_r.view(torch.bfloat16)
    step_log2 = 24.0
    c = step_log2 / (0.5 * 64 * wl.sm_scale / math.log(2.0))
    rows = table[:L].long()
    k = torch.arange(L, device=dev)
    bump = (c * ((k // 64) % 8).float()).unsqueeze(1)
    pool_r = pool.clone()
    pool_r[rows, 512:] = (pool_r[rows, 512:].float() + bump).to(torch.bfloat16)
    plan = va.verify_attn_plan(H, wl.prefix_len, wl.num_tree)
    ws = va.workspace_for(plan, dev)
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)

    def step(i):
        va.verify_attn_run(plan, q_r, pool_r, table, indptr, prefix, parent, wl.sm_scale, ws, stream)
        va.verify_attn_reduce(plan, ws, out, lse, stream)

    with torch.cuda.stream(stream):
        step(0)
    torch.cuda.synchronize()
    status = va.verify_attn_read_status(plan, ws, stream)
    finite = bool(torch.isfinite(out.float()).all() and torch.isfinite(lse).all())
    ms = time_graph(step, 50)
    return {"workload": "the bench shape, scores rising ~24 log2 units per tile within every split",
            "passes": 3, "us_per_call": round(ms * 1e3, 3),
            "vs_plain_warm": round(ms * 1e3 / us_plain_warm, 3),
            "status": int(status), "finite": finite}


def measure_config(torch, va, inputs, dev, stream, idx, n_pools, steps):
    """One of the other workloads (full head count, ragged batch): µs per call
    from a HIP graph of `steps` calls rotating over `n_pools` pool copies (the
    median of 5 rounds, alternating with the partial-only graph), effective KV
    GB/s and MFMA use against the dense bf16 peak."""
    t0 = time.time()
    wl = inputs.make_config(idx)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q = to_dev(wl.q.view(np.int16)).view(torch.bfloat16)
    pool0 = to_dev(wl.kv_pool.view(np.int16)).view(torch.bfloat16)
    pools = [pool0] + [pool0.clone() for _ in range(n_pools - 1)]
    table, indptr = to_dev(wl.slot_table), to_dev(wl.slot_indptr)
    prefix, parent = to_dev(wl.prefix_len), to_dev(wl.parent)
    H = wl.num_heads
    T = int(wl.num_tree.sum())
    plan = va.verify_attn_plan(H, wl.prefix_len, wl.num_tree)
    ws = va.workspace_for(plan, dev)
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)

    def step(i, reduce=True):
        va.verify_attn_run(plan, q, pools[i % n_pools], table, indptr, prefix, parent,
                           wl.sm_scale, ws, stream)
        if reduce:
            va.verify_attn_reduce(plan, ws, out, lse, stream)

    with torch.cuda.stream(stream):
        step(0)
    torch.cuda.synchronize()
    if va.verify_attn_read_status(plan, ws, stream) != 0:
        raise RuntimeError(f"config {idx}: device status")
    ms, ms_partial = capture_timer_interleaved(torch, stream)(
        [step, lambda i: step(i, reduce=False)], steps, 5)
    n_row_keys = sum(int(T_r) * H * (int(L_r) + int(T_r))
                     for T_r, L_r in zip(wl.num_tree, wl.prefix_len))
    flops = 2.0 * n_row_keys * (576 + 512)
    kv_bytes = wl.kv_bytes()
    print(f"# config {idx} {wl.name}: {ms * 1e3:.1f} us/call ({time.time() - t0:.1f}s)",
          file=sys.stderr, flush=True)
    return {
        "workload": wl.name, "requests": len(wl.num_tree), "num_heads": H,
        "num_tree": [int(x) for x in wl.num_tree], "prefix_len": [int(x) for x in wl.prefix_len],
        "us_per_call": round(ms * 1e3, 3),
        "partial_us": round(ms_partial * 1e3, 3),
        "kv_gbs": round(kv_bytes / (ms * 1e-3) / 1e9, 2),
        "pct_hbm_peak": round(100.0 * kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
        "mfma_util_pct": round(100.0 * flops / (ms * 1e-3) / 1e12 / BF16_DENSE_PEAK_TFLOPS, 2),
        "partial_mfma_util_pct": round(100.0 * flops / (ms_partial * 1e-3) / 1e12
                                       / BF16_DENSE_PEAK_TFLOPS, 2),
        "nsplit": plan.splits(),
        "work_items": int(plan.total_work),
        "rows_per_block": 64 * int(plan.groups_per_block),
        "pools_rotated": n_pools,
        "steps": steps,
    }


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--warmup-seconds", type=float, default=2.0,
                    help="replay the warmup steps for at least this long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--pools", type=int, default=N_POOLS)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--eager", action="store_true", help="launch without graph capture")
    ap.add_argument("--no-stream-peak", action="store_true",
                    help="skip the 2 GiB streaming-read calibration")
    ap.add_argument("--no-defrag", action="store_true",
                    help="skip the compaction (Tier 1 defrag) measurement")
    ap.add_argument("--no-restart", action="store_true",
                    help="skip the softmax slow-path leg (profiling runs: its three-pass launches "
                         "would mix into the partial kernel's per-dispatch counter means)")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the full-head and ragged-batch workloads")
    ap.add_argument("--workload", type=int, default=WORKLOAD,
                    help="workload index of the main measurement (profiling runs of the "
                         "other workloads; the default is the headline)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the verify path on one GPU only; multi-GPU runs are not "
              "supported (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import speculative_tree_verify_mla_amd as va
    from speculative_tree_verify_mla_amd import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    wl = inputs.make_config(args.workload)
    print(f"# workload {wl.name} generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q = to_dev(wl.q.view(np.int16)).view(torch.bfloat16)
    pool0 = to_dev(wl.kv_pool.view(np.int16)).view(torch.bfloat16)
    pools = [pool0] + [pool0.clone() for _ in range(max(0, args.pools - 1))]
    table = to_dev(wl.slot_table)
    indptr = to_dev(wl.slot_indptr)
    prefix = to_dev(wl.prefix_len)
    parent = to_dev(wl.parent)
    H = wl.num_heads
    T = int(wl.num_tree.sum())

    plan = va.verify_attn_plan(H, wl.prefix_len, wl.num_tree)
    ws = va.workspace_for(plan, dev)
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()

    # split-verify decomposition of the same call (prefix kernel + tree-block
    # kernel + the same reduce), timed beside the fused kernel
    plan_split = va.verify_attn_plan(H, wl.prefix_len, wl.num_tree, split_tree=True)
    ws_split = va.workspace_for(plan_split, dev)

    def step(i, reduce=True, pool_set=None, split=False):
        ps = pools if pool_set is None else pool_set
        pl, w = (plan_split, ws_split) if split else (plan, ws)
        va.verify_attn_run(pl, q, ps[i % len(ps)], table, indptr, prefix, parent, wl.sm_scale,
                           w, stream)
        if reduce:
            va.verify_attn_reduce(pl, w, out, lse, stream)

    def capture(n, reduce=True, pool_set=None, split=False):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for i in range(n):
                    step(i, reduce, pool_set, split)
        return g

    def timed(n, reduce=True, pool_set=None, split=False):
        """Run n steps between two syncs; return (ms from HIP events recorded on
        `stream` around the steps, host wall seconds between the syncs)."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        g = None if args.eager else capture(n, reduce, pool_set, split)
        if g is not None:
            # a graph's first replay carries one-time launch set-up; the
            # timed replay is the second
            with torch.cuda.stream(stream):
                g.replay()
        torch.cuda.synchronize()
        w0 = time.time()
        with torch.cuda.stream(stream):
            e0.record(stream)
            if g is None:
                for i in range(n):
                    step(i, reduce, pool_set, split)
            else:
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1), time.time() - w0

    # correctness of this exact launch configuration against the eager path
    step(0)
    torch.cuda.synchronize()
    status = va.verify_attn_read_status(plan, ws, stream)
    if status != 0:
        raise RuntimeError(f"device status {status}")
    ref_out = out.clone()

    K, W = args.steps, args.warmup
    if W > 0:
        # untimed warm-up: the W-step graph replayed until the GPU has run the
        # path for --warmup-seconds, so the timed steps see steady clocks and
        # translation caches, as a serving loop does
        gw = None if args.eager else capture(W)
        w_end = time.time() + args.warmup_seconds
        while True:
            with torch.cuda.stream(stream):
                if gw is None:
                    for i in range(W):
                        step(i)
                else:
                    gw.replay()
            torch.cuda.synchronize()
            if time.time() >= w_end:
                break
    ms, t_wall = timed(K)
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "graph output differs"
    ms_per_step = ms / K
    ms_partial = timed(K, reduce=False)[0] / K
    ms_warm = timed(K, pool_set=[pools[0]])[0] / K
    ms_partial_warm = timed(K, reduce=False, pool_set=[pools[0]])[0] / K
    ms_split = timed(K, split=True)[0] / K
    out_split = out.clone()        # the split-verify graph's output (all pool copies are equal)
    # spread: the same cold step graph (50 steps) replayed 11 times
    spread_n = 50
    with torch.cuda.stream(stream):
        gs = capture(spread_n)
    torch.cuda.synchronize()
    per_call = []
    for _ in range(12):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            gs.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        per_call.append(e0.elapsed_time(e1) * 1e3 / spread_n)
    per_call = np.array(per_call[1:])   # the first replay carries launch set-up
    spread = {"replays": int(per_call.size), "steps_per_replay": spread_n,
              "us_per_call_p10": round(float(np.percentile(per_call, 10)), 3),
              "us_per_call_p50": round(float(np.percentile(per_call, 50)), 3),
              "us_per_call_p90": round(float(np.percentile(per_call, 90)), 3)}
    split_vs_fused = float((out_split.float() - ref_out.float()).abs().max())
    split_bitwise_equal = bool(torch.equal(out_split.view(torch.int16), ref_out.view(torch.int16)))
    print(f"# timed {K} steps: {ms_per_step * 1e3:.2f} us/step", file=sys.stderr, flush=True)

    kv_bytes = wl.kv_bytes()
    n_keys = wl.num_keys
    rows = wl.total_rows
    flops = 2.0 * rows * n_keys * (576 + 512)
    gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9
    gbs_partial = kv_bytes / (ms_partial * 1e-3) / 1e9

    if args.calibrate_copy_mib > 0:
        nbytes = args.calibrate_copy_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# calibration copy of {nbytes} bytes x3 done", file=sys.stderr, flush=True)

    defrag = None
    if not args.no_defrag:
        defrag = measure_defrag(torch, va, wl, pools[:4], table, indptr, prefix, parent, q, H,
                                K, stream, capture_timer(torch, stream))

    marshal = measure_marshal(torch, va, inputs, dev, capture_timer(torch, stream))

    restart = None
    if args.workload == WORKLOAD and not args.no_restart:
        restart = measure_restart(torch, va, inputs, wl, pools[0], table, indptr, prefix, parent,
                                  H, stream, capture_timer(torch, stream), ms_warm * 1e3)

    other = None
    if not args.no_other_configs:
        # the MFMA-bound workloads: all 64 heads over a 200k prefix, and the
        # ragged four-request batch (parity cases in the tests; timed here)
        other = {"full_heads": measure_config(torch, va, inputs, dev, stream, 4, 3, 20),
                 "ragged": measure_config(torch, va, inputs, dev, stream, 5, 2, 20)}

    stream_peak = None
    if not args.no_stream_peak:
        # measured read ceiling of this GPU: the library's streaming-read
        # helper over 2 GiB (every word read once), best of 5 passes
        big = torch.ones(1 << 29, dtype=torch.float32, device=dev)
        sink = torch.zeros(4096, dtype=torch.int32, device=dev)
        best = None
        with torch.cuda.stream(stream):
            va.verify_attn_stream_read(big, sink, stream)
            for _ in range(5):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                va.verify_attn_stream_read(big, sink, stream)
                e1.record(stream)
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1)
                best = ms if best is None else min(best, ms)
        stream_peak = big.numel() * 4 / (best * 1e-3) / 1e9
        del big

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
        reps = 0
        t_cpu = 0.0
        ref = None
        while reps == 0 or (t_cpu < args.cpu_seconds and reps < 20):
            c0 = time.time()
            ref, ref_lse = oracle.verify_attn_workload(wl, num_threads=threads)
            t_cpu += time.time() - c0
            reps += 1
        per_call = t_cpu / reps
        # one core: every 8th query row of the same call, scaled to all rows
        sub = list(range(0, rows, 8))
        c0 = time.time()
        oracle.verify_attn_workload(wl, rows=sub, num_threads=1)
        per_call_1 = (time.time() - c0) * rows / len(sub)
        cpu = {"value": round(kv_bytes / per_call / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle", "cpu_model": cpu_model(), "nproc": os.cpu_count(),
               "sample": f"{reps} full verify call(s) of the bench workload "
                         f"({rows} rows x {n_keys} keys, fp64), {per_call * 1e3:.0f} ms/call",
               "single_core": {"value": round(kv_bytes / per_call_1 / 1e9, 4), "unit": "GB/s",
                               "cores": 1, "ms_per_call": round(per_call_1 * 1e3, 1),
                               "sample": f"{len(sub)} of the {rows} rows (every 8th), "
                                         f"time scaled by {rows / len(sub):g}"}}
        got = ref_out.float().cpu().numpy().astype(np.float64)
        parity = {"max_abs_out": float(np.abs(got - ref).max()),
                  "max_abs_lse": float(np.abs(lse.cpu().numpy() - ref_lse).max())}

    # the committed counter summary covers the headline workload only
    traffic = traffic_from_profile() if args.workload == WORKLOAD else None
    result = {
        "metric": "effective KV GB/s (% HBM peak) + us/verify call @65k prefix, H=8, T=16",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "requests": 1, "num_heads": H, "num_tree": T,
            "prefix_len": int(wl.prefix_len[0]), "num_slots": wl.num_slots,
            "slot_table": "50% runs of 1-64 consecutive slots, 50% scattered",
            "tree": "random, depth<=6", "pools_rotated": len(pools),
            "timing": "eager" if args.eager else "hip graph replay",
        },
        "us_per_call": round(ms_per_step * 1e3, 3),
        "spread": spread,
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "stream_read_peak_gbs": None if stream_peak is None else round(stream_peak, 1),
        "pct_stream_read_peak": None if stream_peak is None else round(100.0 * gbs / stream_peak, 2),
        "mfma_util_pct": round(100.0 * flops / (ms_per_step * 1e-3) / 1e12
                               / BF16_DENSE_PEAK_TFLOPS, 2),
        "warm_us_per_call": round(ms_warm * 1e3, 3),
        "warm_value": round(kv_bytes / (ms_warm * 1e-3) / 1e9, 2),
        "nsplit": plan.splits(),
        "work_items": int(plan.total_work),
        "rows_per_block": 64 * int(plan.groups_per_block),
        "kv_bytes_per_call": kv_bytes,
        "roofline": {
            "kernel": "va_wide_kernel" if plan.groups_per_block == 2 else "va_partial_kernel",
            "bound": roofline_bound(flops, kv_bytes),
            "arith_intensity_flop_per_byte": round(flops / kv_bytes, 1),
            "ridge_flop_per_byte": round(BF16_DENSE_PEAK_TFLOPS * 1e3 / HBM_PEAK_GBS, 1),
            "warm_over_cold": round(ms_partial_warm / ms_partial, 3),
            "hbm_limited": bool(ms_partial_warm < HBM_LIMITED_WARM_RATIO * ms_partial),
            "achieved": round(gbs_partial, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs_partial / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_us": round(ms_partial * 1e3, 3),
            "warm_avg_us": round(ms_partial_warm * 1e3, 3),
        },
        "ab_split_verify": {
            "mode": "prefix kernel without tree mask + tree-block kernel + the same reduce",
            "us_per_call": round(ms_split * 1e3, 3),
            "value": round(kv_bytes / (ms_split * 1e-3) / 1e9, 2),
            "nsplit": plan_split.splits(),
            "max_abs_out_vs_fused": split_vs_fused,
            "bitwise_equal_to_fused": split_bitwise_equal,
        },
        "other_configs": other,
        "defrag": defrag,
        "tree_marshal": marshal,
        "restart_path": restart,
        "cpu_baseline": cpu,
        "parity_vs_oracle": parity,
        "wall_s_timed": round(t_wall, 3),
    }
    if args.workload != WORKLOAD:
        result["note"] = f"profiling run of workload {wl.name}, not the headline configuration"
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
