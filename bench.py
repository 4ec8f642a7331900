"""Benchmark of one rank's FSDP2 sharded step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--also 4]

A step is one pass of the whole per-rank hot path over every parameter group
of the workload: for each group, reduce (bf16 [N, S] gradient contributions
-> fp32 mean) -> AdamW (fp32 master, m, v) -> pack (bf16 copy-in, written in
place into row `rank` of the all-gather buffer) -> unpack (bf16 [N, S] ->
full parameters).  Other ranks' rows are synthetic data already in HBM; the
collectives themselves are not part of the step.  Inputs are resident in HBM
before the timed region starts.

Prints one JSON line for the headline workload (the 7B-shaped per-rank share
by default): params/s of this rank's shard (value), effective HBM GB/s (the
bytes the step's kernels move / time) and its fraction of the 8 TB/s HBM
peak and of a copy ceiling measured in the same run with the library's own
copy kernel, the roofline of the dominant kernel (the one with the most
algorithmic bytes) measured with HIP events around one launch per group
inside the timed region, and the CPU oracle timed on a bounded sample of the
same workload.  The same record for each workload named by --also (the
70B-shaped per-rank share by default) sits under "also".

By default reduce, AdamW and pack run as one fused launch per group
(fsdp_step_shard, bit-identical to the three calls); --unfused runs them as
three launches per group, --group-set as separate kernels through a group
set (a reduce per group, then one AdamW and one copy-in launch over every
group), and --group-set-fused as a group set with AdamW and the copy-in fused
in one launch.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "sharded-step params/sec per GPU + effective HBM GB/s (% of MI355X peak)"


def algorithmic_bytes(S, V, F, N, fused, adamw_copy_in=False):
    """Bytes each kernel must move once per group.

    reduce: read N bf16 contributions (2NV) + write the fp32 grad (4V);
    adamw: read p, g, m, v (16V) + write p, m, v (12V); pack: read 4V fp32 +
    write 2S bf16; unpack: read 2F + write 2F.  The fused step reads 2NV + 12V
    and writes 12V + 2S: the gradient never goes to HBM.  AdamW fused with the
    copy-in (adamw_copy_in) reads 16V and writes 12V + 2S: the master is read
    once for both.
    """
    if fused:
        return {"step": 2 * N * V + 24 * V + 2 * S, "unpack": 4 * F}
    if adamw_copy_in:
        return {"reduce": 2 * N * V + 4 * V, "adamw_pack": 28 * V + 2 * S, "unpack": 4 * F}
    return {"reduce": 2 * N * V + 4 * V, "adamw": 28 * V, "pack": 4 * V + 2 * S,
            "unpack": 4 * F}


# rocprofv3 kernel names; the fused step has variants for 16-byte aligned rows
# (the wide one from 16 ranks)
KERNEL_SYMBOLS = {"step": ("step_kernel_wide", "step_kernel_aligned", "step_kernel"),
                  "reduce": ("reduce_kernel",),
                  "adamw": ("adamw_kernel",), "pack": ("pack_kernel",),
                  "unpack": ("unpack_kernel",), "adamw_pack": ("adamw_pack_kernel",)}


def measured_traffic(workload, rank, align, kind):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/pmc_traffic.json), or None when there is none for this kernel
    and workload or the kernel source has changed since it was taken."""
    from sharded_shard_amd.build import kernel_sources_sha256
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        rec = json.load(open(path))
        sha = kernel_sources_sha256()
    except (OSError, ValueError):
        return None
    if rec.get("kernels_source_sha256") != sha:
        return None
    wl = rec.get("workloads", {}).get(workload)
    if not wl or wl.get("rank") != rank or wl.get("align_elems") != align:
        return None
    for sym in KERNEL_SYMBOLS.get(kind, ()):
        k = wl.get("kernels", {}).get(sym)
        if k is not None:
            return k["traffic_bytes_per_launch"]
    return None


TRAFFIC_SOURCE = ("HBM bytes per launch from the rocprofv3 memory-request counters "
                  "(TCC_EA0_RDREQ_32B/64B/128B, TCC_EA0_WRREQ/WRREQ_64B) in the committed "
                  "profiles/pmc_traffic.json; valid only for the kernel sources it was taken on "
                  "(null otherwise)")


KERNEL_NAMES = {"step": "step_kernel (fused reduce+adamw+pack)", "reduce": "reduce_kernel",
                "adamw": "adamw_kernel", "pack": "pack_kernel (copy-in)",
                "unpack": "unpack_kernel (copy-out)",
                "adamw_pack": "adamw_pack_kernel (AdamW fused with the copy-in)"}
# kinds a group set launches once per step over every group; the others run
# once per group
SET_KINDS = ("adamw", "pack", "adamw_pack")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4])
    ap.add_argument("--also", default=None,
                    help="comma-separated configs measured after the headline one and reported "
                         "under 'also' (default: 4 with --config 2, none otherwise; 'none')")
    ap.add_argument("--rank", type=int, default=None, help="simulated rank (default: the config's)")
    ap.add_argument("--align", type=int, default=1, choices=[1, 8])
    ap.add_argument("--unfused", action="store_true",
                    help="run reduce, adamw and pack as separate launches per group instead of "
                         "the fused step")
    ap.add_argument("--group-set", action="store_true",
                    help="separate kernels through a group set: reduce per group, then one "
                         "adamw and one copy-in launch over every group")
    ap.add_argument("--group-set-fused", action="store_true",
                    help="as --group-set, with AdamW and the copy-in fused in one launch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown-steps", type=int, default=3,
                    help="extra untimed steps per kernel kind, with events around its launches")
    ap.add_argument("--isolated", action=argparse.BooleanOptionalAction, default=True,
                    help="also time every kernel kind alone per group after flushing the "
                         "last-level cache (per-kernel roofline protocol)")
    ap.add_argument("--no-copy-ceiling", action="store_true",
                    help="skip the copy-ceiling measurement (profiled runs: its copies use the "
                         "resharding kernel)")
    ap.add_argument("--no-next", action="store_true",
                    help="skip timing the reduce-scatter copy-in and fp32-contribution kernels")
    ap.add_argument("--no-next-group-set", action="store_true",
                    help="skip timing the FP8 copy-in of every group in one launch (a kernel "
                         "trace would merge it with the per-group launches)")
    ap.add_argument("--graph", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the step captured in a HIP graph and replayed")
    ap.add_argument("--no-references", action="store_true",
                    help="skip timing the AdamW and copy-in kernels beside torch's kernels of "
                         "the same access pattern")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain device-to-device copy of 2 GiB instead (the "
                         "reference for HBM byte counters and the copy ceiling)")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be at least 1 and --warmup at least 0")
    if args.group_set_fused:
        args.group_set = True
    if args.also is None:
        args.also = "4" if args.config == 2 else "none"
    try:
        args.also = [] if args.also == "none" else [int(c) for c in args.also.split(",") if c]
    except ValueError:
        ap.error("--also takes comma-separated config numbers or 'none'")
    if any(c not in (1, 2, 3, 4) or c == args.config for c in args.also):
        ap.error("--also configs must be among 1-4 and differ from --config")
    return args


def copy_calibration(reps=10):
    """torch's own copy kernel on 2 GiB: known bytes read and written per launch."""
    import torch
    n = 1 << 29
    src = torch.ones(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    nbytes = 4 * n
    return {"copy_calibration": {"bytes_read_per_launch": nbytes, "bytes_written_per_launch": nbytes,
                                 "avg_launch_ms": ms, "GBps": 2 * nbytes / (ms * 1e-3) / 1e9,
                                 "hbm_frac": 2 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}}


def cpu_baseline(cfg, rank, min_s=10.0, max_s=30.0):
    """Time the CPU oracle on whole groups (first block, root, more blocks) for
    one step each, until at least min_s of oracle time has accumulated."""
    import numpy as np
    import torch

    from oracle import fsdp as O
    from workloads import synth

    n = cfg.world
    hp = vars(cfg.hp)
    order = [0] + ([len(cfg.groups) - 1] if len(cfg.groups) > 1 else []) + \
        list(range(1, len(cfg.groups) - 1))
    sample = [cfg.groups[i] for i in order]
    total_t, total_v = 0.0, 0
    names = []
    for gi, grp in enumerate(sample):
        shapes = [p.shape for p in grp.params]
        plan = O.plan(shapes, n, rank)
        masters = [synth.normal_f32(e.valid_numel, cfg.master_std, ("cpu", gi, i)).numpy()
                   for i, e in enumerate(plan.entries)]
        ms = [np.zeros_like(x) for x in masters]
        vs = [np.zeros_like(x) for x in masters]
        rs = np.empty((n, plan.S), dtype=np.uint16)
        ag = np.empty((n, plan.S), dtype=np.uint16)
        for j in range(n):
            rs[j] = synth.bf16_bits_to_u16(synth.normal_bf16_bits(plan.S, cfg.grad_std, ("cpu-rs", gi, j)))
            ag[j] = synth.bf16_bits_to_u16(synth.normal_bf16_bits(plan.S, cfg.master_std, ("cpu-ag", gi, j)))
        t0 = time.perf_counter()
        grads = O.reduce(plan, rs)
        for x, g, m, v in zip(masters, grads, ms, vs):
            O.adamw(x, g, m, v, 1, **hp)
        ag[rank] = O.pack(plan, masters)
        O.unpack(plan, ag)
        total_t += time.perf_counter() - t0
        total_v += plan.V
        names.append(grp.name)
        del rs, ag, grads
        if total_t >= min_s or total_t + total_t / len(names) > max_s:
            break
    rate = total_v / total_t
    all_v = sum(O.plan([p.shape for p in g.params], n, rank).V for g in cfg.groups)
    out = {
        "value": rate,
        "unit": "params/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"one step of {len(names)} of {len(cfg.groups)} groups ({names[0]}, "
                   f"{names[-1]}, ...) of {cfg.name}, rank {rank}: {total_v} params "
                   f"in {total_t:.2f} s (NumPy, single thread; host has {os.cpu_count()} cpus, "
                   f"affinity {len(os.sched_getaffinity(0))})"),
        "extrapolated": len(names) < len(cfg.groups),
    }
    if out["extrapolated"]:
        out["extrapolation"] = (f"rate over the sampled groups applied to the whole step: "
                                f"{all_v} params at this rate = {all_v / rate:.1f} s per step")
    return out


def measure_next(groups, n, rs_bf16, full_arena, stream, reps, with_set=True):
    """Per-kernel rates of the kernels beyond the step, on the same groups:
    the reduce-scatter copy-ins (full bf16 grads -> [N, S] bf16, widened to
    fp32, and from fp32 accumulators), the reduction of fp32 contributions,
    accumulation, the FP8 copy-in (per group, and of every group in one
    launch through a group set) and copy-out, and resharding of the first
    group.  The full-parameter arena stands in for the unsharded
    gradients."""
    import torch
    from sharded_shard_amd import capi

    max_ns = max(n * g.S for g in groups)
    rs_f32 = torch.empty(max_ns, dtype=torch.float32, device=full_arena.device)
    acc_arena = torch.zeros(max(g.full_space for g in groups), dtype=torch.float32,
                            device=full_arena.device)
    ag_u8 = rs_bf16.view(torch.uint8)               # [N, S] bytes fit in the bf16 arena
    fp8_scales = torch.full((max(len(g.rows) for g in groups),), 448.0 / 0.1,
                            dtype=torch.float32, device=full_arena.device)
    for g in groups:
        g.bind_full_grad(full_arena, stream)
        g.bind_grad_acc(acc_arena, stream)
        g.bind_full_fp8(full_arena.view(torch.uint8), stream)
    kinds = {
        "rs_copy_in_bf16": (lambda g: g.pack_reduce_scatter(rs_bf16[:n * g.S], capi.FSDP_DTYPE_BF16, stream),
                            lambda g: 2 * g.F + 2 * n * g.S),
        "rs_copy_in_f32": (lambda g: g.pack_reduce_scatter(rs_f32[:n * g.S], capi.FSDP_DTYPE_F32, stream),
                           lambda g: 2 * g.F + 4 * n * g.S),
        "reduce_f32": (lambda g: g.reduce_f32(rs_f32[:n * g.S], stream),
                       lambda g: 4 * n * g.V + 4 * g.V),
        "fp8_copy_in": (lambda g: g.pack_fp8(ag_u8[:g.S], fp8_scales, stream),
                        lambda g: 4 * g.V + g.S),
        "fp8_copy_out": (lambda g: g.unpack_fp8(ag_u8[:n * g.S], stream), lambda g: 2 * g.F),
        "grad_accumulate": (lambda g: g.accumulate_grad(False, stream), lambda g: 10 * g.F),
        "rs_copy_in_from_acc": (lambda g: g.pack_reduce_scatter_acc(rs_f32[:n * g.S], stream),
                                lambda g: 4 * g.F + 4 * n * g.S),
    }
    # resharding: load the first group's fp32 shards, saved by N ranks (the
    # rows of rs_f32 as [N, S] segments), into rank 0 of N/2 ranks
    g0 = groups[0]
    n2 = max(1, n // 2)
    rplan = capi.fsdp_reshard_plan_create(g0.rows, g0.cols, n, n2, 0)
    _, dst_numel = capi.fsdp_reshard_plan_runs(rplan)
    dst = torch.empty(max(1, dst_numel + 64 * len(g0.rows)), dtype=torch.float32, device=full_arena.device)
    src_ptrs = [rs_f32[s * g0.S + e.shard_offset:].data_ptr()
                for e in g0.entries for s in range(n)]
    dst_ptrs, o = [], 0
    for r, c in zip(g0.rows, g0.cols):
        dst_ptrs.append(dst[o:].data_ptr())
        o += (-(-r // n2) * c + 63) // 64 * 64
    capi.fsdp_reshard_bind(rplan, src_ptrs, dst_ptrs, 4, stream)
    kinds[f"reshard_f32_{n}_to_{n2}_first_group"] = (
        lambda g: capi.fsdp_reshard_execute(rplan, stream) if g is g0 else None,
        lambda g: 8 * dst_numel if g is g0 else 0)
    # the FP8 copy-in of every group as one launch through a group set (a
    # kernel trace would merge it with the per-group launches of the same
    # kernel: profiled runs leave it out)
    gset = capi.fsdp_group_set_create([g.plan for g in groups], stream) if with_set else None
    set_scales = set_arena8 = None
    if with_set:
        _, n_params, set_elems = capi.fsdp_group_set_sizes(gset)
        set_scales = torch.full((max(1, n_params),), 448.0 / 0.1, dtype=torch.float32,
                                device=full_arena.device)
        set_arena8 = torch.empty(max(1, set_elems), dtype=torch.uint8, device=full_arena.device)
        kinds["fp8_copy_in_group_set"] = (
            lambda g: capi.fsdp_pack_allgather_fp8_groups(gset, set_arena8, set_scales, stream)
            if g is g0 else None,
            lambda g: sum(4 * x.V + x.S for x in groups) if g is g0 else 0)
    res = {}
    for name, (fn, nbytes) in kinds.items():
        busy = [g for g in groups if nbytes(g) > 0]
        evs = []
        for _ in range(reps + 1):
            for g in busy:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn(g)
                b.record(stream)
                evs.append((a, b))
        torch.cuda.synchronize()
        evs = evs[len(busy):]                       # first pass warms up
        ms = sum(a.elapsed_time(b) for a, b in evs) / reps
        byts = sum(nbytes(g) for g in groups)
        gbps = byts / (ms * 1e-3) / 1e9
        res[name] = {"ms_per_step": round(ms, 4), "algorithmic_GB_per_step": round(byts / 1e9, 4),
                     "GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}
    capi.fsdp_reshard_plan_destroy(rplan)
    if gset is not None:
        capi.fsdp_group_set_destroy(gset)
    del rs_f32, dst, acc_arena, fp8_scales, set_scales, set_arena8
    res["adamw_host_cpu_offload"] = measure_host_adamw()
    return res


def _pct(sorted_vals, q):
    """Nearest-rank percentile of an ascending list."""
    i = max(0, min(len(sorted_vals) - 1, -(-q * len(sorted_vals) // 100) - 1))
    return round(sorted_vals[i], 4)


def measure_isolated(groups, kinds, n, rank, hp, rs_arena, ag_arena, fused, stream,
                     gset=None, arena=None, adamw_copy_in=False):
    """Each kernel kind launched alone per group (or, for the kinds a group
    set runs in one launch, alone over every group) after the 256 MB MALL has
    been flushed, so no input can come from the last-level cache: the
    per-kernel roofline protocol.  The flush writes 1 GiB and then reads
    another 1 GiB, so the cache holds only clean lines when the timed launch
    starts (no write-back of the flush lands in it).

    A launch can end with up to 256 MB of its own writes still dirty in the
    MALL, written back to HBM after its end event; for a short, write-heavy
    launch that flatters its rate.  So each launch is also followed by a
    1 GiB read sweep, which evicts those lines, and timed up to the sweep's
    end, minus the same sweep's time on a clean cache: the launch's full
    cost, write-backs included.  Reports sum of algorithmic bytes / sum of
    durations over the launches, both ways."""
    import torch
    from sharded_shard_amd import capi
    dev = rs_arena[0].device
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sweep = torch.zeros(1 << 28, dtype=torch.int32, device=dev)
    evict = torch.zeros(1 << 28, dtype=torch.int32, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def clean(tag):
        flush.fill_(tag & 0xFF)
        sweep.max()                         # read-only pass over another 1 GiB

    def timed(launch, tag):
        """(launch alone, launch plus the write-backs it left) in ms."""
        clean(tag)
        a, b, c = ev(), ev(), ev()
        a.record(stream)
        launch()
        b.record(stream)
        evict.max()
        c.record(stream)
        clean(tag + 1)
        a2, c2 = ev(), ev()
        a2.record(stream)
        evict.max()
        c2.record(stream)
        c2.synchronize()
        return a.elapsed_time(b), a.elapsed_time(c) - a2.elapsed_time(c2)

    res = {}
    t = 10_000
    for k in kinds:
        tot_b = tot_ms = tot_wb = 0.0
        if gset is not None and k in SET_KINDS:
            launch = {"adamw": lambda: capi.fsdp_adamw_groups(gset, step=t, stream=stream, **hp),
                      "pack": lambda: capi.fsdp_pack_allgather_groups(gset, arena, stream),
                      "adamw_pack": lambda: capi.fsdp_adamw_pack_groups(
                          gset, arena, step=t, stream=stream, **hp)}[k]
            tot_ms, tot_wb = timed(launch, t)
            tot_b = sum(algorithmic_bytes(g.S, g.V, g.F, n, fused, adamw_copy_in)[k]
                        for g in groups)
            t += 1
        else:
            for gi, g in enumerate(groups):
                rs = rs_arena[gi & 1][:n * g.S]
                ag_in = ag_arena[gi & 1][rank * g.S:(rank + 1) * g.S]
                ag_out = ag_arena[gi & 1][:n * g.S]
                launch = {"step": lambda: g.step(rs, ag_in, t, **hp, stream=stream),
                          "reduce": lambda: g.reduce(rs, stream),
                          "adamw": lambda: g.adamw(t, **hp, stream=stream),
                          "pack": lambda: g.pack(ag_in, stream),
                          "unpack": lambda: g.unpack(ag_out, stream)}[k]
                ms, wb = timed(launch, gi)
                tot_ms += ms
                tot_wb += wb
                tot_b += algorithmic_bytes(g.S, g.V, g.F, n, fused, adamw_copy_in)[k]
                t += 1
        gbps = tot_b / (tot_ms * 1e-3) / 1e9
        wb_gbps = tot_b / (tot_wb * 1e-3) / 1e9 if tot_wb > 0 else None
        res[k] = {"isolated_GBps": round(gbps, 1), "isolated_hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
                  "isolated_with_writeback_GBps": round(wb_gbps, 1) if wb_gbps else None,
                  "isolated_with_writeback_hbm_frac":
                      round(wb_gbps / HBM_PEAK_GBPS, 4) if wb_gbps else None}
    del flush, sweep, evict
    return res


def measure_pattern_references(dev, stream, n=1 << 28, reps=5):
    """The library's AdamW and copy-in beside torch's own kernels with the
    same access pattern, on the same n-element fp32 shards (4 GiB of p, g, m
    and v: the launches stream from HBM): torch's fused AdamW reads p, g, m,
    v and writes p, m, v (28 B per element, as fsdp_adamw_shard); torch's
    fp32 -> bf16 cast reads 4 B and writes 2 B per element (as the copy-in).
    Each rate is the best of `reps` event-timed launches; context for the
    kernels' fractions of peak, not a target."""
    import torch
    from sharded_shard_amd import capi
    from workloads import synth
    p = synth.normal_f32(n, 0.02, ("ref-p",), device=dev)
    g = synth.normal_f32(n, 1e-3, ("ref-g",), device=dev)
    m, v = torch.zeros_like(p), torch.zeros_like(p)
    out = torch.empty(n, dtype=torch.bfloat16, device=dev)
    plan = capi.fsdp_plan_create([n], [1], 1, 0, 1)
    hp = dict(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    step_t = torch.zeros((), dtype=torch.float32, device=dev)

    def best(fn):
        ms = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ms.append(a.elapsed_time(b))
        return min(ms)

    def torch_adamw():
        step_t.add_(1)      # a tiny launch of its own, before the timed region's main kernel
        torch._fused_adamw_([p], [g], [m], [v], [], [step_t], lr=hp["lr"], beta1=hp["beta1"],
                            beta2=hp["beta2"], weight_decay=hp["weight_decay"], eps=hp["eps"],
                            amsgrad=False, maximize=False)

    try:
        capi.fsdp_bind(plan, [p], [g], [m], [v], None, stream)
        t = [0]

        def ours_adamw():
            t[0] += 1
            capi.fsdp_adamw_shard(plan, step=t[0], stream=stream, **hp)

        res = {}
        for name, fn, bpe in (("adamw_kernel", ours_adamw, 28),
                              ("torch_fused_adamw", torch_adamw, 28),
                              ("pack_kernel", lambda: capi.fsdp_pack_allgather(plan, out, stream), 6),
                              ("torch_cast_f32_to_bf16", lambda: out.copy_(p), 6)):
            try:
                fn()                               # warm
            except (RuntimeError, AttributeError, TypeError) as e:
                if name.startswith("torch"):       # a torch build without that kernel
                    res[name] = {"error": f"{type(e).__name__}: {e}"[:200]}
                    continue
                raise
            ms = best(fn)
            gbps = bpe * n / (ms * 1e-3) / 1e9
            res[name] = {"ms": round(ms, 4), "GBps": round(gbps, 1),
                         "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}
        res["elements"] = n
        res["note"] = ("same fp32 shards for all four; torch's AdamW timing includes its step "
                       "counter's own small launch")
        return res
    finally:
        capi.fsdp_plan_destroy(plan)
        del p, g, m, v, out
        torch.cuda.empty_cache()


def measure_host_adamw(n=1 << 25, reps=3):
    """CPU-offload AdamW on 32M host fp32 elements (28 B each per step): the
    rate of host memory, on every hardware thread the process may use."""
    import numpy as np
    from sharded_shard_amd import capi
    rng = np.random.default_rng(0)
    p = rng.standard_normal(n, dtype=np.float32) * np.float32(0.02)
    g = rng.standard_normal(n, dtype=np.float32) * np.float32(1e-3)
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    threads = len(os.sched_getaffinity(0))
    best = None
    for t in range(1, reps + 2):
        t0 = time.perf_counter()
        capi.fsdp_adamw_host(p, g, m, v, 3e-4, 0.9, 0.999, 1e-8, 0.01, step=t, n_threads=threads)
        dt = time.perf_counter() - t0
        if t > 1:
            best = dt if best is None else min(best, dt)
    return {"ms": round(best * 1e3, 3), "elements": n, "threads": threads,
            "host_GBps": round(28 * n / best / 1e9, 1), "note": "host DRAM, not HBM"}


def measure_copy_ceiling(dev, stream, sizes=(1 << 29, 1 << 30, 1 << 31), reps=5):
    """A plain device copy through the library's own copy kernel (the
    resharding executor at 1 -> 1 rank: one run, the copy-out's block shape
    and cache policy), timed with HIP events over `reps` launches for each
    size (source plus destination 4x to 16x the 256 MB MALL, so the launches
    stream from HBM).  The fastest size is the ceiling of a 1:1 read/write
    stream on this GPU, measured in the same run as the step; every size's
    rate is listed (on MI355X a 1 GiB copy measured faster than a 4 GiB one)."""
    import torch
    from sharded_shard_amd import capi
    rates = {}
    rows = 8192
    for nbytes in sizes:
        cols = nbytes // 2 // rows
        src = torch.ones(rows * cols, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        rp = capi.fsdp_reshard_plan_create([rows], [cols], 1, 1, 0)
        try:
            capi.fsdp_reshard_bind(rp, [src.data_ptr()], [dst.data_ptr()], 2, stream)
            for _ in range(3):
                capi.fsdp_reshard_execute(rp, stream)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                capi.fsdp_reshard_execute(rp, stream)
            b.record(stream)
            b.synchronize()
            ms = a.elapsed_time(b) / reps
            if not torch.equal(dst, src):
                raise RuntimeError("copy ceiling: the copy kernel did not reproduce its source")
        finally:
            capi.fsdp_reshard_plan_destroy(rp)
        rates[nbytes] = (ms, 2 * rows * cols * 2 / (ms * 1e-3) / 1e9)
        del src, dst
        torch.cuda.empty_cache()
    best = max(rates, key=lambda k: rates[k][1])
    ms, gbps = rates[best]
    return {"kernel": "copy_runs_kernel via fsdp_reshard_execute (1 -> 1 rank, one bf16 run)",
            "bytes_per_launch": 2 * best, "avg_launch_ms": round(ms, 4),
            "GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "by_size_GBps": {f"{k >> 20} MiB": round(v[1], 1) for k, v in rates.items()}}


def run_workload(cfg_index, args, dev, copy_gbps):
    """Build, time and describe one workload; returns its record."""
    import torch
    from sharded_shard_amd import capi
    from sharded_shard_amd.group import ShardedGroup
    from workloads import configs, synth

    cfg = configs.get(cfg_index)
    n = cfg.world
    rank = cfg.timing_rank if args.rank is None else args.rank
    hp = vars(cfg.hp)
    print(f"bench: {cfg.name} rank={rank} groups={len(cfg.groups)}", file=sys.stderr, flush=True)

    # ---- persistent state: per-group shards, shared double-buffered arenas --------
    groups = []
    for gi, grp in enumerate(cfg.groups):
        g = ShardedGroup([p.shape for p in grp.params], n, rank, args.align, bind=False)
        groups.append(g)
    full_space = max(g.full_space for g in groups)
    max_ns = max(n * g.S for g in groups)
    full_arena = torch.empty(full_space, dtype=torch.int16, device=dev)
    rs_arena = [torch.empty(max_ns, dtype=torch.int16, device=dev) for _ in range(2)]
    ag_arena = [torch.empty(max_ns, dtype=torch.int16, device=dev) for _ in range(2)]
    for b in range(2):
        synth.fill_normal_bf16_bits_(rs_arena[b], cfg.grad_std, ("bench-rs", cfg_index, b))
        synth.fill_normal_bf16_bits_(ag_arena[b], cfg.master_std, ("bench-ag", cfg_index, b))
    for gi, g in enumerate(groups):
        g.full_flat = full_arena
        g.allocate(full=False)
        synth.fill_normal_f32_(g.master_flat, cfg.master_std, ("bench-master", cfg_index, gi))
        g.bind()
    torch.cuda.synchronize()
    print("bench: state resident", file=sys.stderr, flush=True)

    V = sum(g.V for g in groups)
    fused = not (args.unfused or args.group_set)
    aci = args.group_set_fused
    kinds = list(algorithmic_bytes(1, 1, 1, n, fused, aci))
    byts = {k: 0 for k in kinds}
    for g in groups:
        for k, b in algorithmic_bytes(g.S, g.V, g.F, n, fused, aci).items():
            byts[k] += b
    step_bytes = sum(byts.values())
    dominant = max(kinds, key=lambda k: byts[k])

    stream = torch.cuda.current_stream()
    step_counter = [0]
    # One native call per step runs every group's launches (no per-launch
    # Python on the critical path); HIP events around one kernel kind per
    # group are recorded by the library on the same stream.  The fused step
    # runs per group; the separate kernels run as a group set: a reduce per
    # group, one AdamW and one copy-in launch over every group (into an arena
    # of every group's segment), a copy-out per group.
    gset = arena = None
    if args.group_set:
        gset = capi.fsdp_group_set_create([g.plan for g in groups], stream)
        arena = torch.empty(max(1, capi.fsdp_group_set_segment(gset, 0)[1]), dtype=torch.int16,
                            device=dev)

    def make_execute(on_stream):
        if not args.group_set:
            return capi.StepGroupsCall(
                [g.plan for g in groups],
                [rs_arena[gi & 1][:n * g.S] for gi, g in enumerate(groups)],
                [ag_arena[gi & 1][rank * g.S:(rank + 1) * g.S] for gi, g in enumerate(groups)],
                [ag_arena[gi & 1][:n * g.S] for gi, g in enumerate(groups)],
                flags=0 if fused else capi.FSDP_STEP_UNFUSED, stream=on_stream, **hp)
        return capi.StepGroupSetCall(
            gset, [g.plan for g in groups],
            [rs_arena[gi & 1][:n * g.S] for gi, g in enumerate(groups)], arena,
            [ag_arena[gi & 1][:n * g.S] for gi, g in enumerate(groups)],
            flags=capi.FSDP_SET_ADAMW_COPY_IN if aci else 0, stream=on_stream, **hp)

    execute = make_execute(stream)
    one_launch = set(SET_KINDS) if args.group_set else set()

    def launch_bytes(kind, gi):
        """Algorithmic bytes of the launch of `kind` timed by group gi's events."""
        if kind in one_launch:
            return byts[kind]
        return algorithmic_bytes(groups[gi].S, groups[gi].V, groups[gi].F, n, fused, aci)[kind]
    kernel_id = {"step": capi.FSDP_KERNEL_STEP, "reduce": capi.FSDP_KERNEL_REDUCE,
                 "adamw": capi.FSDP_KERNEL_ADAMW, "pack": capi.FSDP_KERNEL_PACK,
                 "unpack": capi.FSDP_KERNEL_UNPACK, "adamw_pack": capi.FSDP_KERNEL_ADAMW_PACK}

    def new_events():
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(groups))]
        for e in evs:          # create the underlying hipEvents now
            e.record(stream)
        return evs

    def step(kind=None, evs=None):
        step_counter[0] += 1
        if kind is None:
            execute(step_counter[0])
        else:
            execute(step_counter[0], kernel_id[kind], evs)

    def elapsed_sampled(evs):
        return [(i, evs[2 * i].elapsed_time(evs[2 * i + 1])) for i in range(len(groups))
                if evs[2 * i] is not None]

    for _ in range(args.warmup):
        step()
    # Each group's launch of the dominant kernel is timed once over the timed
    # steps (group g in step g mod K): a recorded event pair costs the two
    # launches around it their back-to-back dispatch (about 6 us per pair on
    # MI355X), so timing every launch of every step would slow the steps the
    # same region measures.
    timed_events = []
    for k in range(args.steps):
        evs = new_events()
        if dominant in one_launch:      # its one launch per step, every step
            timed_events.append([e if i < 2 else None for i, e in enumerate(evs)])
        else:
            timed_events.append([e if (i // 2) % args.steps == k else None
                                 for i, e in enumerate(evs)])
    torch.cuda.synchronize()
    print(f"bench: {args.warmup} warmup steps done", file=sys.stderr, flush=True)

    # one event at every step boundary: the distribution of step times
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    start, end = bounds[0], bounds[-1]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        step(dominant, timed_events[k])
        bounds[k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = start.elapsed_time(end) / args.steps
    step_ms = sorted(bounds[k].elapsed_time(bounds[k + 1]) for k in range(args.steps))
    print(f"bench: {args.steps} timed steps, {ms_step:.3f} ms/step", file=sys.stderr, flush=True)
    dom = [x for evs in timed_events for x in elapsed_sampled(evs)]
    dom_launches = len(dom)
    dom_avg_ms = sum(ms for _, ms in dom) / max(1, dom_launches)
    dom_bytes_per_launch = sum(launch_bytes(dominant, i) for i, _ in dom) / max(1, dom_launches)
    achieved = dom_bytes_per_launch / (dom_avg_ms * 1e-3) / 1e9

    # per-kernel breakdown: extra untimed steps, each timing one kernel kind
    # (events around every launch of that kind)
    per = {k: 0.0 for k in kinds}
    if args.breakdown_steps > 0:
        runs = {k: [new_events() for _ in range(args.breakdown_steps)] for k in kinds}
        for k in one_launch & set(kinds):
            runs[k] = [[e if i < 2 else None for i, e in enumerate(evs)] for evs in runs[k]]
        torch.cuda.synchronize()
        for k in kinds:
            for evs in runs[k]:
                step(k, evs)
        torch.cuda.synchronize()
        per = {k: sum(sum(ms for _, ms in elapsed_sampled(evs)) for evs in runs[k])
               / args.breakdown_steps for k in kinds}

    # the same step captured once in a HIP graph and replayed: the launches
    # without host work between them (step index fixed in the graph; the
    # same kernels and bytes)
    graph_rec = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            gcall = make_execute(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=side):
                gcall(step_counter[0] + 1)
        torch.cuda.synchronize()
        for _ in range(2):
            graph.replay()
        ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ga.record(stream)
        for _ in range(args.steps):
            graph.replay()
        gb.record(stream)
        gb.synchronize()
        g_ms = ga.elapsed_time(gb) / args.steps
        graph_rec = {"ms_per_step": g_ms, "params_per_s": V / (g_ms * 1e-3), "steps": args.steps,
                     "note": "one step captured in a HIP graph (its step index fixed) and "
                             "replayed; the same kernels and bytes as the timed steps"}
        del graph, gcall

    def frac(gbps, ref):
        return round(gbps / ref, 4) if gbps and ref else None

    kernels = {}
    for k in kinds:
        gbps = byts[k] / (per[k] * 1e-3) / 1e9 if per[k] else None
        kernels[k] = {"kernel": KERNEL_NAMES[k], "ms_per_step": round(per[k], 4),
                      "launches_per_step": 1 if k in one_launch else len(groups),
                      "algorithmic_GB_per_step": round(byts[k] / 1e9, 4),
                      "GBps": round(gbps, 1) if gbps else None,
                      "hbm_frac": frac(gbps, HBM_PEAK_GBPS),
                      "frac_of_copy_ceiling": frac(gbps, copy_gbps),
                      "traffic_bytes_per_launch": measured_traffic(cfg.name, rank, args.align, k)}
    if args.isolated:
        iso = measure_isolated(groups, kinds, n, rank, hp, rs_arena, ag_arena, fused, stream,
                               gset, arena, aci)
        for k in kinds:
            kernels[k].update(iso[k])

    eff_gbps = step_bytes / (ms_step * 1e-3) / 1e9
    # the method's own bytes per step, counted kernel by kernel as if unfused
    # (reduce 2NV+4V, AdamW 28V, copy-in 4V+2S, copy-out 4F): what a step
    # moves when each stage is its own pass over HBM.  Divided by the fused
    # step's time it credits bytes the fused step never moves, so it is a
    # method-equivalent rate, not an HBM rate.
    method_bytes = sum(sum(algorithmic_bytes(g.S, g.V, g.F, n, False).values()) for g in groups)
    method_gbps = method_bytes / (ms_step * 1e-3) / 1e9
    rec = {
        "value": V / (ms_step * 1e-3),
        "unit": "params/s",
        "ms_per_step": ms_step,
        "config": {"workload": cfg.name, "world": n, "rank": rank, "groups": len(groups),
                   "params_per_rank": V, "align_elems": args.align,
                   "step": ("per group: fused reduce+adamw+pack -> unpack" if fused else
                            "reduce per group -> one adamw+copy-in launch over every group -> "
                            "unpack per group" if aci else
                            "reduce per group -> one adamw launch over every group -> one "
                            "copy-in launch over every group -> unpack per group"
                            if args.group_set else "per group: reduce -> adamw -> pack -> unpack"),
                   "io": "fp32 master/m/v shards, bf16 [N,S] grads and all-gather buffers"},
        "effective_GBps": eff_gbps,
        "hbm_frac": eff_gbps / HBM_PEAK_GBPS,
        "frac_of_copy_ceiling": frac(eff_gbps, copy_gbps),
        "step_algorithmic_bytes": step_bytes,
        "bytes_note": ("bytes the step's kernels must move once each (fused step "
                       "(2N+24)V+2S, copy-out 4F per group); hbm_frac = these / time / 8 TB/s"
                       if fused else "bytes of the separate kernels (reduce (2N+4)V, AdamW "
                       "and copy-in fused 28V+2S, copy-out 4F per group) / time / 8 TB/s" if aci
                       else "bytes of the four separate kernels (reduce (2N+4)V, AdamW "
                       "28V, copy-in 4V+2S, copy-out 4F per group) / time / 8 TB/s"),
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "step_ms": {"median": _pct(step_ms, 50), "p10": _pct(step_ms, 10), "p90": _pct(step_ms, 90)},
        "method_equivalent": {
            "bytes_per_step": method_bytes, "GBps": method_gbps,
            "frac_of_peak": method_gbps / HBM_PEAK_GBPS,
            "note": "separate-pass bytes over this step's time; counts bytes a fused step never "
                    "moves, so it is not an HBM rate"},
        "roofline": {"bound": "hbm", "kernel": KERNEL_NAMES[dominant],
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(cfg.name, rank, args.align, dominant),
                     "traffic_source": TRAFFIC_SOURCE,
                     "frac_of_copy_ceiling": frac(achieved, copy_gbps),
                     "avg_launch_ms": dom_avg_ms, "launches": dom_launches,
                     "algorithmic_bytes_per_launch": dom_bytes_per_launch,
                     "timing": ("HIP events around its one launch per step"
                                if dominant in one_launch else
                                "HIP events around one launch per group") +
                               " on the step's stream, inside the timed steps"},
        "kernels": kernels,
    }
    if graph_rec is not None:
        rec["graph_replay"] = graph_rec
    if per.get("unpack"):
        # derived, not timed: with reshard-after-forward a step all-gathers
        # every group twice (forward and backward), so one more copy-out per
        # group is added at its measured per-step time
        t2 = ms_step + per["unpack"]
        rec["two_allgather_variant"] = {
            "derived": True, "ms_per_step": t2, "params_per_s": V / (t2 * 1e-3),
            "effective_GBps": (step_bytes + byts["unpack"]) / (t2 * 1e-3) / 1e9,
            "hbm_frac": (step_bytes + byts["unpack"]) / (t2 * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    if not args.no_next:
        rec["next_kernels"] = measure_next(groups, n, rs_arena[0], full_arena, stream,
                                           max(1, args.breakdown_steps),
                                           with_set=not args.no_next_group_set)
    if gset is not None:
        capi.fsdp_group_set_destroy(gset)
    for g in groups:
        g.close()
    del groups, full_arena, rs_arena, ag_arena, execute, arena
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(cfg, rank)
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only: the collectives between "
                          "ranks are not part of it, so --gpus must be 1"}))
        sys.exit(2)
    import torch

    if args.copy_calibration:
        print(json.dumps(copy_calibration()), flush=True)
        return

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    ceiling = None if args.no_copy_ceiling else measure_copy_ceiling(dev, stream)
    if ceiling:
        print(f"bench: copy ceiling {ceiling['GBps']:.0f} GB/s", file=sys.stderr, flush=True)
    torch.cuda.empty_cache()
    copy_gbps = ceiling["GBps"] if ceiling else None
    head = run_workload(args.config, args, dev, copy_gbps)
    out = {
        "metric": METRIC,
        "value": head.pop("value"),
        "unit": head.pop("unit"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": head.pop("config"),
    }
    out.update(head)
    out["copy_ceiling"] = ceiling
    if not args.no_references:
        out["pattern_references"] = measure_pattern_references(dev, stream)
    also = []
    for c in args.also:
        also.append(run_workload(c, args, dev, copy_gbps))
    if also:
        out["also"] = also
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
