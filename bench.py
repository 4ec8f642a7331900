"""Benchmark of one rank's FSDP2 sharded step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

A step is one pass of the whole per-rank hot path over every parameter group
of the workload: for each group, reduce (bf16 [N, S] gradient contributions
-> fp32 mean) -> AdamW (fp32 master, m, v) -> pack (bf16 copy-in, written in
place into row `rank` of the all-gather buffer) -> unpack (bf16 [N, S] ->
full parameters).  Other ranks' rows are synthetic data already in HBM; the
collectives themselves are not part of the step.  Inputs are resident in HBM
before the timed region starts.

Prints one JSON line: params/s of this rank's shard (value), effective HBM
GB/s (algorithmic bytes / time) and its fraction of the 8 TB/s HBM peak, the
roofline of the dominant kernel (copy-out) measured with HIP events around its
launches inside the timed region, and the CPU oracle timed on a bounded sample
of the same workload.
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


def algorithmic_bytes(S, V, F, N):
    """Bytes each kernel must move once per group (see the design notes).

    pack: read 4V fp32, write 2S bf16; unpack: read 2F + write 2F;
    reduce: read 2NV bf16 + write 4V fp32; AdamW: read p, g, m, v (16V) +
    write p, m, v (12V).
    """
    return {"reduce": 2 * N * V + 4 * V, "adamw": 28 * V, "pack": 4 * V + 2 * S,
            "unpack": 4 * F}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4])
    ap.add_argument("--rank", type=int, default=None, help="simulated rank (default: the config's)")
    ap.add_argument("--align", type=int, default=1, choices=[1, 8])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown-steps", type=int, default=3,
                    help="extra untimed steps with events around every kernel")
    return ap.parse_args()


def cpu_baseline(cfg, rank, budget_s=30.0):
    """Time the CPU oracle on one block group plus the root group, one step."""
    import numpy as np
    import torch

    from oracle import fsdp as O
    from workloads import synth

    n = cfg.world
    hp = vars(cfg.hp)
    sample = [cfg.groups[0]] + ([cfg.groups[-1]] if len(cfg.groups) > 1 else [])
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
        if total_t > budget_s:
            break
    return {
        "value": total_v / total_t,
        "unit": "params/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"one step of groups {names} of {cfg.name}, rank {rank}: {total_v} params "
                   f"in {total_t:.2f} s (NumPy, single thread; host has {os.cpu_count()} cpus, "
                   f"affinity {len(os.sched_getaffinity(0))})"),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only: the collectives between "
                          "ranks are out of scope, so --gpus must be 1"}))
        sys.exit(2)
    import torch

    from sharded_shard_amd.group import ShardedGroup
    from workloads import configs, synth

    cfg = configs.get(args.config)
    n = cfg.world
    rank = cfg.timing_rank if args.rank is None else args.rank
    hp = vars(cfg.hp)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
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
        synth.fill_normal_bf16_bits_(rs_arena[b], cfg.grad_std, ("bench-rs", args.config, b))
        synth.fill_normal_bf16_bits_(ag_arena[b], cfg.master_std, ("bench-ag", args.config, b))
    for gi, g in enumerate(groups):
        g.full_flat = full_arena
        g.allocate(full=False)
        synth.fill_normal_f32_(g.master_flat, cfg.master_std, ("bench-master", args.config, gi))
        g.bind()
    torch.cuda.synchronize()
    print("bench: state resident", file=sys.stderr, flush=True)

    V = sum(g.V for g in groups)
    byts = {k: 0 for k in ("reduce", "adamw", "pack", "unpack")}
    for g in groups:
        for k, b in algorithmic_bytes(g.S, g.V, g.F, n).items():
            byts[k] += b
    step_bytes = sum(byts.values())

    stream = torch.cuda.current_stream()
    step_counter = [0]

    def step(events=None, all_events=None):
        step_counter[0] += 1
        t = step_counter[0]
        for gi, g in enumerate(groups):
            rs = rs_arena[gi & 1][:n * g.S]
            ag = ag_arena[gi & 1][:n * g.S]
            if all_events is not None:
                e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
                e[0].record(stream)
                g.reduce(rs, stream)
                e[1].record(stream)
                g.adamw(t, stream=stream, **hp)
                e[2].record(stream)
                g.pack(ag[rank * g.S:(rank + 1) * g.S], stream)
                e[3].record(stream)
                g.unpack(ag, stream)
                e[4].record(stream)
                all_events.append(e)
                continue
            g.reduce(rs, stream)
            g.adamw(t, stream=stream, **hp)
            g.pack(ag[rank * g.S:(rank + 1) * g.S], stream)
            if events is not None:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                g.unpack(ag, stream)
                b.record(stream)
                events.append((a, b))
            else:
                g.unpack(ag, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"bench: {args.warmup} warmup steps done", file=sys.stderr, flush=True)

    unpack_events = []
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step(events=unpack_events)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    print(f"bench: {args.steps} timed steps, {ms_step:.3f} ms/step", file=sys.stderr, flush=True)
    unpack_ms = sum(a.elapsed_time(b) for a, b in unpack_events)
    unpack_launches = len(unpack_events)
    unpack_avg_ms = unpack_ms / max(1, unpack_launches)
    unpack_bytes_per_launch = byts["unpack"] / len(groups)
    achieved = unpack_bytes_per_launch / (unpack_avg_ms * 1e-3) / 1e9

    # per-kernel breakdown (untimed steps, events around every launch)
    per = {k: 0.0 for k in ("reduce", "adamw", "pack", "unpack")}
    if args.breakdown_steps > 0:
        evs = []
        for _ in range(args.breakdown_steps):
            step(all_events=evs)
        torch.cuda.synchronize()
        for e in evs:
            for k, (i, j) in zip(("reduce", "adamw", "pack", "unpack"), ((0, 1), (1, 2), (2, 3), (3, 4))):
                per[k] += e[i].elapsed_time(e[j])
        per = {k: v / args.breakdown_steps for k, v in per.items()}
    kernels = {k: {"ms_per_step": round(per[k], 4),
                   "algorithmic_GB_per_step": round(byts[k] / 1e9, 4),
                   "GBps": round(byts[k] / (per[k] * 1e-3) / 1e9, 1) if per[k] else None,
                   "hbm_frac": round(byts[k] / (per[k] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4) if per[k] else None}
               for k in per}

    eff_gbps = step_bytes / (ms_step * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": V / (ms_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "world": n, "rank": rank, "groups": len(groups),
                   "params_per_rank": V, "align_elems": args.align,
                   "step": "per group: reduce -> adamw -> pack -> unpack",
                   "io": "fp32 master/m/v/grad shards, bf16 [N,S] grads and all-gather buffers"},
        "effective_GBps": eff_gbps,
        "hbm_frac": eff_gbps / HBM_PEAK_GBPS,
        "step_algorithmic_bytes": step_bytes,
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "roofline": {"bound": "hbm", "kernel": "unpack_kernel (copy-out)",
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                     "avg_launch_ms": unpack_avg_ms, "launches": unpack_launches,
                     "algorithmic_bytes_per_launch": unpack_bytes_per_launch},
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, rank)
    for g in groups:
        g.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
