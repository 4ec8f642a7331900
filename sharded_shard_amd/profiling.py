"""Summaries of rocprofv3 runs of the sharded-step kernels.

    python -m sharded_shard_amd.profiling <rocprof dir> <profiles dir>

The rocprof directory holds, per workload tag (c1, c2, c3, c4; c2u/c4u for
the separate kernels per group, c2s/c4s for them through a group set and
c2f/c4f for a group set with AdamW and the copy-in fused), the output of

* ``<tag>_trace``: ``rocprofv3 --kernel-trace --stats -T -f csv`` of bench.py
  (kernel durations, averaged per kernel name);
* ``<tag>_FETCH`` / ``<tag>_WRITE``: ``--pmc FETCH_SIZE`` and ``--pmc
  WRITE_SIZE`` (KiB the L2 requested from and wrote to the memory fabric);
* ``<tag>_RD`` / ``<tag>_WR``: ``--pmc TCC_EA0_RDREQ_32B_sum
  TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum TCC_EA0_RDREQ_sum`` and
  ``--pmc TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_64B_sum`` (memory requests by size),

and ``cal_*`` the same counters of ``bench.py --copy-calibration`` (torch's
copy kernel: 2 GiB read and 2 GiB written per launch, known bytes).  Fetched
bytes come two ways: FETCH_SIZE scaled by what it reads for the calibration
copy, and the request sizes summed (32, 64 and 128 bytes, the figure
``pmc_traffic.json`` keeps: it needs no fitted scale); written bytes from
WRITE_SIZE and from the write requests (64 bytes, the rest 32).  Writes one
markdown summary per workload and ``pmc_traffic.json`` (HBM bytes per launch
per kernel, keyed by the kernel sources' sha256) into the profiles directory.
These counters count the L2's requests to the fabric, so reads served by the
256 MB MALL are included: they bound DRAM traffic from above and show
re-reads, not cache hits.
"""
from __future__ import annotations

import csv
import glob
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
CAL_BYTES = 2 * (1 << 30)            # bytes read (and written) per calibration launch

WORKLOADS = {   # tag: (config, label, file stem)
    "c1": (1, "one Llama block d=4096, N=8, rank 0", "llama_block_n8"),
    "c2": (2, "7B-shaped, 33 groups, N=8, rank 0", "llama7b_n8"),
    "c3": (3, "ragged MoE, 2 groups, N=6, rank 5", "moe_ragged_n6"),
    "c4": (4, "70B-shaped, 81 groups, N=64, rank 0", "llama70b_n64"),
}
# separate-kernel traces: tag -> (workload tag, bench options, group set)
SEPARATE = {"c2u": ("c2", "--unfused", False), "c4u": ("c4", "--unfused", False),
            "c2s": ("c2", "--group-set", True), "c4s": ("c4", "--group-set", True),
            "c2f": ("c2", "--group-set-fused", True), "c4f": ("c4", "--group-set-fused", True)}
# kernels a group set launches once per step over every group: one launch
# moves the bytes of all groups
SET_KERNELS = ("adamw_kernel", "pack_kernel", "adamw_pack_kernel")

# kernel name -> algorithmic bytes of one launch for a group (S, V, F, N)
ALG = {
    "step_kernel_wide": lambda S, V, F, N: 2 * N * V + 24 * V + 2 * S,
    "step_kernel_aligned": lambda S, V, F, N: 2 * N * V + 24 * V + 2 * S,
    "step_kernel": lambda S, V, F, N: 2 * N * V + 24 * V + 2 * S,
    "unpack_kernel": lambda S, V, F, N: 4 * F,
    "reduce_kernel": lambda S, V, F, N: 2 * N * V + 4 * V,
    "adamw_kernel": lambda S, V, F, N: 28 * V,
    "adamw_pack_kernel": lambda S, V, F, N: 28 * V + 2 * S,
    "pack_kernel": lambda S, V, F, N: 4 * V + 2 * S,
    "rspack_bf16_kernel": lambda S, V, F, N: 2 * F + 2 * N * S,
    "rspack_f32_kernel": lambda S, V, F, N: 2 * F + 4 * N * S,
    "reduce_f32_kernel": lambda S, V, F, N: 4 * N * V + 4 * V,
    "pack_fp8_kernel": lambda S, V, F, N: 4 * V + S,
    "unpack_fp8_kernel": lambda S, V, F, N: 2 * F,
    "accumulate_kernel": lambda S, V, F, N: 10 * F,
    "rspack_acc_kernel": lambda S, V, F, N: 4 * F + 4 * N * S,
}


def _one(pattern):
    files = glob.glob(pattern, recursive=True)
    if len(files) != 1:
        raise FileNotFoundError(f"{pattern}: {files}")
    return files[0]


def group_sizes(cfg_index):
    """(S, V, F) of every group at the config's timing rank, from the C
    planner (needs no GPU)."""
    from sharded_shard_amd import capi
    from workloads import configs
    cfg = configs.get(cfg_index)
    out = []
    for g in cfg.groups:
        rows = [p.rows for p in g.params]
        cols = [p.cols for p in g.params]
        plan = capi.fsdp_plan_create(rows, cols, cfg.world, cfg.timing_rank, 1)
        try:
            info = capi.fsdp_plan_info(plan)
            out.append((info.S, info.V, info.F))
        finally:
            capi.fsdp_plan_destroy(plan)
    return cfg, out


def alg_bytes_per_launch(cfg_index, kernel):
    """Average algorithmic bytes of one launch of `kernel` over the groups."""
    cfg, sizes = group_sizes(cfg_index)
    f = ALG[kernel]
    return sum(f(S, V, F, cfg.world) for S, V, F in sizes) / len(sizes)


def kernel_stats(prof, tag):
    rows = list(csv.DictReader(open(_one(f"{prof}/{tag}_trace/**/*kernel_stats.csv"))))
    return {r["Name"]: {"calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                        "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3,
                        "total_us": float(r["TotalDurationNs"]) / 1e3} for r in rows}


def counters(prof, run):
    """Per kernel name: {counter: average value per dispatch}."""
    acc = {}
    for r in csv.DictReader(open(_one(f"{prof}/{run}/**/*counter_collection.csv"))):
        k = acc.setdefault(r["Kernel_Name"], {})
        c = k.setdefault(r["Counter_Name"], [0, 0.0])
        c[0] += 1
        c[1] += float(r["Counter_Value"])
    return {k: {c: v / n for c, (n, v) in cs.items()} for k, cs in acc.items()}


def request_bytes(rd, wr):
    """(read, write) bytes from the request-size counters of one dispatch."""
    read = (32 * rd.get("TCC_EA0_RDREQ_32B_sum", 0.0) + 64 * rd.get("TCC_EA0_RDREQ_64B_sum", 0.0)
            + 128 * rd.get("TCC_EA0_RDREQ_128B_sum", 0.0))
    w64 = wr.get("TCC_EA0_WRREQ_64B_sum", 0.0)
    write = 64 * w64 + 32 * (wr.get("TCC_EA0_WRREQ_sum", 0.0) - w64)
    return read, write


def calibration(prof):
    """Scales of FETCH_SIZE and WRITE_SIZE, and the request-derived bytes,
    for torch's 2 GiB copy (the largest dispatch in the calibration runs)."""
    def big(run):
        cs = counters(prof, run)
        return max(cs.values(), key=lambda d: max(d.values()))
    fetch = big("cal_FETCH")["FETCH_SIZE"] * 1024.0
    write = big("cal_WRITE")["WRITE_SIZE"] * 1024.0
    rd, wr = request_bytes(big("cal_RD"), big("cal_WR"))
    return {"fetch_scale": CAL_BYTES / fetch, "write_scale": CAL_BYTES / write,
            "fetch_size_bytes": fetch, "write_size_bytes": write,
            "request_read_bytes": rd, "request_write_bytes": wr,
            "request_read_ratio": rd / CAL_BYTES, "request_write_ratio": wr / CAL_BYTES}


def _trace_cmd(tag, args):
    return ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -T -f csv "
            f"-d $OUT/{tag}_trace -o {tag} -- python3 $REPO/bench.py {args} "
            "--also none --steps 10 --warmup 2 --breakdown-steps 0 --no-isolated "
            "--no-copy-ceiling --no-cpu-baseline" + (" --no-next" if tag in SEPARATE else "") +
            " --no-references --no-next-group-set --no-graph")


def _pmc_cmd(tag, args, counters_):
    return ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc " + " ".join(counters_) +
            f" -T -f csv -d $OUT/{tag}_<run> -o {tag} -- python3 $REPO/bench.py "
            f"{args} --also none --steps 1 --warmup 1 --breakdown-steps 0 --no-isolated "
            "--no-copy-ceiling --no-cpu-baseline --no-references --no-next-group-set --no-graph")


RD_COUNTERS = ["TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum",
               "TCC_EA0_RDREQ_sum"]
WR_COUNTERS = ["TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum"]


def summarize(prof, out_dir, sha):
    os.makedirs(out_dir, exist_ok=True)
    cal = calibration(prof)
    traffic = {"kernels_source_sha256": sha, "fetch_scale": cal["fetch_scale"],
               "write_scale": cal["write_scale"], "calibration": cal, "workloads": {}}
    files = []
    for tag, (ci, label, stem) in WORKLOADS.items():
        from workloads import configs
        cfg = configs.get(ci)
        stats = kernel_stats(prof, tag)
        cf, cw = counters(prof, f"{tag}_FETCH"), counters(prof, f"{tag}_WRITE")
        crd, cwr = counters(prof, f"{tag}_RD"), counters(prof, f"{tag}_WR")
        args = f"--config {ci}"
        lines = [f"# Kernels of the sharded step -- {cfg.name}, rank {cfg.timing_rank}", "",
                 "REPO is the repository root and OUT the rocprofv3 output directory (the one this "
                 "summary was written from), on the machine with the GPU.", "",
                 "## Kernel trace", "", "```", _trace_cmd(tag, args), "```", "",
                 "Timed steps plus the next-row kernels; no per-kernel event steps, no "
                 "isolated launches.", "",
                 "| kernel | calls | avg us | min us | max us | share of GPU time |",
                 "|---|---|---|---|---|---|"]
        tot = sum(s["total_us"] for s in stats.values())
        for name, s in sorted(stats.items(), key=lambda kv: -kv[1]["total_us"]):
            lines.append(f"| {name} | {s['calls']} | {s['avg_us']:.1f} | {s['min_us']:.1f} | "
                         f"{s['max_us']:.1f} | {100 * s['total_us'] / tot:.1f}% |")
        lines += ["", "## Rates and HBM traffic per launch", "",
                  "```", _pmc_cmd(tag, args, ["FETCH_SIZE"]).replace("<run>", "FETCH"),
                  _pmc_cmd(tag, args, ["WRITE_SIZE"]).replace("<run>", "WRITE"),
                  _pmc_cmd(tag, args, RD_COUNTERS).replace("<run>", "RD"),
                  _pmc_cmd(tag, args, WR_COUNTERS).replace("<run>", "WR"), "```", "",
                  "Algorithmic bytes: the group average of the bytes each launch must move "
                  "once.  Counter traffic per launch (average over dispatches): FETCH_SIZE x "
                  f"{cal['fetch_scale']:.3f} + WRITE_SIZE x {cal['write_scale']:.3f} (scales "
                  "from the calibration copy), and the request-size sum.", "",
                  "| kernel | avg us | algorithmic bytes | GB/s | % of 8 TB/s | traffic "
                  "(FETCH/WRITE) | / algorithmic | traffic (requests) | / algorithmic |",
                  "|---|---|---|---|---|---|---|---|---|"]
        wl = {"config": ci, "rank": cfg.timing_rank, "align_elems": 1, "kernels": {}}
        for name, s in sorted(stats.items(), key=lambda kv: -kv[1]["total_us"]):
            if name not in ALG:
                continue
            alg = alg_bytes_per_launch(ci, name)
            gbps = alg / (s["avg_us"] * 1e-6) / 1e9
            fs = cf.get(name, {}).get("FETCH_SIZE")
            ws = cw.get(name, {}).get("WRITE_SIZE")
            t1 = (fs * 1024 * cal["fetch_scale"] + ws * 1024 * cal["write_scale"]
                  if fs is not None and ws is not None else None)
            t2 = (sum(request_bytes(crd[name], cwr[name]))
                  if name in crd and name in cwr else None)
            lines.append(
                f"| {name} | {s['avg_us']:.1f} | {alg:.4g} | {gbps:.0f} | "
                f"{100 * gbps / HBM_PEAK_GBPS:.1f} | "
                + (f"{t1:.4g} | {t1 / alg:.4f} | " if t1 else "n/a | n/a | ")
                + (f"{t2:.4g} | {t2 / alg:.4f} |" if t2 else "n/a | n/a |"))
            wl["kernels"][name] = {"avg_launch_us": s["avg_us"], "algorithmic_bytes_per_launch": alg,
                                   "GBps": gbps,
                                   "traffic_bytes_per_launch": t2 if t2 is not None else t1,
                                   "traffic_fetch_write_bytes_per_launch": t1}
        traffic["workloads"][cfg.name] = wl
        for sep_tag, (of, opt, is_set) in SEPARATE.items():
            if of != tag or not glob.glob(f"{prof}/{sep_tag}_trace"):
                continue
            sstats = kernel_stats(prof, sep_tag)
            lines += ["", f"## Separate-kernel path ({opt})", "", "```",
                      _trace_cmd(sep_tag, args + " " + opt), "```", ""]
            lines += (["A reduce and a copy-out per group; " + " / ".join(SET_KERNELS) +
                       " run once per step over every group (a group set), so one launch "
                       "moves the bytes of all groups.", ""] if is_set else
                      ["Reduce, AdamW, copy-in and copy-out per group, one group after the "
                       "other.", ""])
            lines += ["| kernel | calls | avg us | algorithmic bytes | GB/s | % of 8 TB/s |",
                      "|---|---|---|---|---|---|"]
            n_groups = len(group_sizes(ci)[1])
            for name, s in sorted(sstats.items(), key=lambda kv: -kv[1]["total_us"]):
                if name not in ALG:
                    continue
                alg = alg_bytes_per_launch(ci, name) * (
                    n_groups if is_set and name in SET_KERNELS else 1)
                gbps = alg / (s["avg_us"] * 1e-6) / 1e9
                lines.append(f"| {name} | {s['calls']} | {s['avg_us']:.1f} | {alg:.4g} | "
                             f"{gbps:.0f} | {100 * gbps / HBM_PEAK_GBPS:.1f} |")
        lines += ["", f"Kernel sources sha256 when measured: `{sha}`", ""]
        path = os.path.join(out_dir, f"kernels_{stem}.md")
        open(path, "w").write("\n".join(lines))
        files.append(path)
    cal_lines = [
        "# HBM byte counters: calibration on a copy of known size", "",
        "REPO is the repository root and OUT the rocprofv3 output directory (the one this "
                 "summary was written from), on the machine with the GPU.", "", "```",
        "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE -T -f csv -d "
        "$OUT/cal_FETCH -o cal -- python3 $REPO/bench.py --copy-calibration",
        "(the same with --pmc WRITE_SIZE, --pmc " + " ".join(RD_COUNTERS) + ", --pmc "
        + " ".join(WR_COUNTERS) + ")", "```", "",
        "torch's copy kernel over 2 GiB: 2,147,483,648 bytes read and written per launch.", "",
        "| counter | per launch | known bytes | scale or ratio |", "|---|---|---|---|",
        f"| FETCH_SIZE x 1024 | {cal['fetch_size_bytes']:.6g} | {CAL_BYTES} | "
        f"scale {cal['fetch_scale']:.4f} |",
        f"| WRITE_SIZE x 1024 | {cal['write_size_bytes']:.6g} | {CAL_BYTES} | "
        f"scale {cal['write_scale']:.4f} |",
        f"| 32 RDREQ_32B + 64 RDREQ_64B + 128 RDREQ_128B | {cal['request_read_bytes']:.6g} | "
        f"{CAL_BYTES} | ratio {cal['request_read_ratio']:.4f} |",
        f"| 64 WRREQ_64B + 32 (WRREQ - WRREQ_64B) | {cal['request_write_bytes']:.6g} | "
        f"{CAL_BYTES} | ratio {cal['request_write_ratio']:.4f} |", ""]
    path = os.path.join(out_dir, "copy_calibration.md")
    open(path, "w").write("\n".join(cal_lines))
    files.append(path)
    path = os.path.join(out_dir, "pmc_traffic.json")
    json.dump(traffic, open(path, "w"), indent=1)
    files.append(path)
    if glob.glob(f"{prof}/cal_LAT"):
        files.append(memory_pressure(prof, out_dir, sha))
    if glob.glob(f"{prof}/default_trace"):
        files.append(default_run(prof, out_dir, sha))
    return files


def default_run(prof, out_dir, sha):
    """The bench's default command under a kernel trace: every kernel's
    average duration, and the headline roofline kernel's trace average beside
    the average the same run's HIP events gave (its JSON line is the last
    line of the run's stdout)."""
    stats = kernel_stats(prof, "default")
    rec = None
    for line in reversed(open(f"{prof}/default_trace.log").read().splitlines()):
        if line.startswith("{"):
            rec = json.loads(line)
            break
    lines = ["# The bench's default command under a kernel trace", "",
             "REPO is the repository root and OUT the rocprofv3 output directory (the one this "
                 "summary was written from), on the machine with the GPU.", "", "```",
             "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -T -f csv -d "
             "$OUT/default_trace -o default -- python3 $REPO/bench.py", "```",
             "", "Both workloads of the default line (the 7B shape, then the 70B shape under "
             "\"also\"), with their per-kernel event steps, isolated launches, next-row "
             "kernels and pattern references; kernels of the same name from the two workloads "
             "share a row.", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for name, st in sorted(stats.items(), key=lambda kv: -kv[1]["total_us"]):
        lines.append(f"| {name} | {st['calls']} | {st['avg_us']:.1f} | {st['min_us']:.1f} | "
                     f"{st['max_us']:.1f} |")
    if rec is not None:
        roof = rec["roofline"]
        # the headline's dominant kernel on aligned rows at 8 ranks
        trace = stats.get("step_kernel_aligned", {}).get("avg_us")
        lines += ["", "## Headline roofline kernel: events against the trace", "",
                  f"Workload: {rec['config']['workload']}; the line's roofline kernel: "
                  f"{roof['kernel']}.", "",
                  "| source | average launch (us) |", "|---|---|",
                  f"| HIP events in the timed steps (roofline.avg_launch_ms) | "
                  f"{1e3 * roof['avg_launch_ms']:.1f} |"]
        if trace is not None:
            lines.append(f"| rocprofv3, step_kernel_aligned, every launch of the run | "
                         f"{trace:.1f} |")
        lines += ["", f"The same run's line: {rec['ms_per_step']:.3f} ms per step, hbm_frac "
                  f"{rec['hbm_frac']:.4f}, roofline.frac {roof['frac']:.4f} (under the "
                  "profiler)."]
    lines += ["", f"Kernel sources sha256 when measured: `{sha}`", ""]
    path = os.path.join(out_dir, "bench_default_trace.md")
    open(path, "w").write("\n".join(lines))
    return path


LAT_COUNTERS = ["TCC_EA0_RDREQ_LEVEL_sum", "TCC_EA0_RDREQ_sum", "TCC_EA0_WRREQ_LEVEL_sum",
                "TCC_EA0_WRREQ_sum"]
STALL_COUNTERS = ["TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum", "TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum",
                  "TCC_CYCLE_sum", "TCC_BUSY_sum"]
# tag: (bench options, kernels to report)
PRESSURE = {
    "c2": ("--config 2", ["step_kernel_aligned", "unpack_kernel"]),
    "c4": ("--config 4", ["step_kernel_wide", "unpack_kernel"]),
    "c4s": ("--config 4 --group-set", ["adamw_kernel", "pack_kernel", "reduce_kernel"]),
}


def memory_pressure(prof, out_dir, sha):
    """Average read and write latency at the L2's memory interface (requests
    in flight summed per cycle / requests, Little's law), reads in flight per
    L2 channel, and the share of L2 cycles the read or write interface was
    out of credits for the memory fabric, per kernel against the calibration
    copy.  The counters are summed over the 16 L2 channels."""
    def copy_kernel(run):      # the 2 GiB copy: the runtime's copy kernel
        cs = counters(prof, run)
        return next(v for k, v in cs.items() if "copyBuffer" in k)

    rows = [("copy (runtime, 2 GiB)", "--copy-calibration",
             {**copy_kernel("cal_LAT"), **copy_kernel("cal_STALL")})]
    for tag, (args, names) in PRESSURE.items():
        lat, st = counters(prof, f"{tag}_LAT"), counters(prof, f"{tag}_STALL")
        for name in names:
            if name in lat and name in st:
                rows.append((name, args, {**lat[name], **st[name]}))
    lines = ["# Memory-side latency and back-pressure per kernel", "",
             "REPO is the repository root and OUT the rocprofv3 output directory (the one this "
                 "summary was written from), on the machine with the GPU.", "", "```"]
    for run, cs in (("LAT", LAT_COUNTERS), ("STALL", STALL_COUNTERS)):
        lines.append("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc " + " ".join(cs) +
                     f" -T -f csv -d $OUT/cal_{run} -o cal -- python3 "
                     "$REPO/bench.py --copy-calibration")
        for tag, (args, _) in PRESSURE.items():
            lines.append("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc " + " ".join(cs) +
                         f" -T -f csv -d $OUT/{tag}_{run} -o {tag} -- python3 "
                         f"$REPO/bench.py {args} --also none --steps 1 --warmup 1 "
                         "--breakdown-steps 0 --no-isolated --no-copy-ceiling --no-cpu-baseline "
                         "--no-references --no-next --no-graph")
    lines += ["```", "",
              "Per dispatch, averaged over the kernel's dispatches: read (write) latency = "
              "TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ (WRREQ), in L2 cycles; reads in flight per "
              "L2 channel = TCC_EA0_RDREQ_LEVEL / TCC_CYCLE (both summed over the channels); "
              "credit stalls = cycles the L2's read (write) interface was out of credits for "
              "the memory fabric / TCC_CYCLE.", "",
              "| kernel | run | read latency | write latency | reads in flight per channel | "
              "read credit stall | write credit stall |",
              "|---|---|---|---|---|---|---|"]
    for name, args, c in rows:
        cyc = c.get("TCC_CYCLE_sum", 0.0) or float("nan")
        rd = c.get("TCC_EA0_RDREQ_sum", 0.0) or float("nan")
        wr = c.get("TCC_EA0_WRREQ_sum", 0.0) or float("nan")
        lines.append(
            f"| {name} | {args} | {c.get('TCC_EA0_RDREQ_LEVEL_sum', 0.0) / rd:.0f} | "
            f"{c.get('TCC_EA0_WRREQ_LEVEL_sum', 0.0) / wr:.0f} | "
            f"{c.get('TCC_EA0_RDREQ_LEVEL_sum', 0.0) / cyc:.1f} | "
            f"{100 * c.get('TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum', 0.0) / cyc:.1f}% | "
            f"{100 * c.get('TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum', 0.0) / cyc:.1f}% |")
    lines += ["", f"Kernel sources sha256 when measured: `{sha}`", ""]
    path = os.path.join(out_dir, "memory_pressure.md")
    open(path, "w").write("\n".join(lines))
    return path


if __name__ == "__main__":
    from sharded_shard_amd.build import kernel_sources_sha256
    for f in summarize(sys.argv[1], sys.argv[2], kernel_sources_sha256()):
        print(f)
