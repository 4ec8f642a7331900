"""bench.py's command-line contract and byte accounting (CPU only).

The per-step byte totals are pinned to numbers derived independently from the
workload shapes (pack 4V+2S, unpack 4F, reduce 2NV+4V, AdamW 28V per group,
summed over the groups), not recomputed with the bench's own helper.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import configs  # noqa: E402
from oracle import fsdp as O  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


@pytest.mark.parametrize("args", [("--steps", "0"), ("--warmup", "-1")])
def test_bad_step_counts_are_rejected(args):
    r = _run(*args)
    assert r.returncode == 2
    assert "--steps must be at least 1" in r.stderr


# bytes per step of the separate-kernel path and of the fused path, from the
# shapes (one block d=4096 ff=14336 N=8; 7B shape; 70B shape N=64)
METHOD_BYTES = {1: 2_615_236_608, 2: 86_505_663_488, 4: 465_213_502_208}
FUSED_BYTES = {2: 74_435_105_792, 4: 451_984_682_240}


@pytest.mark.parametrize("ci", sorted(METHOD_BYTES))
def test_byte_accounting_matches_the_shapes(ci):
    cfg = configs.get(ci)
    n, r = cfg.world, cfg.timing_rank
    sep = fused = 0
    for g in cfg.groups:
        p = O.plan([q.shape for q in g.params], n, r)
        sep += sum(bench.algorithmic_bytes(p.S, p.V, p.F, n, False).values())
        fused += sum(bench.algorithmic_bytes(p.S, p.V, p.F, n, True).values())
    assert sep == METHOD_BYTES[ci]
    if ci in FUSED_BYTES:
        assert fused == FUSED_BYTES[ci]
    # fusing saves the gradient's write and re-read and the master's re-read
    assert sep - fused == sum(12 * O.plan([q.shape for q in g.params], n, r).V for g in cfg.groups)


@pytest.mark.parametrize("args,want", [((), [4]), (("--config", "4"), []),
                                       (("--also", "none"), []), (("--also", "3,4"), [3, 4]),
                                       (("--config", "1", "--also", "2"), [2])])
def test_also_workloads(monkeypatch, args, want):
    """The 7B-shaped headline carries the 70B-shaped share by default."""
    monkeypatch.setattr(sys, "argv", ["bench.py", *args])
    assert bench.parse().also == want


@pytest.mark.parametrize("args", [("--also", "2"), ("--also", "7"), ("--also", "x")])
def test_bad_also_is_rejected(args):
    r = _run(*args)
    assert r.returncode == 2
    assert "--also" in r.stderr


def test_traffic_lookup_covers_every_kernel_kind():
    """Every kernel kind the bench can time has a traffic lookup (a number
    from the committed counters or None), for every path."""
    kinds = set()
    for fused, aci in ((True, False), (False, False), (False, True)):
        kinds |= set(bench.algorithmic_bytes(8, 8, 8, 2, fused, aci))
    for cfg in (configs.get(2), configs.get(4)):
        for k in sorted(kinds):
            got = bench.measured_traffic(cfg.name, cfg.timing_rank, 1, k)
            assert got is None or got > 0, (cfg.name, k, got)
            assert k in bench.KERNEL_NAMES
