"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU).

tests/native/host_harness.cpp drives the real planner, C ABI, device-table
management, multi-group executor, FSDP_FAULT hook, reshard planner and host
AdamW, compiled with g++ -fsanitize=address,undefined against a host-memory
stand-in for the HIP runtime and launch stand-ins that read the first and last
element of every range each uploaded tile names.  Every tensor is its own
exact-size allocation, so a tile reaching outside its tensor is an ASan
report; the harness also checks that every call writes each element of its
outputs exactly once, and that injected launch failures reach the caller as
FSDP_E_HIP with nothing launched after them.
"""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT
from workloads import configs

NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "sharded_shard_amd", "csrc")
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")

# Ragged shape sets (the GPU parity cases), the MLP probe, a Llama block at
# an eighth of the d = 4096 widths (same layout, N = 8), and the ragged MoE
# root group at rank 5 (full size: an odd segment, short last chunk).
RAGGED = [
    ("ragged-n6", [(1000, 70), (333,), (77, 129), (1, 2048), (1,), (64, 2048)], 6),
    ("empty-rows", [(5, 3), (0, 4), (7,), (1, 5), (13, 2)], 4),
    ("more-ranks", [(6, 3), (17,)], 8),
    ("n1", [(9, 7), (4097,)], 1),
    ("tiles", [(300, 1000), (4096, 33), (70001,)], 8),
    ("odd-n12", [(1000, 37), (4097,), (129, 3), (25, 8)], 12),
    ("odd-n64", [(700, 9), (129,), (64, 33)], 64),
    ("wide-n64", [(5000, 24), (64, 72), (129, 8), (1, 8)], 64),
]


def _cols(shape):
    c = 1
    for d in shape[1:]:
        c *= d
    return c


def _line(name, shapes, n, r, align):
    rc = " ".join(f"{s[0]} {_cols(s)}" for s in shapes)
    return f"{name}/r{r}/a{align} {n} {r} {align} {len(shapes)} {rc}"


def _workloads():
    lines = []
    for name, shapes, n in RAGGED:
        for r in sorted({0, n - 1}):
            for align in (1, 8):
                lines.append(_line(name, shapes, n, r, align))
    small_block = configs.llama_block("layers.0", 512, 1792)
    for r in (0, 7):
        for align in (1, 8):
            lines.append(_line("llama-block-d512", [p.shape for p in small_block.params], 8, r,
                               align))
    for ci, gi, ranks in ((0, 0, (0, 1)), (3, 1, (5,))):
        cfg = configs.get(ci)
        shapes = [p.shape for p in cfg.groups[gi].params]
        for r in ranks:
            lines.append(_line(f"c{ci}-{cfg.groups[gi].name}", shapes, cfg.world, r, 1))
    return lines


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(os.path.join(ROCM_INCLUDE, "hip")):
        pytest.skip("needs g++ and the HIP headers")
    out = str(tmp_path_factory.mktemp("asan") / "host_harness")
    srcs = [os.path.join(NATIVE, f) for f in ("host_harness.cpp", "fake_hip.cpp", "fake_launch.cpp")]
    srcs += [os.path.join(CSRC, f) for f in ("capi.cpp", "plan.cpp", "reshard.cpp", "host_adamw.cpp")]
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-ffp-contract=off", "-D__HIP_PLATFORM_AMD__", "-I" + ROCM_INCLUDE,
           "-Wall", "-Wextra", "-Wno-unused-parameter", *srcs, "-pthread", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    return out


def test_host_code_under_asan_and_ubsan(harness):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("FSDP_FAULT", None)
    r = subprocess.run([harness], input="\n".join(_workloads()) + "\n", capture_output=True,
                       text=True, timeout=900, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
    assert "ALL OK" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
