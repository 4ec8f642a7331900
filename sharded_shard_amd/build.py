"""Build the sharded-step library for gfx950 in-tree.

    python -m sharded_shard_amd.build          # writes sharded_shard_amd/lib/libfsdp_shard.so

hipcc cross-compiles for gfx950 without a GPU.  Device code is built with
fp-contraction off and correctly rounded fp32 divide and square root (the
reduction and AdamW must round every operation once), and with packed-fp32
instructions disabled.
"""
from __future__ import annotations

import os
import shlex
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "lib")
LIB = os.path.join(OUT_DIR, "libfsdp_shard.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter"]
DEVICE = [f"--offload-arch={ARCH}", "-ffp-contract=off",
          "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
          "-fno-gpu-rdc", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

SOURCES = [
    ("plan.cpp", ["-x", "c++"]),
    ("capi.cpp", ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include")]),
    ("host_adamw.cpp", ["-x", "c++", "-ffp-contract=off", "-fno-fast-math", "-pthread"]),
    ("reshard.cpp", ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include")]),
    ("copy.hip", ["-x", "hip"] + DEVICE),
    ("pack.hip", ["-x", "hip"] + DEVICE),
    ("reduce.hip", ["-x", "hip"] + DEVICE),
    ("step.hip", ["-x", "hip"] + DEVICE),
]
KERNEL_SOURCES = [n for n, _ in SOURCES if n.endswith(".hip")]


def kernel_sources_sha256() -> str:
    """sha256 over the device sources (every .hip file and the headers they
    include), in name order: identifies the kernels a measurement was taken
    on."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(KERNEL_SOURCES + ["device.hpp", "rows.hpp", "launch.hpp", "plan.hpp"]):
        h.update(name.encode() + b"\0")
        with open(os.path.join(SRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _run(cmd, verbose):
    if verbose:
        print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {cmd[0]} ... {cmd[-1]}")
    return r


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    """Compile every source and link the shared library; returns its path.

    extra_flags (e.g. -DFSDP_TILE_UNPACK=65536) and out select a variant build.
    """
    out_dir = os.path.dirname(os.path.abspath(out))
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for name, flags in SOURCES:
        src = os.path.join(SRC, name)
        obj = os.path.join(out_dir, name + ".o")
        _run([HIPCC, *COMMON, *flags, *extra_flags, "-c", src, "-o", obj], verbose)
        objs.append(obj)
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    for o in objs:
        os.remove(o)
    return out


def emit_asm(out_dir: str) -> list:
    """Write the gfx950 assembly of every kernel source into out_dir (for
    inspecting the ISA); returns the paths."""
    os.makedirs(out_dir, exist_ok=True)
    paths = []
    for name in KERNEL_SOURCES:
        path = os.path.join(out_dir, name.replace(".hip", ".s"))
        _run([HIPCC, *COMMON, "-x", "hip", *DEVICE, "--cuda-device-only", "-S",
              os.path.join(SRC, name), "-o", path], False)
        paths.append(path)
    return paths


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
