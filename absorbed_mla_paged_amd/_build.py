"""Build libmla_decode.so (gfx950) in-tree with hipcc.

    python -m absorbed_mla_paged_amd._build

The library lands next to this file, where the binding looks for it. The
flags keep every kernel gfx950-only and turn off packed fp32 arithmetic.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla_decode.so")
SOURCES = ["plan.cpp", "partition.hip", "partition_wide.hip", "reduce.hip"]
HEADERS = ["internal.h", "device_common.h", "partition_common.h"]


def hipcc() -> str:
    root = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(root, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def command(out: str = LIB, extra=()) -> list[str]:
    return [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-kernarg-preload-count=16",
            "-I", os.path.join(HERE, "..", "include"),
            *extra, "-o", out, *[os.path.join(CSRC, s) for s in SOURCES]]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
