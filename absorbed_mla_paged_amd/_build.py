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
SOURCES = ["plan.cpp", "partition.hip", "partition_wide.hip", "reduce.hip", "project.hip",
           "noalloc.hip", "stream_read.hip", "copy_probe.hip"]
HEADERS = ["internal.h", "device_common.h", "partition_common.h", "fused_common.h"]
# Per-source extra flags (none needed at present).
EXTRA: dict[str, list[str]] = {}


def hipcc() -> str:
    root = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(root, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-kernarg-preload-count=16"]


def compile_command(src: str, obj: str) -> list[str]:
    return [hipcc(), *COMMON, *EXTRA.get(src, []), "-I", os.path.join(HERE, "..", "include"),
            "-c", os.path.join(CSRC, src), "-o", obj]


def link_command(objs, out: str) -> list[str]:
    return [hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", out]


def _run(cmd, verbose):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd[:3])} ... failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)


def build(verbose: bool = False) -> str:
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    with tempfile.TemporaryDirectory(prefix="mla_build_") as tmpd:
        objs = [os.path.join(tmpd, s + ".o") for s in SOURCES]
        with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            for f in [ex.submit(_run, compile_command(s, o), verbose)
                      for s, o in zip(SOURCES, objs)]:
                f.result()
        tmp = LIB + ".tmp"
        _run(link_command(objs, tmp), verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
