"""Build libkvz.so (the C-ABI library) in-tree with hipcc for gfx950.

Each source is compiled to its own object in parallel (under _build/, next to this file), then
the objects are linked into the shared library.  Every call compiles every source again.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvz.so")
SOURCES = ["api.hip", "pool.hip", "codec.hip", "attention.hip", "measure.hip", "gaac.hip", "fp8.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # no packed fp32 instructions are generated (the vector units handle fp32 one lane-op
    # at a time); hipcc's host pass warns that it does not know the feature
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str) -> tuple[str, subprocess.CompletedProcess]:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", "-o", obj, os.path.join(CSRC, src)]
    return obj, subprocess.run(cmd, capture_output=True, text=True)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = max(1, min(len(SOURCES), os.cpu_count() or 1, 8))
    if verbose:
        print(f"{HIPCC} {' '.join(FLAGS)} -c <each of {', '.join(SOURCES)}> ({jobs} at a time)",
              flush=True)
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    failed = [(o, r) for o, r in results if r.returncode != 0]
    for _, r in failed:
        sys.stderr.write(r.stdout + r.stderr)
    if failed:
        raise RuntimeError("hipcc failed compiling " + ", ".join(os.path.basename(o) for o, _ in failed))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *[o for o, _ in results]]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError("hipcc failed linking libkvz.so")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
