"""Build libmuonh.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m matrix_orthogonalizing_optimizer_momentum_amd.build

compiles every csrc/*.hip with hipcc --offload-arch=gfx950, the host-only
planner with g++, and links them into libmuonh.so next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libmuonh.so")
BUILD_DIR = os.path.join(ROOT, "_build", "muonh")

ARCH = os.environ.get("MUONH_ARCH", "gfx950")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 ALU ops off: scalar / float2 code stays unpacked
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass of hipcc does not know the packed-fp32 feature: drop that noise
    lines = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def sources():
    hip = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".cpp"))
    return hip, cpp


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile and link; returns the path of the built library."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    hip, cpp = sources()
    cmds = []
    objs = []
    for src in hip:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmds.append([HIPCC, *HIP_FLAGS, "-c", src, "-o", obj])
        objs.append(obj)
    for src in cpp:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmds.append(["g++", *HOST_FLAGS, "-c", src, "-o", obj])
        objs.append(obj)
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = OUT + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, OUT)
    return OUT


def clean():
    shutil.rmtree(BUILD_DIR, ignore_errors=True)
    if os.path.exists(OUT):
        os.remove(OUT)


if __name__ == "__main__":
    p = build(verbose="-v" in sys.argv)
    print(p)
