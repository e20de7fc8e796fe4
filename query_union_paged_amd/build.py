"""Build libpageweaver.so (gfx950) in-tree with hipcc.

Usage: python -m query_union_paged_amd.build   (or build() from Python)

Every HIP source is compiled to its own object (in parallel, under
query_union_paged_amd/_build/), then the objects are linked into one shared
library.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpageweaver.so")
OBJDIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMPILE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # keep the device compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
LINK_FLAGS = ["--offload-arch=gfx950", "-shared", "-fPIC"]

# Per-source compiler options.  The search kernel is a chain of dependent
# steps at two waves per SIMD: the ILP-first machine scheduler (more registers,
# the same occupancy at the windows' count) runs it about 10 % faster; every
# other source keeps the default scheduler, which is the fastest for the
# attention.
PER_FILE = {
    "group.hip": ["-mllvm", "--amdgpu-sched-strategy=max-ilp"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    return res.returncode, msgs


def build(verbose: bool = False, extra=None, out: str = LIB) -> str:
    """Compile every HIP source and link them into one shared library
    (`extra`: more hipcc flags for every source)."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = []
    for src in sources():
        obj = os.path.join(OBJDIR, os.path.basename(src)[:-4] + ".o")
        cmd = [HIPCC, *COMPILE_FLAGS, *PER_FILE.get(os.path.basename(src), []), *(extra or []),
               "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        jobs.append((cmd, obj))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as pool:
        results = list(pool.map(lambda j: _run(j[0]), jobs))
    for (cmd, _), (rc, msgs) in zip(jobs, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
        if verbose and msgs:
            print("\n".join(msgs))
    link = [HIPCC, *LINK_FLAGS, *[o for _, o in jobs], "-o", out + ".tmp"]
    if verbose:
        print(" ".join(link), flush=True)
    rc, msgs = _run(link)
    if rc != 0:
        raise RuntimeError("hipcc link failed:\n" + "\n".join(msgs))
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
