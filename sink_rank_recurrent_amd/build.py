"""Build libseed.so (the gfx950 HIP library) in-tree with hipcc.

    python -m sink_rank_recurrent_amd.build [--incremental]

Compiles every source under csrc/ for gfx950 (in parallel) into
_build/ at the repository root and links sink_rank_recurrent_amd/libseed.so.
Always rebuilds.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libseed.so")

ARCH = "gfx950"
CXXFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libseed.so")
    return exe


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *CXXFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _local_includes(path: str, seen: set) -> set:
    """The repository headers `path` includes, directly or not."""
    import re
    for name in re.findall(r'^\s*#include\s+"([^"]+)"', open(path).read(), flags=re.M):
        dep = os.path.normpath(os.path.join(os.path.dirname(path), name))
        if os.path.exists(dep) and dep not in seen:
            seen.add(dep)
            _local_includes(dep, seen)
    return seen


def _stale(src: str) -> bool:
    """True if src's object is missing or older than src or a header it includes."""
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(f) > t for f in [src, *_local_includes(src, set())])


def build(verbose: bool = True, incremental: bool = False) -> str:
    """Compile every source (incremental=True: only those whose object is
    older than the source or any header) and link libseed.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))
    todo = [s for s in srcs if _stale(s)] if incremental else srcs
    jobs = max(1, min(len(todo), 16, os.cpu_count() or 1))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(_compile, todo))
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in srcs]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources ({len(todo)} compiled)")
    return LIB


if __name__ == "__main__":
    build(incremental="--incremental" in sys.argv[1:])
    sys.exit(0)
