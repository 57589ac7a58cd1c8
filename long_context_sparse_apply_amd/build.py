"""Build the gfx950 shared library in-tree with hipcc.

    python long_context_sparse_apply_amd/build.py      (or __graft_entry__.build())

Each source compiles to an object under ``_build/`` (in parallel), then one
link produces ``long_context_sparse_apply_amd/libsa_mi355x.so``.  A build
always recompiles every source.
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
LIB_NAME = "libsa_mi355x.so"
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm required to build)")
    return path


def _compile(src: str, obj: str) -> str:
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build_library(out_dir: str = HERE, jobs: int | None = None, verbose: bool = True) -> str:
    bdir = os.path.join(ROOT, "_build", "sa")
    os.makedirs(bdir, exist_ok=True)
    sources = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    objs = []
    jobs = jobs or min(8, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = {}
        for s in sources:
            obj = os.path.join(bdir, os.path.splitext(s)[0] + ".o")
            futs[ex.submit(_compile, os.path.join(CSRC, s), obj)] = s
            objs.append(obj)
        for f in cf.as_completed(futs):
            f.result()
            if verbose:
                print(f"  compiled {futs[f]}", flush=True)
    lib = os.path.join(out_dir, LIB_NAME)
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}", flush=True)
    return lib


if __name__ == "__main__":
    build_library()
    sys.exit(0)
