"""Build the gfx950 HIP library ``libjssa.so`` in-tree.

Usage: ``python -m token_level_sparse_dim_amd.build`` (also called by
``__graft_entry__.build()``).  Every source is compiled for gfx950 only, with
packed-fp32 instruction selection disabled, then linked into one shared
library next to this file.
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
LIB = os.path.join(PKG, "libjssa.so")
SOURCES = ["abi.cpp", "append.hip", "score.hip", "select.hip", "attn.hip", "pipeline.hip", "mla.hip", "gather.hip", "vote.hip", "noalloc.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # single-lane claim atomics stay as written: the wave-aggregated rewrite
    # waits for the atomic's result at once, and with it for every load in flight
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in r.stdout.splitlines() if "not a recognized feature" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES]

    def compile_one(i):
        src = os.path.join(CSRC, SOURCES[i])
        cmd = [HIPCC, *CFLAGS, "-x", "hip", "-c", src, "-o", objs[i]]
        out = _run(cmd)
        if verbose and out.strip():
            print(out)

    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        list(ex.map(compile_one, range(len(SOURCES))))
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp,
          "-Wl,-rpath,/opt/rocm/lib"])
    os.replace(tmp, LIB)
    return LIB



def source_digest(name: str) -> str:
    """Short content hash of one kernel source plus the shared headers (used to
    tell whether a stored counter measurement still describes the current kernel)."""
    import hashlib
    h = hashlib.sha256()
    for f in (name, "jssa_device.hpp", "jssa_internal.hpp", "select_common.hpp", "score_core.hpp",
              "attn_core.hpp", "resolve.hpp", "append_core.hpp"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
