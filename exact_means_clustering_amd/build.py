"""Build libflashkm.so (the HIP/gfx950 k-means library) in-tree with hipcc.

Each ``csrc/*.hip`` source compiles to an object in parallel under
``_build/``; the objects link into ``libflashkm.so`` next to this file.
Usage: ``python exact_means_clustering_amd/build.py`` (or ``build()``).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libflashkm.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # keep the compiler from forming packed-fp32 instructions (see notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Per-source extra flags.  The assign kernel's running max needs no NaN
# canonicalisation (non-finite inputs give unspecified labels by contract).
EXTRA = {"assign.hip": ["-fno-honor-nans"]}


def _compile(src, obj, verbose):
    cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source for gfx950 and link libflashkm.so; returns its path."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(bdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], verbose), zip(srcs, objs)))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
