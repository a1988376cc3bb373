"""Build libgemm.so in-tree with hipcc for gfx950 (no JIT, no torch extension).

Every translation unit is compiled with
  -Xclang -target-feature -Xclang -packed-fp32-ops
which keeps the compiler from forming packed fp32 instructions on its own; the host
pass prints a harmless "not a recognized feature" warning for it.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "lib", "libgemm.so")

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "libgemm.cpp")]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = ["hipcc", *COMMON, *extra, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    noise = [l for l in (r.stderr or "").splitlines()
             if l.strip() and "packed-fp32-ops" not in l]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(extra=(), jobs: int = 8, verbose: bool = True) -> str:
    """Compile every HIP source and link libgemm.so (always rebuilds).  With the
    environment variable GEMM_ALL_TILES=1 the matrix-core variants that lose on every
    measured workload are built too (they are left out of the default library)."""
    extra = list(extra)
    if os.environ.get("GEMM_ALL_TILES", "0") not in ("", "0"):
        extra.append("-DGEMM_ALL_TILES")
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    # the matrix-core units take longest: start them first
    srcs = sorted(sources(), key=lambda f: (not os.path.basename(f).startswith("kernels_mfma_"), f))
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
