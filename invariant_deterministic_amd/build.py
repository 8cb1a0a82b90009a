"""Build libbi.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

Usage: ``python -m invariant_deterministic_amd.build``.  Every call compiles
from source: each ``csrc/*.hip`` is compiled to an object under ``_build/``
in parallel, then linked into ``invariant_deterministic_amd/libbi.so``.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libbi.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
# -ffp-contract=off: no fused multiply-add formed behind the source's back, so
# every fp32 operation rounds exactly where the source says.
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-ffp-contract=off", f"-I{INCLUDE}", f"-I{CSRC}"]


# Per-source additions.  gemm.hip: keep matrix-core accumulators in ordinary
# VGPRs whenever they fit.  Left to its heuristic, the compiler puts the 4x4
# accumulator blocks of the 4-wavefront kernels in AGPRs and shuffles them
# between register files inside the K loop; with them in VGPRs those kernels
# measured 2-20 % faster with the same bits (the ping-pong kernel already
# compiles that way).
EXTRA_FLAGS = {"gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    extra = EXTRA_FLAGS.get(os.path.basename(src), [])
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("packed-fp32-ops", "hip-link")
    err = "\n".join(ln for ln in r.stderr.splitlines() if not any(n in ln for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int | None = None) -> str:
    """Compile every HIP source and link libbi.so; return its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2) - 1), 16)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
