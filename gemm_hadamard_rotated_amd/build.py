"""Build libpq1.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m gemm_hadamard_rotated_amd.build

Every HIP translation unit is compiled with hipcc for gfx950 only, then
linked into ``gemm_hadamard_rotated_amd/libpq1.so``.  The measurement
kernels bench.py times beside it (an MFMA loop and a streaming read) go into
a separate ``libpq1_bench.so``, so the library itself holds only the path.
Flags:

* ``-O3``, no fast-math;
* ``-ffp-contract=fast``: the device compiler may fuse multiply-adds.  No
  result of this library is claimed bit-exact where rounding occurs; the
  bit-exact tests use inputs on which every operation is exact;
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed fp32
  (v_pk_*_f32) instructions are generated;
* ``-mllvm -amdgpu-kernarg-preload-count=16``: the hardware places the first
  kernel arguments (up to 14 dwords next to the kernarg pointer) in SGPRs at
  wave launch, so a wave issues its first loads without waiting for scalar
  loads of its arguments (fused decode step on ffn_gate 6.13 -> 5.60 us; the
  rotation, the canonical GEMVs and the embedding lookup 3-9 % faster).  The
  kernels keep the arguments they need first at the front of their parameter
  lists, ahead of any struct (a by-value struct ends the preloaded run).  The
  code object also carries the prologue that loads them itself where the
  firmware does not preload.  ``SOURCE_FLAGS`` adds flags for single files.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpq1.so")
BENCH_LIB = os.path.join(PKG, "libpq1_bench.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "rotate.hip", "gemv.hip", "gemv_packed.hip", "gemm.hip", "gemm_skinny.hip"]
BENCH_SOURCES = ["bench_kernels.hip"]

# gemm_skinny.hip: MFMA results stay in ordinary VGPRs (the per-group fold
# reads them right away; the accumulator-register form cost a copy each).
SOURCE_FLAGS: dict = {"gemm_skinny.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=fast",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libpq1)")


def flags_for(src: str) -> list:
    """hipcc flags for one source file of csrc/."""
    return [*HIPCC_FLAGS, *SOURCE_FLAGS.get(src, [])]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature name; that warning is noise
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libpq1.so; returns the library path."""
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in SOURCES + BENCH_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        jobs.append([cc, *flags_for(src), "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    for lib, srcs in ((LIB, SOURCES), (BENCH_LIB, BENCH_SOURCES)):
        objs = [os.path.join(BUILD, src.replace(".hip", ".o")) for src in srcs]
        tmp = lib + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
