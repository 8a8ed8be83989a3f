"""Builds libmoe.so (HIP, gfx950) in-tree with hipcc, and its bounds-checked
twin libmoe_checked.so.

Each source is compiled to an object in parallel (both variants at once),
then each variant is linked into one shared library next to this file.  The
checked variant is compiled with MOE_CHECKED: its kernels check the indices
they take from device data (tile table, sorted ids, reduce row map) against
their buffers and report a miss in the device status word (MOE_DEV_BOUNDS)
instead of making the access.  Every HIP compile disables the packed fp32
instructions (-packed-fp32-ops); the host pass warns that it does not know
that feature, which is harmless.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe.so")
LIB_CHECKED = os.path.join(HERE, "libmoe_checked.so")
VARIANTS = {"release": ([], LIB), "checked": (["-DMOE_CHECKED"], LIB_CHECKED)}
SOURCES = ["moe_api.hip", "moe_kernels.hip", "moe_gemm.hip", "moe_gemm_fp8.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libmoe)")


COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str, variant: str, verbose: bool) -> str:
    out_dir = os.path.join(BUILD_DIR, variant)
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *VARIANTS[variant][0], "-I", INCLUDE, "-I", CSRC, "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed on {src} ({variant})")
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compiles every HIP source for gfx950 and links libmoe.so and
    libmoe_checked.so (always rebuilds); returns the release library's path."""
    jobs = [(src, v) for v in VARIANTS for src in SOURCES]
    for v in VARIANTS:
        os.makedirs(os.path.join(BUILD_DIR, v), exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], j[1], verbose), jobs))
    for v, (_, lib) in VARIANTS.items():
        _link([o for (src, vv), o in zip(jobs, objs) if vv == v], lib, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
