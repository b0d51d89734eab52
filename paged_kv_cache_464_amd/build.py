"""Build libpa.so (gfx950) in-tree with hipcc.

    python -m paged_kv_cache_464_amd.build [--verbose]

Objects go to ``_build/`` at the repository root; the shared library lands
next to this file so the Python binding finds it.  Every call rebuilds.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libpa.so")

HIP_SOURCES = ["cache_kernels.hip", "decode_kernels.hip", "capi.cpp"]
# decode_inst.hip is compiled once per (element kind, head_dim): the decode and
# multi-token kernel instantiations of each pair build in parallel.
INST_SOURCE = "decode_inst.hip"
INSTANCES = [(kind, d) for kind in (0, 1, 2) for d in (64, 128)]
HOST_SOURCES = ["block_manager.cpp"]
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
          f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
# Packed-fp32 instructions are kept out of every HIP object.
HIP_FLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics"]
# Per-source flags.  The attention kernels never let a NaN reach arithmetic
# whose result matters (unused slots are masked by selects on the position,
# not by tests on values; the encoders test NaN on bit patterns), so they are
# built without NaN semantics: fmaxf then needs no quieting of its inputs,
# which took two of every three v_max_f32 in the softmax maxima.
FILE_FLAGS = {"decode_kernels.hip": ["-fno-honor-nans"], INST_SOURCE: ["-fno-honor-nans"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    if verbose and r.stdout.strip():
        print(r.stdout)
    return r.stdout


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source and link libpa.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append([hipcc, *HIP_FLAGS, *COMMON, *FILE_FLAGS.get(src, []), *extra_flags, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    for kind, d in INSTANCES:
        obj = os.path.join(BUILD_DIR, f"decode_inst_k{kind}_d{d}.o")
        jobs.append([hipcc, *HIP_FLAGS, *COMMON, *FILE_FLAGS[INST_SOURCE], *extra_flags,
                     f"-DPA_INST_KIND={kind}", f"-DPA_INST_D={d}", "-c",
                     os.path.join(CSRC, INST_SOURCE), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append([hipcc, *COMMON, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    objs = [j[-1] for j in jobs]
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true",
                    help="print per-kernel register/LDS usage remarks")
    a = ap.parse_args(argv)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if a.resource_usage else []
    print(build(verbose=a.verbose or a.resource_usage, extra_flags=extra))


if __name__ == "__main__":
    sys.exit(main())
