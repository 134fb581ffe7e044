"""Build libsbf.so for gfx950 in-tree with hipcc (one object per source, in
parallel, then one shared-library link).

    python -m minimizer_sharded_bloom_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libsbf.so")
OBJDIR = os.path.join(PKG, "_build")
ARCH = os.environ.get("SBF_OFFLOAD_ARCH", "gfx950")

SOURCES = ["inst_grid_best_a.hip", "inst_grid_best_b.hip", "inst_wide.hip", "inst_slice_s_a.hip", "inst_slice_s_b.hip", "inst_slice_m_a.hip", "inst_slice_m_b.hip",
           "inst_slice_m_c.hip", "inst_slice_h.hip", "inst_m16.hip", "inst_m12.hip", "inst_m20.hip", "inst_extra.hip",
           "sbf_alpha.hip", "sbf_generic.hip", "sbf_membench.hip", "sbf_api.cpp", "sbf_host.cpp", "sbf_fastx.cpp", "sbf_bgzf.cpp"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def common_flags() -> list[str]:
    return ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
            # no packed-FP32 instruction selection
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # unroll pragmas that only the compile-time instances can honour
            "-Wall", "-Wno-unused-function", "-Wno-pass-failed", "-I" + os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    """Compile every source and link libsbf.so; always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-lz", "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    build(ap.parse_args().jobs)
