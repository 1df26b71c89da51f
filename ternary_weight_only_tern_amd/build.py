"""Build libtern.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Every source is compiled to its own object in parallel (under _build/ next to
this file), then the objects are linked into libtern.so.
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
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtern.so")
OBJDIR = os.path.join(PKG, "_build")

SOURCES = ["tern_api.cpp", "pack.hip", "gemv.hip", "gemv_mfma.hip", "gemv_b3.hip", "gemm.hip", "quant.hip", "noalloc.hip",
           "rotate.hip"]
ARCH = os.environ.get("TERN_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set ROCM_PATH)")


def _flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # packed FP32 VALU forms are disabled on purpose
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            "-I", INCLUDE, "-I", CSRC]


def _run(cmd: list) -> tuple:
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    return proc.returncode, out


def build(verbose: bool = False) -> str:
    """Compile every source into libtern.so; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    cc = hipcc()
    jobs = []
    for s in SOURCES:
        obj = os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o")
        jobs.append((s, obj, [cc] + _flags() + ["-c", os.path.join(CSRC, s), "-o", obj]))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(lambda j: (j, _run(j[2])), jobs))
    for (s, _, cmd), (rc, out) in results:
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {s} ({rc}):\n{' '.join(cmd)}\n{out}")
        if verbose and out.strip():
            print(out, file=sys.stderr)
    tmp = LIB + ".tmp"
    rc, out = _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + [j[1] for j in jobs] + ["-o", tmp])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{out}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
