"""Build libfdec.so (the HIP kernels and the C ABI) for gfx950, in the package directory.

    python -m memory_bound_decode_add_amd.build [--jobs N] [--save-temps]

Each source is compiled to an object in ``_build/`` with hipcc, then linked into
``memory_bound_decode_add_amd/libfdec.so``.  Packed-fp32 instruction selection is
disabled for device code (``-packed-fp32-ops``); hipcc's host pass does not know the
feature and says so, which is harmless.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfdec.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "add_rmsnorm.hip", "w4_gemv.hip", "w4_gemv_mfma.hip", "unfused.hip", "fp4_gemv.hip", "probes.hip", "w4_gemv_kmfma.hip", "w4_gemv_ring.hip", "w4_gemm.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfdec)")


def common_flags(save_temps: bool) -> list[str]:
    f = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
         "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    if save_temps:
        f.append("-save-temps=obj")
    return f


def compile_one(src: str, save_temps: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags(save_temps) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, cwd=BUILD, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stderr or "").splitlines() if ln.strip() and noise not in ln]
    if msgs:
        print(f"[{src}]\n" + "\n".join(msgs), file=sys.stderr)
    return obj


def build(jobs: int = 4, save_temps: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: compile_one(s, save_temps), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libfdec.so failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--save-temps", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.save_temps))


if __name__ == "__main__":
    main()
