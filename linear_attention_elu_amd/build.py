"""Build liblinattn.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Every translation unit is compiled by hipcc in parallel into _build/, then
linked into linear_attention_elu_amd/liblinattn.so.  Packed fp32 instructions
are switched off for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblinattn.so")
ARCH = "gfx950"

SOURCES = [
    "la_api.cpp",
    "la_decode.hip",
    "la_bwd.hip",
    "la_scan.hip",
    "la_noalloc.hip",
    "la_prf.hip",
    "la_fwd_dk16.hip",
    "la_fwd_dk32.hip",
    "la_fwd_dk64.hip",
    "la_fwd_dk128.hip",
    "la_bwd_dk16.hip",
    "la_bwd_dk32.hip",
    "la_bwd_dk64.hip",
    "la_bwd_dk128.hip",
]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]  # host-only code, but built with the HIP headers and flags
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
