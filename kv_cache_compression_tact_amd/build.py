"""Build step of the TACT-KV library: codebook generation and libtact.so.

    python kv_cache_compression_tact_amd/build.py

1. Compiles the codebook generator (csrc/gen_codebooks.cpp) with the host
   compiler and regenerates csrc/generated/codebooks.inc.
2. Compiles the C-ABI host layer and the gfx950 kernels with hipcc into
   kv_cache_compression_tact_amd/libtact.so (in tree; no GPU is needed).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtact.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division and square root (the quantizer decides in fp32)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function",
]
SOURCES = ["tact_api.cpp", "tact_codebooks.cpp", "tact_mfma.hip", "tact_quant.hip",
           "tact_attend.hip", "tact_static_ws.hip"]


def _run(cmd, **kw):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, **kw)


def gen_codebooks() -> None:
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "gen_codebooks")
    _run(["g++", "-O2", "-std=c++17", os.path.join(CSRC, "gen_codebooks.cpp"), "-o", exe])
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    dst = os.path.join(CSRC, "generated", "codebooks.inc")
    os.makedirs(os.path.dirname(dst), exist_ok=True)
    old = open(dst).read() if os.path.exists(dst) else None
    if old != out:
        with open(dst, "w") as f:
            f.write(out)


def build_library() -> str:
    """Every source compiled to an object in parallel (hipcc per file), then
    linked into the shared library."""
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [HIPCC, *HIP_FLAGS, "-c", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               os.path.join(CSRC, src), "-o", obj]
        print("+", " ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd))
    failed = [src for src, pr in zip(SOURCES, procs) if pr.wait() != 0]
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def build() -> str:
    gen_codebooks()
    return build_library()


if __name__ == "__main__":
    print(build())
    sys.exit(0)
