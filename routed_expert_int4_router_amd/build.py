"""Build libmoe.so (HIP kernels for gfx950 + C ABI) in-tree.

Usage: python -m routed_expert_int4_router_amd.build   (or build() from Python)

Host-only C++ (packer, pool policy, blob-file reader) is compiled with g++ and strict IEEE
float semantics (no FMA contraction); the HIP sources and the ABI layer with
hipcc for gfx950. Objects go to _build/ at the repository root, the library
next to this file.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HOST_SOURCES = ["pack.cpp", "pool_policy.cpp", "blob_file.cpp"]
HIP_SOURCES = ["abi.cpp", "decode.hip", "prefill.hip", "scalar.hip", "gdn.hip", "attn.hip"]

COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-result"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src in HOST_SOURCES:
        cmd = ["g++", *COMMON, "-ffp-contract=off", "-fno-fast-math", "-c", path, "-o", obj]
    else:
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [HIPCC, *COMMON, *HIP_FLAGS, *lang, "-c", path, "-o", obj]
    _run(cmd)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libmoe.so; returns the library path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = HOST_SOURCES + HIP_SOURCES
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-lpthread"])
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
