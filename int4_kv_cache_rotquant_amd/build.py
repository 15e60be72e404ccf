"""Build ``libkvrq.so`` (HIP for gfx950 + the C-ABI host layer) in-tree.

    python -m int4_kv_cache_rotquant_amd.build

Every call recompiles.  Flags that matter for results:
  * ``-ffp-contract=off`` on the write kernel: the encoding's binary32
    operations must each round on their own (no fused multiply-add);
  * ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed fp32
    instructions are generated anywhere (hipcc's host pass warns that it does
    not know the feature; that warning is harmless).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvrq.so")
ARCH = os.environ.get("KVRQ_OFFLOAD_ARCH", "gfx950")

HIP_COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
              "-DKVRQ_BUILDING_LIBRARY", "-I", os.path.join(ROOT, "include"),
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Wall", "-Wno-unused-result"]

SOURCES = [
    ("kvrq_write.hip", ["-ffp-contract=off"]),
    ("kvrq_decode.hip", []),
    ("kvrq_noalloc.hip", []),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise subprocess.CalledProcessError(r.returncode, cmd)
    if out.strip():
        sys.stderr.write(out + "\n")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src, extra in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = ["hipcc", "-c", os.path.join(CSRC, src), "-o", obj, *HIP_COMMON, *extra]
        if verbose:
            print(" ".join(cmd))
        _run(cmd)
        objs.append(obj)
    abi_obj = os.path.join(BUILD, "kvrq_abi.o")
    cmd = ["g++", "-c", os.path.join(CSRC, "kvrq_abi.cpp"), "-o", abi_obj, "-O2", "-std=c++17",
           "-fPIC", "-fvisibility=hidden", "-DKVRQ_BUILDING_LIBRARY", "-Wall", "-Wextra",
           "-I", os.path.join(ROOT, "include")]
    if verbose:
        print(" ".join(cmd))
    _run(cmd)
    objs.append(abi_obj)
    tmp = LIB + ".tmp"
    cmd = ["hipcc", "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    _run(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
