"""Build libattn.so in-tree with hipcc for gfx950.

    python -m transformer_attention_attn_amd.build

Every HIP source is compiled with packed-fp32 instructions disabled (the
compiler may otherwise fuse pairs of fp32 operations into v_pk_* forms).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattn.so")

# (source, object name, extra flags): the bf16 kernel is compiled once per head
# dimension, each object holding only the constants of its own tile shape
SOURCES = [
    ("attn_api.cpp", "attn_api", []),
    ("attn_layout.cpp", "attn_layout", []),
    ("kernel_fp32.hip", "kernel_fp32", []),
    ("kernel_bf16.hip", "kernel_bf16_d64", ["-DATTN_HEAD_DIM=64"]),
    ("kernel_bf16.hip", "kernel_bf16_d128", ["-DATTN_HEAD_DIM=128"]),
    ("kernel_decode.hip", "kernel_decode", []),
    ("kernel_fp8.hip", "kernel_fp8", []),
]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
]


def _compile(unit, verbose: bool) -> str:
    src, name, flags = unit
    obj = os.path.join(BUILD_DIR, name + ".o")
    cmd = [hipcc(), *COMMON, *flags, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; that warning is harmless
    err = "\n".join(line for line in res.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    # a kernel template whose host pass failed silently leaves its launch stub undefined
    nm = shutil.which("nm")
    if nm:
        undef = subprocess.run([nm, "-u", tmp], capture_output=True, text=True).stdout
        bad = [line for line in undef.splitlines() if "__device_stub__" in line]
        if bad:
            raise RuntimeError("undefined kernel launch stubs in libattn.so:\n" + "\n".join(bad))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
