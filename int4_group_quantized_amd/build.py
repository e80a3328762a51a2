"""Build libq4g128.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage:  python int4_group_quantized_amd/build.py   (or call build_library()).
Run it as a script, not as a module of the package: importing the package
loads the library that this script replaces.
The shared object is written next to this file so that it travels with the
source tree; intermediate objects go to _build/ (not committed).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libq4g128.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
# Benchmark diagnostics (read-only GEMV twin, streaming read, empty launch):
# a library of their own, outside the product ABI.
DIAG_NAME = "libq4g128_diag.so"
DIAG_PATH = os.path.join(PKG_DIR, DIAG_NAME)
DIAG_SOURCES = ["diag.hip"]

SOURCES = ["api.cpp", "gemv.hip", "gemv_group.hip", "gemv_seg.hip", "prefill.hip", "prefill_split.hip", "prefill_pair.hip", "prefill_epilogue.hip", "pack.hip",
           "quantize.hip", "head_int8.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError(f"hipcc not found ({cand}); the library needs ROCm's hipcc")
    return cand


COMPILE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # explicit fma/dot builtins define the arithmetic; no silent contraction
    "-ffp-contract=off",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-fvisibility=hidden",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


# Flags of single sources.  The quantiser's inputs are finite by contract and
# it forms no NaN from them: without NaNs its min/max reductions need no
# operand quieting, and each DPP move folds into its min or max.
SOURCE_FLAGS = {"quantize.hip": ["-fno-honor-nans"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMPILE_FLAGS + SOURCE_FLAGS.get(src, []) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(
        line for line in (res.stdout + res.stderr).splitlines()
        if "packed-fp32-ops" not in line and "--hip-link" not in line
    )
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return obj


def _link(objs, name: str, path: str, verbose: bool) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs + [
        f"-Wl,-soname,{name}",
        "-Wl,-rpath,/opt/rocm/lib",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, path)


def build_library(verbose: bool = False) -> str:
    """Compile and link libq4g128.so and the diagnostics library; returns the former's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + DIAG_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB_NAME, LIB_PATH, verbose)
    _link([objs[s] for s in DIAG_SOURCES], DIAG_NAME, DIAG_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    path = build_library(verbose="-v" in sys.argv)
    print(path)
