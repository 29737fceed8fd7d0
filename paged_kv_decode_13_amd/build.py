"""Build libpagedkv.so (the gfx950 kernels and their C ABI) in-tree with hipcc,
and libpkvstream.so, the plain streaming-read kernel that the benchmark
times beside the decode (not part of the attention path).

Usage: python -m paged_kv_decode_13_amd.build  (or call ``build()``).
Every call recompiles.  Objects go to ``_build/`` next to the sources; the
shared libraries land in the package directory.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
OBJ_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libpagedkv.so")
STREAM_SRC = os.path.join(PKG_DIR, "probe", "stream_read.hip")
STREAM_LIB_PATH = os.path.join(PKG_DIR, "libpkvstream.so")
ARCH = "gfx950"

SOURCES = ["pkv_api.hip", "kv_write.hip", "paged_decode.hip", "paged_decode_mfma.hip",
           "paged_prefix_mfma.hip", "paged_prefill_mfma.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libpagedkv")
    return exe


def _compile(src: str) -> str:
    path = src if os.path.isabs(src) else os.path.join(CSRC, src)
    obj = os.path.join(OBJ_DIR, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, lib_path: str) -> None:
    tmp = lib_path + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib_path)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(len(SOURCES) + 1) as ex:
        objs = list(ex.map(_compile, SOURCES + [STREAM_SRC]))
    _link(objs[:-1], LIB_PATH)
    _link(objs[-1:], STREAM_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {STREAM_LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
