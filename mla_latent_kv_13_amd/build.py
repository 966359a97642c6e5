"""Build the HIP library (gfx950) in-tree: csrc/*.hip + csrc/api.cpp -> libtpla_mi355x.so.

Every source is compiled by hipcc for gfx950 only.  Packed fp32 instructions are
switched off for device code (-packed-fp32-ops); hipcc's host pass warns that it
does not know that feature, which is harmless.  Loops start on 64-byte boundaries
(-falign-loops=64): the decode kernel's steady loop otherwise lands wherever the code
before it ends, and its speed moved by a few percent with that offset.
"""

from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libtpla_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ROOT = os.path.dirname(PKG)

SOURCES = ["api.cpp", "decode_generic.hip", "decode_mfma.hip", "merge.hip", "append.hip", "upproj.hip", "prefill.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-falign-loops=64",
         "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the library needs ROCm's hipcc to build")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), "-x", "hip", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
