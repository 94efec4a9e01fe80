"""Build libsplr.so (gfx950 only) in-tree with hipcc.

    python -m sparse_rank_linear_prune24_amd.build

Every HIP source is compiled with `-Xclang -target-feature -Xclang -packed-fp32-ops`, which keeps
the compiler from emitting packed float32 instructions (the host pass warns that it does not know
the feature; that warning is harmless).
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libsplr.so")
SOURCES = ["api.hip", "pack.hip", "residual.hip", "lowrank.hip", "linear_bf16.hip", "linear_f32.hip", "reconstruct.hip",
           "cholqr.hip", "decode.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def source_files():
    """Every file the library is built from: the HIP sources, their headers and the public header."""
    names = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".hpp")))
    return [os.path.join(CSRC, f) for f in names] + [os.path.join(INCLUDE, "splr.h")]


def source_hash() -> str:
    """First 16 hex digits of the SHA-256 over the sources (name and contents, in name order); the
    build embeds it in splr_version()."""
    h = hashlib.sha256()
    for path in source_files():
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    return h.hexdigest()[:16]


def _compile(src: str, defines=()) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 4)), 16)
    defines = [f'-DSPLR_SOURCE_SHA="{source_hash()}"']
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, defines), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
