"""Build the HIP library in-tree: kv_cache_vector_append_amd/libtq_hip.so (gfx950).

    python -m kv_cache_vector_append_amd.build [--jobs N]

hipcc cross-compiles for gfx950 without a GPU present.  Every source is
compiled on each call (objects go to _build/), then linked into one shared
library exporting the C ABI declared in include/tq.h.
"""
from __future__ import annotations

import argparse
import hashlib
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
LIB = os.path.join(PKG, "libtq_hip.so")
ARCH = os.environ.get("TQ_OFFLOAD_ARCH", "gfx950")

SOURCES = ["tq_abi.cpp", "tq_host.cpp", "tq_append.hip", "tq_decode_mfma.hip", "tq_codec.hip", "tq_scratch.hip"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep packed fp32 instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]

# Per-file additions.  The matrix-core decode never relies on NaN propagation
# (every test is against -inf or an ordered compare), and without NaN
# semantics a max of a cross-lane (DPP) value is one instruction instead of
# three.
FILE_FLAGS = {"tq_decode_mfma.hip": ["-fno-honor-nans"]}


def source_hash() -> str:
    """sha256 (first 16 hex digits) over the library's sources: every file of
    csrc/ and include/, in name order, with its name."""
    h = hashlib.sha256()
    for d in (CSRC, INCLUDE):
        for name in sorted(os.listdir(d)):
            path = os.path.join(d, name)
            if os.path.isfile(path):
                h.update(name.encode())
                with open(path, "rb") as f:
                    h.update(f.read())
    return h.hexdigest()[:16]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    extra = [f'-DTQ_SOURCE_HASH="{source_hash()}"'] if src == "tq_abi.cpp" else []
    cmd = [hipcc()] + COMMON + FILE_FLAGS.get(src, []) + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    args = ap.parse_args(argv)
    build(args.jobs, verbose=True)


if __name__ == "__main__":
    sys.exit(main())
