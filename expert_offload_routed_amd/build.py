"""Compile the HIP sources into the in-tree shared library ``libmoe_offload.so``.

hipcc cross-compiles for gfx950 without a GPU. Every source is compiled with
packed fp32 instructions disabled (``-packed-fp32-ops``); the library links
only the HIP runtime.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmoe_offload.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["route.hip", "permute.hip", "ffn.hip", "ffn_int4.hip", "gemm.hip", "skinny.hip",
           "decode_int4.hip", "decode_bf16.hip", "combine.hip", "slots.hip", "split.hip", "runtime.hip"]
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libmoe_offload)")
    return exe


def _run(cmd: list[str]) -> None:
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build(jobs: int | None = None) -> str:
    """Compile every source (always) and link the library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in srcs]
    cmds = [[cc, *CFLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(srcs, objs)]
    jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(_run, cmds))
    tmp = LIB_PATH + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
