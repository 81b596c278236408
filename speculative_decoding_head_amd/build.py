"""Build libmtp.so (HIP, gfx950 only) in place: ``python -m speculative_decoding_head_amd.build``.

Every HIP source is compiled with hipcc for gfx950 with packed-fp32 instruction
selection disabled, then linked into one shared library next to this file.  A second,
small library (libmtp_probe.so) holds the read-only streaming probe the benchmark uses to
measure the access pattern's bandwidth ceiling; it is not part of the C ABI.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmtp.so")
PROBE_LIB = os.path.join(HERE, "libmtp_probe.so")
PROBE_SOURCES = ["stream_probe.hip"]
SOURCES = ["api.cpp", "lmhead.hip", "lmhead_wide.hip", "accept.hip", "commit.hip", "pack.hip", "width.cpp",
           "noalloc.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    "-x", "hip", "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return h


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def _link(objs, lib, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
