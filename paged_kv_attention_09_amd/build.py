"""Build libpagedattn.so for gfx950 with hipcc, in-tree.

Usage: python -m paged_kv_attention_09_amd.build [-v]
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
OUT_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(OUT_DIR, "libpagedattn.so")
# The block manager (pa_block_manager.cpp) and the precondition checks
# (pa_check.cpp) are host code; hipcc compiles them as C++.
SOURCES = ["pa_api.hip", "pa_append.hip", "pa_decode.hip", "pa_prefill.hip",
           "pa_block_manager.cpp", "pa_check.cpp"]
# The benchmark's streaming-read probe is a library of its own, outside the
# attention library's ABI.
PROBE_SOURCES = ["bench/read_probe.hip"]
PROBE_LIB = os.path.join(OUT_DIR, "libpa_readprobe.so")

ARCH = "gfx950"
# Packed-fp32 VALU forms are kept out of the generated code (-packed-fp32-ops).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def _compile(src: str, obj: str, verbose: bool) -> None:
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    for o in objs:
        os.remove(o)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the attention library and the
    benchmark's read probe.  Always rebuilds."""
    os.makedirs(OUT_DIR, exist_ok=True)
    obj = lambda s: os.path.join(OUT_DIR, os.path.basename(os.path.splitext(s)[0]) + ".o")  # noqa
    srcs = SOURCES + PROBE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(7, len(srcs))) as ex:
        list(ex.map(lambda s: _compile(s, obj(s), verbose), srcs))
    _link([obj(s) for s in SOURCES], LIB, verbose)
    _link([obj(s) for s in PROBE_SOURCES], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
