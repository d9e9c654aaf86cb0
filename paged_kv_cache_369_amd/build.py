"""Build the HIP library libpkv.so in-tree (hipcc, gfx950).

    python -m paged_kv_cache_369_amd.build              # libpkv.so
    python -m paged_kv_cache_369_amd.build --timeline   # libpkv_timeline.so as well

Every HIP source is compiled with packed-fp32 instructions disabled; the C ABI
layer is host C++ compiled by the same driver.  The shared library lands next
to this file, where the Python binding loads it from.  The timeline library is
the same sources with PKV_TIMELINE defined: the decode waves also record a few
clock stamps each (pkv_timeline_read), for `bench.py --timeline`; nothing else
loads it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpkv.so")
OUT_TIMELINE = os.path.join(HERE, "libpkv_timeline.so")
OBJ = os.path.join(HERE, "_build")
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_SOURCES = ["kv_write.hip", "paged_decode.hip", "check.hip"]
CXX_SOURCES = ["capi.cpp", "block_manager.cpp"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I" + CSRC, "-I" + os.path.join(HERE, "..", "include")]
HIP_FLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-fno-gpu-rdc",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, flags, objdir: str) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, timeline: bool = False) -> str:
    """Build libpkv.so, or with timeline=True the instrumented libpkv_timeline.so."""
    out = OUT_TIMELINE if timeline else OUT
    objdir = OBJ + ("_timeline" if timeline else "")
    extra = ["-DPKV_TIMELINE"] if timeline else []
    os.makedirs(objdir, exist_ok=True)
    jobs = [(s, HIP_FLAGS + extra) for s in HIP_SOURCES] + [(s, extra) for s in CXX_SOURCES]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], j[1], objdir), jobs))
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    if "--timeline" in sys.argv[1:]:
        build(verbose=True, timeline=True)
    sys.exit(0)
