"""Build the HIP library libpkv.so in-tree (hipcc, gfx950).

    python -m paged_kv_cache_369_amd.build

Every HIP source is compiled with packed-fp32 instructions disabled; the C ABI
layer is host C++ compiled by the same driver.  The shared library lands next
to this file, where the Python binding loads it from.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpkv.so")
OBJ = os.path.join(HERE, "_build")
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_SOURCES = ["kv_write.hip", "paged_decode.hip", "check.hip"]
CXX_SOURCES = ["capi.cpp", "block_manager.cpp"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I" + CSRC, "-I" + os.path.join(HERE, "..", "include")]
HIP_FLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-fno-gpu-rdc",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, flags) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = [(s, HIP_FLAGS) for s in HIP_SOURCES] + [(s, []) for s in CXX_SOURCES]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
