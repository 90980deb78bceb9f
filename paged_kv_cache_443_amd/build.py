"""Build ``libpa.so`` (the C ABI library) in-tree with hipcc for gfx950.

Usage: ``python -m paged_kv_cache_443_amd.build [-v]``.  Each source is
compiled to an object in ``_build/`` (in parallel), then linked into
``paged_kv_cache_443_amd/libpa.so``.  Always recompiles.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")

SOURCES = [
    "pa_api.cpp",
    "pa_validate.cpp",
    "pa_decode_mfma.hip",
    "pa_decode_f32.hip",
    "pa_reduce.hip",
    "pa_append.hip",
    "pa_copy.hip",
    "pa_noalloc.hip",
    "pa_probe.hip",
    "pa_mla.hip",
    "pa_decode_valu.hip",
    "pa_block_manager.cpp",
]

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm not installed?)")


def common_flags() -> list:
    return [
        "-O3",
        "-std=c++17",
        "-fPIC",
        f"--offload-arch={ARCH}",
        # packed fp32 VALU ops are kept out of every device build
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # keep matrix-core accumulators in ordinary VGPRs: the online-softmax
        # rescale multiplies them every chunk, and AGPR homes cost a copy each way
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wall",
        "-Wno-unused-result",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *common_flags(), *lang, "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host compilation pass does not know the device-only target feature
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in (r.stdout + r.stderr).splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
