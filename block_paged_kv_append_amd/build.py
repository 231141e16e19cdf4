"""Build libpkv.so (HIP, gfx950) in-tree: ``python -m block_paged_kv_append_amd.build``."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpkv.so")
SOURCES = ["api.cpp", "graph.cpp", "allocator.cpp", "append.hip", "blocks.hip", "decode.hip",
           "prefill.hip", "mixed.hip", "check.hip", "bandwidth.hip"]
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # packed fp32 vector ops are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# per-source flags.  The matrix-core results stay in the vector register
# file: the decode's (rare) rescale multiplies its accumulators, and the
# prefill's softmax reads every score tile, which in the accumulator file
# cost a copy across per element (prefill 3.9% faster in the vector file).
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
SOURCE_FLAGS = {"decode.hip": _VGPR_FORM, "prefill.hip": _VGPR_FORM, "mixed.hip": _VGPR_FORM}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm toolchain required to build libpkv)")
    return path


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj, "-I", INCLUDE,
           "-I", CSRC] + HIPCC_FLAGS + SOURCE_FLAGS.get(src, []) + list(extra)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


TIMELINE_LIB = os.path.join(PKG, "libpkv_timeline.so")


def build(extra_flags=(), out: str = LIB, verbose: bool = False) -> str:
    """Compile every source for gfx950 and link ``libpkv.so``.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra_flags), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def build_timeline(verbose: bool = False) -> str:
    """The timeline build: the same library, with the decode kernels writing
    per-workgroup phase stamps (``bench.py --timeline`` reads them)."""
    global BUILD
    saved, BUILD = BUILD, os.path.join(PKG, "_build_timeline")
    try:
        return build(extra_flags=["-DPKV_TIMELINE"], out=TIMELINE_LIB, verbose=verbose)
    finally:
        BUILD = saved


if __name__ == "__main__":
    if sys.argv[1:] == ["--timeline"]:
        build_timeline(verbose=True)
    else:
        build(extra_flags=sys.argv[1:], verbose=True)
