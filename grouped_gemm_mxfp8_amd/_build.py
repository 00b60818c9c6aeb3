"""Build libmxmoe.so (HIP, gfx950) in-tree with hipcc.

    python -m grouped_gemm_mxfp8_amd._build

Compiles each source to an object in ``_build/`` (in parallel) and links the
shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmxmoe.so")
SOURCES = ["api.cpp", "quantize.hip", "gemm_mxfp8.hip", "gemm_bf16.hip", "route.hip",
           "fp8_tensor.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 arithmetic is kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host AddressSanitizer on the C-ABI layer (api.cpp holds only host code);
# each sanitizer flag applies to the host compilation only.
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_asan(dest: str) -> str:
    """libmxmoe.so with api.cpp built under host AddressSanitizer, into
    ``dest``; the kernel objects are the ones build() made (compiled first if
    missing or older than their source).  Load it with the sanitizer runtime
    preloaded (LD_PRELOAD of libasan) and MXMOE_LIB pointing at it."""
    os.makedirs(OBJ, exist_ok=True)
    os.makedirs(dest, exist_ok=True)
    objs = []
    for src in SOURCES:
        if src == "api.cpp":
            continue
        obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(os.path.join(CSRC, src)):
            obj = _compile(src)
        objs.append(obj)
    api_obj = os.path.join(dest, "api_asan.o")
    cmd = [hipcc(), *FLAGS, "-g", *HOST_ASAN, "-c", os.path.join(CSRC, "api.cpp"), "-o", api_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    lib = os.path.join(dest, "libmxmoe.so")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *HOST_ASAN, api_obj, *objs,
           "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
