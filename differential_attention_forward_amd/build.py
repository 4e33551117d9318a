"""Builds libdiffattn.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Each source is compiled to an object under ``_build/`` in parallel, then the
objects are linked into ``differential_attention_forward_amd/libdiffattn.so``.
Usage: ``python -m differential_attention_forward_amd.build``.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdiffattn.so")

KERNEL_SOURCES = ["prefill.hip", "decode.hip", "lambda.hip", "backward.hip"]
HOST_SOURCES = ["abi.hip"]

COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          # packed-fp32 VALU forms stay off; fp contraction only where written
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-ffp-contract=off"]
# device-only: no IEEE-mode NaN quieting around min/max in the kernels
KERNEL_FLAGS = ["-mno-amdgpu-ieee", "-fno-honor-nans"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the gfx950 library cannot be built")
    return path


def _compile(src: str, flags) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def build_library(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(s, KERNEL_FLAGS) for s in KERNEL_SOURCES] + [(s, []) for s in HOST_SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build_library()
    sys.exit(0)
