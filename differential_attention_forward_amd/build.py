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
MICRO_LIB = os.path.join(PKG, "libdiffattn_micro.so")
# debug variant: every kernel fills its LDS with NaN patterns at entry
# (DIFFATTN_LDS_POISON in csrc/common.h); tests compare it with LIB bit for bit
POISON_LIB = os.path.join(PKG, "libdiffattn_poison.so")

KERNEL_SOURCES = ["prefill.hip", "decode.hip", "lambda.hip", "backward.hip", "scratch.hip"]
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


def _compile(src: str, flags, tag: str = "") -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    cmd = [hipcc(), *COMMON, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, out)


def build_library(verbose: bool = True) -> str:
    """libdiffattn.so (the attention library), libdiffattn_poison.so (the same
    with LDS poisoned at every kernel's entry, for tests) and
    libdiffattn_micro.so (the microbenchmarks bench.py reports measured
    ceilings from)."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = ([(s, KERNEL_FLAGS, "") for s in KERNEL_SOURCES + ["micro.hip"]] +
            [(s, [], "") for s in HOST_SOURCES] +
            [(s, KERNEL_FLAGS + ["-DDIFFATTN_LDS_POISON"], "_poison") for s in KERNEL_SOURCES])
    workers = min(len(jobs), os.cpu_count() or 8)
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = dict(zip([j[0] + j[2] for j in jobs], ex.map(lambda j: _compile(*j), jobs)))
    _link([objs[s] for s in KERNEL_SOURCES + HOST_SOURCES], LIB)
    _link([objs[s + "_poison"] for s in KERNEL_SOURCES] + [objs[s] for s in HOST_SOURCES], POISON_LIB)
    _link([objs["micro.hip"]], MICRO_LIB)
    if verbose:
        print(f"built {LIB}, {POISON_LIB} and {MICRO_LIB}")
    return LIB


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime that ships with ROCm's LLVM, or ''."""
    root = "/opt/rocm/llvm/lib/clang"
    if os.path.isdir(root):
        for ver in sorted(os.listdir(root), reverse=True):
            path = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
            if os.path.exists(path):
                return path
    return ""


def build_sanitized_host(out_dir: str) -> str:
    """Host-only build of the C ABI (abi.hip) with AddressSanitizer and
    UndefinedBehaviorSanitizer, linked with stand-ins for the kernel launchers
    (tests/abi_san_stubs.cpp), as libdiffattn_san.so in ``out_dir``.  It serves
    the CPU tests of argument validation, which never launch a kernel; the GPU
    code is not built or instrumented."""
    os.makedirs(out_dir, exist_ok=True)
    clangxx = "/opt/rocm/llvm/bin/clang++"
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    abi_o = os.path.join(out_dir, "abi.o")
    stub_o = os.path.join(out_dir, "stubs.o")
    lib = os.path.join(out_dir, "libdiffattn_san.so")
    steps = [
        [hipcc(), "--offload-arch=gfx950", "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fPIC",
         "-ffp-contract=off", *san, "-c", os.path.join(CSRC, "abi.hip"), "-o", abi_o],
        [clangxx, "-O1", "-g", "-std=c++17", "-fPIC", "-fsanitize=address,undefined",
         "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-c",
         os.path.join(ROOT, "tests", "abi_san_stubs.cpp"), "-o", stub_o],
        [clangxx, "-shared", "-fsanitize=address,undefined", "-shared-libasan", "-o", lib, abi_o, stub_o,
         "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"],
    ]
    for cmd in steps:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"sanitizer build step failed: {' '.join(cmd[:2])}\n{res.stderr}")
    return lib


if __name__ == "__main__":
    build_library()
    sys.exit(0)
