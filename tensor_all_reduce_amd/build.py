"""Build libfc.so (the HIP kernels + C ABI) in-tree for gfx950.

``python -m tensor_all_reduce_amd.build`` compiles every source under ``csrc/`` with hipcc and links
the shared library next to this file.  The library is linked against the HIP runtime that PyTorch
loads (torch/lib/libamdhip64.so), so that torch's streams and device pointers are valid inside it:
one HIP runtime per process.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
# FC_SANITIZE=1 builds libfc_san.so instead: the host code (fc_api.cpp, the argument checks and launch
# set-up) instrumented with AddressSanitizer and UndefinedBehaviorSanitizer, the kernels unchanged, linked
# against the compiler's shared sanitizer runtime.  Load it with FC_LIB_PATH and that runtime preloaded,
# on the CPU (the checks run before any GPU call):
#   FC_SANITIZE=1 python -m tensor_all_reduce_amd.build
#   FC_LIB_PATH=$PWD/tensor_all_reduce_amd/libfc_san.so ASAN_OPTIONS=detect_leaks=0 \
#       LD_PRELOAD=$(/opt/rocm/lib/llvm/bin/clang++ -print-file-name=libclang_rt.asan-x86_64.so) \
#       python -m pytest tests/test_abi.py tests/test_binding.py
SANITIZE = os.environ.get("FC_SANITIZE") == "1"
# host-only instrumentation: each flag reaches the host compiler and linker only
HOST_SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libsan"]
LIB = os.path.join(HERE, "libfc_san.so" if SANITIZE else "libfc.so")
BUILD_DIR = os.path.join(ROOT, "_build", "san" if SANITIZE else "")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["fc_twostep.hip", "fc_slots.hip", "fc_live.hip", "fc_api.cpp"]

# -ffp-contract=off: a*b+c stays two roundings unless written as an explicit fma, which the bit-exact
# quantization codes depend on.  Packed fp32 instructions are disabled.  -fno-honor-nans on the kernels:
# NaN inputs are outside the contract, and without NaNs fminf/fmaxf need no quieting of their operands,
# which the compiler otherwise inserts before every min/max (and which blocks folding DPP moves).
COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wno-unused-function", "-I", INCLUDE]
# Kernel-argument preloading (gfx950): the leading kernel arguments (up to 16 dwords) are loaded into
# registers at dispatch, so a kernel's first memory address does not wait for an argument fetch.  The
# code object keeps a prologue that fetches them itself where the firmware does not preload.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc", "-fno-honor-nans", "-mllvm", "-amdgpu-kernarg-preload-count=16"]


def torch_lib_dir() -> str:
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.origin:
        raise RuntimeError("torch is required to locate the HIP runtime it loads")
    return os.path.join(os.path.dirname(spec.origin), "lib")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("command failed: " + " ".join(cmd))
    return out


def build(verbose: bool = False, csrc: str = CSRC, lib: str = LIB, build_dir: str = BUILD_DIR) -> str:
    """Compile the sources of `csrc` (default: the package's) into the shared library `lib` (default: the
    in-tree libfc.so), with object files in `build_dir`.  Returns the library's path."""
    os.makedirs(build_dir, exist_ok=True)
    from concurrent.futures import ThreadPoolExecutor
    jobs = []
    for src in SOURCES:
        path = os.path.join(csrc, src)
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        if src.endswith(".hip"):
            cmd = [HIPCC, *DEVICE, *COMMON, "-I", csrc, "-c", path, "-o", obj]
        else:
            cmd = [HIPCC, *COMMON, "-I", csrc, *(HOST_SAN if SANITIZE else []), "-x", "c++", "-D__HIP_PLATFORM_AMD__",
                   "-I/opt/rocm/include", "-c", path, "-o", obj]
        jobs.append((cmd, obj))
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:  # one compiler process per source file
        outs = list(ex.map(lambda j: _run(j[0]), jobs))
    for out in outs:
        if verbose and out.strip():
            print(out)
    objs = [obj for _, obj in jobs]
    tlib = torch_lib_dir()
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(HOST_SAN if SANITIZE else []), *objs, "-o", tmp,
           "-L" + tlib, "-l:libamdhip64.so", "-Wl,-rpath," + tlib, "-Wl,--no-undefined"]
    _run(cmd)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
