"""Build the test-support library libfc_selfcheck.so (exhaustive checks of device helpers against the GPU's
IEEE arithmetic) next to this file, with the same compiler flags and HIP runtime as libfc.so.

    python tests/native/build_selfcheck.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libfc_selfcheck.so")


def build() -> str:
    sys.path.insert(0, ROOT)
    from tensor_all_reduce_amd import build as b
    src = os.path.join(HERE, "fc_selfcheck.hip")
    tlib = b.torch_lib_dir()
    tmp = LIB + ".tmp%d" % os.getpid()
    b._run([b.HIPCC, *b.DEVICE, *b.COMMON, "-I", b.CSRC, "-shared", src, "-o", tmp, "-L" + tlib, "-l:libamdhip64.so",
            "-Wl,-rpath," + tlib, "-Wl,--no-undefined"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
