"""Exhaustive checks of the quantizer's exact-quotient helpers (fc_device.h) against this GPU's IEEE
division: the fma-corrected quotient by 15 and by 255 for every non-negative finite float, and the
fma-corrected hardware reciprocal for every positive finite fp16 scale.  Every quantizer and requantizer
takes its scale and reciprocal through them, so codes stay those of the definition (IEEE quotients) for
every group; the parity tests check the codes themselves."""
import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu
LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "libfc_selfcheck.so")


def test_exact_quotients_match_ieee_division():
    import torch
    torch.cuda.init()  # the library shares PyTorch's HIP runtime
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is missing: build it with `python tests/native/build_selfcheck.py` "
                    "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB)
    lib.fc_selfcheck_quotients.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
    lib.fc_selfcheck_quotients.restype = ctypes.c_int
    out = (ctypes.c_uint64 * 3)()
    assert lib.fc_selfcheck_quotients(out) == 0, "HIP error in the self-check"
    assert list(out) == [0, 0, 0], (f"mismatches against IEEE division: x/15 {out[0]}, x/255 {out[1]}, "
                                    f"1/s {out[2]}")
