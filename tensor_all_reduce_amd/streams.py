"""Streams on disjoint sets of compute units, for a sender and a receiver that must run at the same time.

HIP multiplexes streams onto a few hardware queues, and two streams that share a queue run their kernels
one after the other: a receiver spinning on one of them would then wait out its whole poll budget before
a sender queued behind it could start.  A stream created with a compute-unit mask gets a hardware queue of
its own, and its kernels run only on the masked units, so a sender and a receiver on two such streams with
disjoint masks neither share a queue nor compete for compute units.  Plumbing only: nothing here computes.
"""
from __future__ import annotations

import ctypes as C


def _hip():
    """PyTorch's HIP runtime (already mapped into the process once torch has initialised the device)."""
    import torch
    torch.cuda.init()
    from ._lib import _hip_runtimes_mapped
    paths = sorted(_hip_runtimes_mapped())
    if len(paths) != 1:
        raise RuntimeError(f"expected exactly one HIP runtime mapped, found {paths}")
    h = C.CDLL(paths[0])
    h.hipExtStreamCreateWithCUMask.argtypes = [C.POINTER(C.c_void_p), C.c_uint32, C.POINTER(C.c_uint32)]
    h.hipExtStreamCreateWithCUMask.restype = C.c_int
    h.hipStreamSynchronize.argtypes = [C.c_void_p]
    h.hipStreamSynchronize.restype = C.c_int
    h.hipStreamDestroy.argtypes = [C.c_void_p]
    h.hipStreamDestroy.restype = C.c_int
    return h


class CUMaskedStream:
    """A stream whose kernels run on compute units [first, first + count) only (default priority)."""

    def __init__(self, first: int, count: int):
        import torch
        total = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
        if not (0 <= first and count > 0 and first + count <= total):
            raise ValueError(f"compute units [{first}, {first + count}) outside [0, {total})")
        words = (total + 31) // 32
        mask = (C.c_uint32 * words)()
        for cu in range(first, first + count):
            mask[cu // 32] |= 1 << (cu % 32)
        self._hip = _hip()
        self._h = C.c_void_p()
        err = self._hip.hipExtStreamCreateWithCUMask(C.byref(self._h), words, mask)
        if err != 0:
            raise RuntimeError(f"hipExtStreamCreateWithCUMask failed with hipError {err}")
        self.first, self.count = first, count

    @property
    def cuda_stream(self) -> int:
        return self._h.value

    def synchronize(self) -> None:
        err = self._hip.hipStreamSynchronize(self._h)
        if err != 0:
            raise RuntimeError(f"hipStreamSynchronize failed with hipError {err}")

    def close(self) -> None:
        if self._h.value:
            self.synchronize()
            self._hip.hipStreamDestroy(self._h)
            self._h = C.c_void_p()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def sender_receiver_streams(receiver_cus: int = 32):
    """(receiver, sender): the receiver on the first `receiver_cus` compute units, the sender on the rest."""
    import torch
    total = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    return CUMaskedStream(0, receiver_cus), CUMaskedStream(receiver_cus, total - receiver_cus)
