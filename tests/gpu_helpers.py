"""Helpers for the GPU parity tests: host<->device transfers of raw bit patterns and bf16 comparisons."""
import numpy as np
import torch

DEV = "cuda:0"


def up(a: np.ndarray) -> torch.Tensor:
    """Upload a numpy array of raw bits (uint8/uint16/uint32/uint64/int32) as a same-width torch tensor."""
    a = np.ascontiguousarray(a)
    view = {1: np.uint8, 2: np.int16, 4: np.int32, 8: np.int64}[a.dtype.itemsize]
    return torch.from_numpy(a.view(view)).to(DEV)


def down(t: torch.Tensor, dtype) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(dtype)


def counters_buf() -> torch.Tensor:
    """A zeroed receiver counters buffer (the library's grouped layout)."""
    from tensor_all_reduce_amd import _lib
    return torch.zeros(_lib.COUNTER_WORDS, dtype=torch.int32, device=DEV)


def counts(cnt: torch.Tensor, k: int = 2) -> np.ndarray:
    """The first k counts of a receiver counters buffer, summed over its groups (uint32)."""
    from tensor_all_reduce_amd import _lib
    return _lib.counter_totals(cnt, k).astype(np.uint32)


def ulp_dist(a, b):
    def ordv(u):
        u = np.asarray(u, np.uint16).astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u & 0x7FFF)
    return np.abs(ordv(a) - ordv(b))


def assert_bf16_close(got, want, max_ulp=2, what=""):
    got = np.asarray(got, np.uint16).ravel()
    want = np.asarray(want, np.uint16).ravel()
    assert got.shape == want.shape, what
    nan = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
    assert not nan.any(), f"{what}: NaN in GPU output"
    d = ulp_dist(got, want)
    bad = np.nonzero(d > max_ulp)[0]
    assert bad.size == 0, (f"{what}: {bad.size} elements beyond {max_ulp} ulp, first at {bad[:5]}: "
                           f"got {got[bad[:5]]} want {want[bad[:5]]}")
    return float(np.mean(d == 0))


def assert_equal_bits(got, want, what=""):
    got = np.asarray(got).ravel()
    want = np.asarray(want).ravel()
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}: got {got[bad[:5]]} want {want[bad[:5]]}"


def sync():
    torch.cuda.synchronize()
