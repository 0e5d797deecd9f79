"""GPU checks of the bandwidth-measurement helper (fc_bandwidth_probe): the copy copies, the writer writes
its documented pattern over exactly the requested range, and the reader leaves its sink alone unless a
lane's fold hits the fixed value (predicted here on the host)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu
SENTINEL = 0x9E3779B9


@pytest.fixture(scope="module")
def fc():
    from tensor_all_reduce_amd import _lib
    return _lib


def test_copy_write_read(fc):
    import torch
    nb = (1 << 20) + 4096 + 16  # a ragged last workgroup tile
    rng = np.random.default_rng(5)
    src_h = rng.integers(0, 256, nb, dtype=np.uint8)
    src = torch.from_numpy(src_h).cuda()
    dst = torch.zeros(nb + 64, dtype=torch.uint8, device="cuda")
    fc.fc_bandwidth_probe(src, dst, nb, 0)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    assert np.array_equal(got[:nb], src_h) and not got[nb:].any()
    # writer: uint4 i holds (0x3F803F80, i, 0, 0), over exactly the requested range
    dst.zero_()
    fc.fc_bandwidth_probe(None, dst, nb, 2)
    torch.cuda.synchronize()
    w = dst.cpu().numpy()[:nb].view(np.uint32).reshape(-1, 4)
    i = np.arange(w.shape[0])
    assert np.all(w[:, 0] == 0x3F803F80) and np.array_equal(w[:, 1], i)
    assert not w[:, 2:].any() and not dst.cpu().numpy()[nb:].any()
    # reader: each lane folds one uint4 (lanes past the end re-read the last one); the sink is written only
    # if some fold hits the fixed value.  First random data (no fold hits), then a source planted with one
    # uint4 whose fold is the value.
    v = src_h.view(np.uint32).reshape(-1, 4)
    folds = np.bitwise_xor.reduce(v, axis=1)
    for planted in (False, True):
        if planted:
            v = v.copy()
            v[12345] = (SENTINEL ^ 0x11 ^ 0x22 ^ 0x33, 0x11, 0x22, 0x33)
            folds = np.bitwise_xor.reduce(v, axis=1)
            src = torch.from_numpy(v.view(np.uint8).reshape(-1)).cuda()
        sink = torch.full((1,), 0x0BADF00D, dtype=torch.int32, device="cuda")
        fc.fc_bandwidth_probe(src, sink, nb, 1)
        torch.cuda.synchronize()
        hit = bool(np.any(folds == SENTINEL))
        assert hit == planted
        assert (int(sink.cpu()[0]) & 0xFFFFFFFF) == (SENTINEL if hit else 0x0BADF00D)
