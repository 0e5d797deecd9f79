"""CPU tests of the Python binding's own checks: a tensor must be in device memory before its address
reaches a kernel (a host address would be dereferenced by the GPU), and helper objects refuse host
buffers.  These checks run before any HIP call, so they need no GPU."""
import pytest
import torch


@pytest.fixture(scope="module")
def L():
    from tensor_all_reduce_amd import _lib
    return _lib


def test_host_tensors_are_refused(L):
    x = torch.zeros(1024, dtype=torch.int16)
    codes, meta = torch.zeros(1024, dtype=torch.uint8), torch.zeros(8, dtype=torch.int32)
    with pytest.raises(ValueError, match="device memory"):
        L.fc_quantize(x, 8, 128, codes, meta)
    with pytest.raises(ValueError, match="device memory"):
        L.fc_reduce_shard([(codes, meta)], 1, 1024, 8, 8, 128, [(codes, meta)])
    with pytest.raises(ValueError, match="device memory"):
        L.fc_ll_unpack_reduce([torch.zeros(512, dtype=torch.int64)], 1024, 64, 1, x,
                              torch.zeros(8, dtype=torch.uint8), torch.zeros(8, dtype=torch.uint8),
                              torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="device memory"):
        L.fc_copy(x, x)


def test_other_argument_types_are_refused(L):
    with pytest.raises(TypeError):
        L.fc_copy([1, 2, 3], None, 4)


def test_helpers_refuse_host_buffers():
    from tensor_all_reduce_amd.flash_allreduce import TwoStepAllReduce, TwoStepShare
    with pytest.raises(ValueError, match="device memory"):
        TwoStepAllReduce(2, 4, 256, 8, 8, 32, device="cpu")
    with pytest.raises(ValueError, match="device memory"):
        TwoStepShare(2, 4, 256, 8, 8, 32, device="cpu")
