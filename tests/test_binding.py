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


def test_pointer_lists_must_have_the_lengths_the_call_reads(L):
    """The C side reads n_shards*R inputs, R outputs per rank list and so on from host pointer arrays; a
    short list is refused before the call (the addresses here are ints that no kernel ever sees)."""
    m = (1 << 20, 1 << 21)  # (codes, meta) device addresses that are never dereferenced
    a = 1 << 22
    with pytest.raises(ValueError, match="inputs: 3 entries, the call reads 4"):
        L.fc_reduce_shard([m] * 3, 2, 1024, 8, 8, 128, [m] * 2)
    with pytest.raises(ValueError, match="inputs: 5 entries, the call reads 4"):
        L.fc_reduce_shard_norm([m] * 5, 2, 1024, 8, 8, 128, dict(gamma=a, hidden=256), [m] * 2)
    with pytest.raises(ValueError, match="out: 1 entries, the call reads 2"):
        L.fc_ll_gather([a, a], 64, 64, 1, [a], a, a, a)
    with pytest.raises(ValueError, match="slots: 1 entries, the call reads 2"):
        L.fc_ll_pack([a, a], 64, 1, [a], n=1024)
    with pytest.raises(ValueError, match="block_order: 1 entries, the call reads 2"):
        L.fc_ll_pack([a, a], 64, 1, [a, a], block_order=[a], n=1024)
    with pytest.raises(ValueError, match="flags: 3 entries, the call reads 2"):
        L.fc_flag_unpack_reduce([a, a], [a, a, a], 1024, 512, 1, a, a, a, a)
    with pytest.raises(ValueError, match="payload: 1 entries, the call reads 2"):
        L.fc_flag_pack([a, a], 512, 1, [a], [a, a], n=1024)
    with pytest.raises(ValueError, match="flags: 1 entries, the call reads 2"):
        L.fc_flag_pack([a, a], 512, 1, [a, a], [a], n=1024)


def test_one_shard_index_is_range_checked():
    """TwoStepAllReduce.reduce_scatter(shard) offsets into its argument table: a shard outside [0, R) is
    refused before any pointer arithmetic (checked without building the object's device buffers)."""
    from tensor_all_reduce_amd.flash_allreduce import TwoStepAllReduce
    p = TwoStepAllReduce.__new__(TwoStepAllReduce)
    p.R = 4
    for bad in (-1, 4, 9):
        with pytest.raises(ValueError, match="shards 0 .. 3"):
            p.reduce_scatter(bad)


def test_epilogue_arguments_keep_their_tensors():
    """The epilogue structure holds raw addresses; it keeps the tensors it was built from, so temporaries
    passed to it stay allocated (checked with weak references; ints stand in for nothing here)."""
    import gc
    import weakref

    from tensor_all_reduce_amd import flash_allreduce as fa

    class Buf:  # stands in for a device tensor: _dev takes its address from an int subclass
        pass
    objs = [Buf() for _ in range(4)]
    refs = [weakref.ref(o) for o in objs]
    orig = fa._lib._dev
    fa._lib._dev = lambda t, nbytes=None, what="": None if t is None else 1 << 20
    try:
        nm = fa._norm_args(objs[0], objs[1], objs[2], objs[3], 1e-5, 256, 1024)
    finally:
        fa._lib._dev = orig
    del objs
    gc.collect()
    assert all(r() is not None for r in refs)
    del nm
    gc.collect()
    assert all(r() is None for r in refs)


def test_shapes_must_split_into_shards_of_whole_groups():
    """TwoStepAllReduce and TwoStepShare refuse shapes whose T*H does not split into R shards of whole
    groups, and a rank outside [0, R), before allocating anything."""
    from tensor_all_reduce_amd.flash_allreduce import TwoStepAllReduce, TwoStepShare
    for R, T, H, G in ((3, 4, 256, 32), (8, 1, 4096, 1024 // 2 + 64), (0, 4, 256, 32), (8, 2, 128, 64)):
        with pytest.raises(ValueError, match="shards of whole"):
            TwoStepAllReduce(R, T, H, 8, 8, G, device="cpu")
        with pytest.raises(ValueError, match="shards of whole"):
            TwoStepShare(R, T, H, 8, 8, G, device="cpu")
    for rank in (-1, 2):
        with pytest.raises(ValueError, match="outside"):
            TwoStepShare(2, 4, 256, 8, 8, 32, rank=rank, device="cpu")
