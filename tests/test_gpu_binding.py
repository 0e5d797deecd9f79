"""The binding refuses device tensors that are strided or too small for the call before any kernel is
enqueued (the kernels trust the sizes they are given), and accepts exactly-sized ones."""
import pytest

pytestmark = pytest.mark.gpu


def test_too_small_and_strided_buffers_are_refused():
    import torch
    from tensor_all_reduce_amd import _lib
    n, G = 4096, 128
    x = torch.zeros(n, dtype=torch.int16, device="cuda")
    codes = torch.empty(n, dtype=torch.uint8, device="cuda")
    meta = torch.empty(n // G, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="out codes"):
        _lib.fc_quantize(x, 8, G, codes[:-1], meta)            # one byte short
    with pytest.raises(ValueError, match="out meta"):
        _lib.fc_quantize(x, 8, G, codes, meta[:-1])
    with pytest.raises(ValueError, match="x:"):
        _lib.fc_quantize(x[: n - 8], 8, G, codes, meta, n=n)
    wide = torch.zeros(2, n, dtype=torch.int16, device="cuda")
    with pytest.raises(ValueError, match="contiguous"):
        _lib.fc_quantize(wide[:, :1].reshape(-1)[:1].expand(n), 8, G, codes, meta)
    with pytest.raises(ValueError, match="contiguous"):
        _lib.fc_quantize(wide.t(), 8, G, codes, meta, n=n)
    torch.cuda.synchronize()
    _lib.fc_quantize(x, 8, G, codes, meta)                     # exactly sized: runs
    torch.cuda.synchronize()
    assert int(codes.max()) == 0 and int(meta.max()) == 0      # a zero group: scale 0, zero 0, codes 0


def test_slot_receiver_checks_every_buffer():
    import torch
    from tensor_all_reduce_amd import _lib
    R, n, B = 2, 8192, 64
    nblk = n // 2 // B
    slots = [torch.zeros(n // 2, dtype=torch.int64, device="cuda") for _ in range(R)]
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    stale = torch.empty(R * nblk, dtype=torch.uint8, device="cuda")
    done = torch.zeros(nblk, dtype=torch.uint8, device="cuda")
    cnt = torch.zeros(2, dtype=torch.int32, device="cuda")
    for args, what in [((slots[:1] + [slots[1][:-1]], out, stale, done, cnt), "slots"),
                       ((slots, out[:-1], stale, done, cnt), "out"),
                       ((slots, out, stale[:-1], done, cnt), "stale"),
                       ((slots, out, stale, done[:-1], cnt), "done"),
                       ((slots, out, stale, done, cnt[:1]), "counters")]:
        s, o, st, d, c = args
        with pytest.raises(ValueError, match=what):
            _lib.fc_ll_unpack_reduce(s, n, B, 1, o, st, d, c)
    _lib.fc_ll_unpack_reduce(slots, n, B, 1, out, stale, done, cnt)  # epoch 1 against zero slots: all stale
    torch.cuda.synchronize()
    assert int(cnt[1]) == nblk and int(done.sum()) == 0
