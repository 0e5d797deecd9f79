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
    cnt = torch.zeros(_lib.COUNTER_WORDS, dtype=torch.int32, device="cuda")
    for args, what in [((slots[:1] + [slots[1][:-1]], out, stale, done, cnt), "slots"),
                       ((slots, out[:-1], stale, done, cnt), "out"),
                       ((slots, out, stale[:-1], done, cnt), "stale"),
                       ((slots, out, stale, done[:-1], cnt), "done"),
                       ((slots, out, stale, done, cnt[:-1]), "counters")]:
        s, o, st, d, c = args
        with pytest.raises(ValueError, match=what):
            _lib.fc_ll_unpack_reduce(s, n, B, 1, o, st, d, c)
    _lib.fc_ll_unpack_reduce(slots, n, B, 1, out, stale, done, cnt)  # epoch 1 against zero slots: all stale
    torch.cuda.synchronize()
    assert int(_lib.counter_totals(cnt)[1]) == nblk and int(done.sum()) == 0


def test_temporaries_passed_to_the_epilogue_stay_allocated():
    """make_norm with temporaries (gamma and residual uploaded inline), then new device buffers allocated
    and filled before the step runs: the epilogue must still read the residual and gamma it was given
    (the structure keeps them), which the oracle's output checks."""
    import numpy as np
    import torch

    import oracle
    from gpu_helpers import assert_bf16_close, assert_equal_bits, down, sync, up
    from tensor_all_reduce_amd import datagen as dg
    from tensor_all_reduce_amd.flash_allreduce import TwoStepAllReduce
    cfg = dg.DECODE_8B
    parts = dg.partials(cfg)
    res, gam = dg.residual(cfg), dg.gamma(cfg)
    p = TwoStepAllReduce(cfg.R, cfg.T, cfg.H, cfg.bits_rs, cfg.bits_ag, cfg.group, parts=up(np.stack(parts)))
    out = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    rout = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    norm = p.make_norm(up(gam), out, residual=up(res), residual_out=rout, eps=cfg.eps)
    # allocations of the same sizes, filled with other values, before the step
    junk = [torch.full((cfg.n,), 0x3F80, dtype=torch.int16, device="cuda"),
            torch.full((cfg.H,), -1, dtype=torch.int16, device="cuda")]
    p.run(norm=norm)
    sync()
    ref = oracle.two_step(parts, cfg.bits_rs, cfg.bits_ag, cfg.group, residual=res, gamma=gam, eps=cfg.eps,
                          hidden=cfg.H)
    assert_equal_bits(down(rout, np.uint16), ref["residual_out"], "residual_out")
    assert_bf16_close(down(out, np.uint16), ref["out"], 2, "out")
    del junk
