"""The hot path captured in HIP graphs, as the benchmark times it, and replayed several times.  Before each
replay every output is poisoned and other eager work runs, with synchronizations in between; every replay
must then give the oracle's result (codes, meta, flags and counters bit-exact, bf16 within 2 ulp where the
other tests allow it).  The library issues no memset, allocation or host synchronization, so a captured
call is the same launches as an eager one; these tests check that replays agree with that.  The first
call of each case is eager (the warm-up), the capture follows."""
import numpy as np
import pytest

from tensor_all_reduce_amd import datagen as dg

pytestmark = pytest.mark.gpu
REPLAYS = 3


@pytest.fixture(scope="module")
def fc():
    from tensor_all_reduce_amd import _lib
    return _lib


def _capture(fn):
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def _between(bufs, i):
    """Eager work between replays: poison the outputs (a replay that wrote nothing would keep the poison)
    and run unrelated kernels, then synchronize."""
    import torch
    for b in bufs:
        b.view(torch.uint8).fill_(0xA5 ^ i)
    x = torch.randn(1 << 20, device="cuda")
    x.mul_(2.0).add_(1.0)
    torch.cuda.synchronize()


@pytest.mark.parametrize("workload", ["tiny-r2-t4-h256", "llama3-8b-decode"])
def test_two_step_replays(fc, orc, workload):
    import torch
    from gpu_helpers import assert_bf16_close, assert_equal_bits, down, up
    from tensor_all_reduce_amd.flash_allreduce import TwoStepAllReduce
    cfg = dg.WORKLOADS[workload]
    parts = dg.partials(cfg)
    res, gam = dg.residual(cfg), dg.gamma(cfg)
    ref = orc.two_step(parts, cfg.bits_rs, cfg.bits_ag, cfg.group, residual=res, gamma=gam, eps=cfg.eps, hidden=cfg.H)
    p = TwoStepAllReduce(cfg.R, cfg.T, cfg.H, cfg.bits_rs, cfg.bits_ag, cfg.group, parts=up(np.stack(parts)))
    y = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    out = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    rout = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    norm = p.make_norm(up(gam), out, residual=up(res), residual_out=rout, eps=cfg.eps)
    g = _capture(lambda: p.run(y=y, norm=norm))
    for i in range(REPLAYS):
        _between([p.codes1, p.meta1, p.codes2, p.meta2, y, out, rout], i)
        g.replay()
        torch.cuda.synchronize()
        where = f"{workload} replay {i}"
        assert_equal_bits(down(p.codes1, np.uint8).ravel(), ref["codes1"].ravel(), "codes1 " + where)
        assert_equal_bits(down(p.meta1, np.uint32).ravel(), ref["meta1"].ravel(), "meta1 " + where)
        assert_equal_bits(down(p.codes2, np.uint8), ref["codes2"], "codes2 " + where)
        assert_equal_bits(down(p.meta2, np.uint32), ref["meta2"], "meta2 " + where)
        assert_equal_bits(down(y, np.uint16), ref["y"], "y " + where)
        assert_equal_bits(down(rout, np.uint16), ref["residual_out"], "residual_out " + where)
        assert_bf16_close(down(out, np.uint16), ref["out"], 2, "out " + where)


def test_norm_first_replays(fc, orc):
    """The norm-first path (quantize, reduce + norm per shard, gather of the normalized rows) on the decode
    workload, against the oracle in the kernels' sum-of-squares order (bit-exact)."""
    import torch
    from gpu_helpers import assert_equal_bits, down, up
    from tensor_all_reduce_amd.flash_allreduce import TwoStepAllReduce
    cfg = dg.DECODE_8B
    parts = dg.partials(cfg)
    res, gam = dg.residual(cfg), dg.gamma(cfg)
    ref = orc.two_step_normfirst(parts, cfg.bits_rs, cfg.bits_ag, cfg.group, res, gam, cfg.eps, cfg.H, order="tree")
    p = TwoStepAllReduce(cfg.R, cfg.T, cfg.H, cfg.bits_rs, cfg.bits_ag, cfg.group, parts=up(np.stack(parts)))
    y = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    rout = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    norm = p.make_norm(up(gam), None, residual=up(res), residual_out=rout, eps=cfg.eps)
    g = _capture(lambda: p.run_norm_first(y, norm))
    for i in range(REPLAYS):
        _between([p.codes2, p.meta2, y, rout], i)
        g.replay()
        torch.cuda.synchronize()
        assert_equal_bits(down(p.codes2, np.uint8), ref["codes2"], f"codes2 replay {i}")
        assert_equal_bits(down(p.meta2, np.uint32), ref["meta2"], f"meta2 replay {i}")
        assert_equal_bits(down(rout, np.uint16), ref["residual_out"], f"residual_out replay {i}")
        assert_equal_bits(down(y, np.uint16), ref["y"], f"y replay {i}")


@pytest.mark.parametrize("max_workgroups", [0, 16])
def test_reduce_rmsnorm_replays(fc, orc, max_workgroups):
    """The unquantized reduce + RMSNorm (8 ranks x [96, 8192]), one workgroup per row or a capped grid."""
    import torch
    from gpu_helpers import assert_bf16_close, assert_equal_bits, down, up
    from tensor_all_reduce_amd.flash_allreduce import ReduceRMSNorm
    R, rows, H = 8, 96, 8192
    rng = np.random.default_rng(96)
    bf = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    parts_h = [bf(rng.standard_normal(rows * H)) for _ in range(R)]
    res_h, gam_h = bf(rng.standard_normal(rows * H)), bf(1.0 + 0.1 * rng.standard_normal(H))
    o, ro, _ = orc.reduce_rmsnorm(parts_h, rows, H, res_h, gam_h, 1e-5)
    parts = [up(x) for x in parts_h]
    out = torch.empty(rows * H, dtype=torch.int16, device="cuda")
    rout = torch.empty(rows * H, dtype=torch.int16, device="cuda")
    rr = ReduceRMSNorm(parts, rows, H, up(gam_h), out, residual=up(res_h), residual_out=rout, eps=1e-5)
    g = _capture(lambda: rr.run(max_workgroups=max_workgroups))
    for i in range(REPLAYS):
        _between([out, rout], i)
        g.replay()
        torch.cuda.synchronize()
        assert_equal_bits(down(rout, np.uint16), ro, f"residual_out replay {i}")
        assert_bf16_close(down(out, np.uint16), o, 2, f"out replay {i}")


def test_slot_receiver_replays(fc, orc):
    """The slot receiver's first pass on the 8-rank slot workload (2% of the (rank, block) copies late):
    between replays the done flags and counters are reset and out, stale poisoned; each replay flags the
    same pairs, completes the same blocks with the oracle's bits and leaves the pending ones untouched."""
    import torch
    from gpu_helpers import assert_equal_bits, counters_buf, counts, down, up
    from tensor_all_reduce_amd.flash_allreduce import LLUnpackReduce
    cfg = dg.SLOTS
    R, n, B, e = cfg.R, cfg.n, cfg.block_slots, cfg.epoch
    nslots, nblk = n // 2, n // 2 // B
    late = []
    for r in range(R):
        good = orc.ll_pack(dg.partial(cfg, r), B, e, order=dg.write_order(cfg, r, nblk))
        ep, _ = dg.stale_epochs(cfg, r, nslots)
        late.append((good & np.uint64(0xFFFFFFFF)) | (ep.astype(np.uint64) << np.uint64(32)))
    ro, rst, rdn, rc = orc.ll_unpack_reduce(late, n, B, e)
    slots = [up(s) for s in late]
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    stale = torch.empty(R * nblk, dtype=torch.uint8, device="cuda")
    done = torch.zeros(nblk, dtype=torch.uint8, device="cuda")
    cnt = counters_buf()
    rx = LLUnpackReduce(slots, n, B, out, stale, done, cnt)
    g = _capture(lambda: rx.run(e))
    fin = np.repeat(rdn.astype(bool), 2 * B)
    for i in range(REPLAYS):
        _between([out, stale], i)
        done.zero_()
        cnt.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o = down(out, np.uint16)
        assert_equal_bits(down(stale, np.uint8), rst.ravel(), f"stale replay {i}")
        assert_equal_bits(down(done, np.uint8), rdn, f"done replay {i}")
        assert_equal_bits(counts(cnt), rc, f"counters replay {i}")
        assert_equal_bits(o[fin], ro[fin], f"out of completed blocks, replay {i}")
        assert np.all(o[~fin] == (0xA5 ^ i) * 0x0101), f"pending blocks written, replay {i}"


@pytest.mark.parametrize("counted", [True, False])
def test_all_gather_on_slots_replays(fc, orc, counted):
    """The standalone all-gather on slots (8 ranks, 64-slot blocks, about 10% of the copies late, every
    kind of wrong epoch word): between replays done, stale, counters and the outputs are reset or
    poisoned; each replay copies the same blocks with the payload's bits and leaves the late ones pending."""
    import torch
    from gpu_helpers import assert_equal_bits, counters_buf, counts, down, up
    R, B, nblk, e = 8, 64, 300, 0x2A
    nw = B * nblk
    rng = np.random.default_rng(0x6A)
    words = [rng.integers(0, 1 << 32, nw, dtype=np.uint64) for _ in range(R)]
    slots_h = []
    for r in range(R):
        ep = np.full(nw, e, np.uint64)
        for b in np.nonzero(rng.random(nblk) < 0.1)[0]:
            if rng.random() < 0.5:
                ep[b * B:(b + 1) * B] = int(rng.choice([e - 1, 0, e + 1, 0xFFFFFFFF ^ e]))
            else:
                ep[b * B + int(rng.integers(B))] = e - 1
        slots_h.append((words[r] & np.uint64(0xFFFFFFFF)) | (ep << np.uint64(32)))
    ro, rst, rdn, rc = orc.ll_gather(slots_h, nw, B, e)
    slots = [up(s) for s in slots_h]
    outs = [torch.empty(nw, dtype=torch.int32, device="cuda") for _ in range(R)]
    stale = torch.empty(R * nblk, dtype=torch.uint8, device="cuda")
    done = torch.zeros(R * nblk, dtype=torch.uint8, device="cuda")
    cnt = counters_buf() if counted else None

    def call():
        fc.fc_ll_gather(slots, nw, B, e, outs, stale, done, cnt)
    g = _capture(call)
    for i in range(REPLAYS):
        _between(outs + [stale], i)
        done.zero_()
        if counted:
            cnt.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        where = f"counted={counted} replay {i}"
        assert_equal_bits(down(stale, np.uint8), np.asarray(rst).ravel(), "stale " + where)
        assert_equal_bits(down(done, np.uint8), np.asarray(rdn).ravel(), "done " + where)
        if counted:
            assert_equal_bits(counts(cnt), rc, "counters " + where)
        fin = np.asarray(rdn).reshape(R, nblk).astype(bool)
        for r in range(R):
            o = down(outs[r], np.uint32)
            ok = np.repeat(fin[r], B)
            assert_equal_bits(o[ok], ro[r][ok], f"out[{r}] of copied blocks, " + where)
            assert np.all(o[~ok] == np.uint32((0xA5 ^ i) * 0x01010101)), f"pending blocks of rank {r} written, {where}"


def test_flag_receiver_replays(fc, orc):
    """The flag receiver (8 ranks, 2048-element blocks, 15% of the flags wrong, a poll budget of 2, a
    capped grid): every replay gives the oracle's out, stale, done and the same re-read count."""
    import torch
    from gpu_helpers import assert_equal_bits, counters_buf, counts, down, up
    cfg = dg.SLOTS
    R, be, nblk, e = 8, 2048, 96, 0x51
    n = be * nblk
    xs = [dg.synth_bf16((be, R, r, 3), n) for r in range(R)]
    fls, _ = zip(*[dg.stale_flags(cfg, r, nblk, epoch=e, p=0.15, salt=77) for r in range(R)])
    ro, rst, rdn, rc = orc.flag_unpack_reduce(xs, fls, n, be, e)
    pay, fl = [up(x) for x in xs], [up(f) for f in fls]
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    stale = torch.empty(R * nblk, dtype=torch.uint8, device="cuda")
    done = torch.zeros(nblk, dtype=torch.uint8, device="cuda")
    cnt = counters_buf()

    def call():
        fc.fc_flag_unpack_reduce(pay, fl, n, be, e, out, stale, done, cnt, max_polls=2, max_workgroups=7)
    done.zero_()
    cnt.zero_()
    g = _capture(call)
    rereads = None
    fin = np.repeat(np.asarray(rdn).astype(bool), be)
    for i in range(REPLAYS):
        _between([out, stale], i)
        done.zero_()
        cnt.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        c = counts(cnt, 4)
        assert_equal_bits(down(stale, np.uint8), np.asarray(rst).ravel(), f"stale replay {i}")
        assert_equal_bits(down(done, np.uint8), rdn, f"done replay {i}")
        assert_equal_bits(c[:2], rc, f"counters replay {i}")
        rereads = c[2] if rereads is None else rereads
        assert c[2] == rereads and c[3] == 0, f"re-reads replay {i}"
        o = down(out, np.uint16)
        assert_equal_bits(o[fin], ro[fin], f"out of completed blocks, replay {i}")
        assert np.all(o[~fin] == (0xA5 ^ i) * 0x0101), f"pending blocks written, replay {i}"


def test_one_gpu_share_replays(fc, orc):
    """One GPU's share (rank 5 of the decode workload: its quantize, the reduce of shard 5, the gather +
    epilogue of all shards), captured and replayed; the peers' chunks and the other shards' payloads are
    the oracle's.  Every replay must rebuild the own message, the own shard's payload and the outputs."""
    import torch
    from gpu_helpers import assert_bf16_close, assert_equal_bits, down, up
    from tensor_all_reduce_amd.flash_allreduce import TwoStepShare
    cfg, rank = dg.DECODE_8B, 5
    R, L, G, b1, b2 = cfg.R, cfg.L, cfg.group, cfg.bits_rs, cfg.bits_ag
    parts = dg.partials(cfg)
    res, gam = dg.residual(cfg), dg.gamma(cfg)
    ref = orc.two_step(parts, b1, b2, G, residual=res, gamma=gam, eps=cfg.eps, hidden=cfg.H, plain=False)
    sh = TwoStepShare(R, cfg.T, cfg.H, b1, b2, G, rank=rank, x=up(parts[rank]))
    cb1, cb2, mb = L * b1 // 8, L * b2 // 8, L // G
    for r in range(R):
        if r != rank:
            sh.inbox_codes[r].copy_(up(ref["codes1"][r, rank * cb1:(rank + 1) * cb1]).view(torch.uint8))
            sh.inbox_meta[r].copy_(up(ref["meta1"][r, rank * mb:(rank + 1) * mb]).view(torch.int32))
    for s in range(R):
        if s != rank:
            sh.codes2[s].copy_(up(ref["codes2"][s * cb2:(s + 1) * cb2]).view(torch.uint8))
            sh.meta2[s].copy_(up(ref["meta2"][s * mb:(s + 1) * mb]).view(torch.int32))
    out = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    rout = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    norm = sh.make_norm(up(gam), out, residual=up(res), residual_out=rout, eps=cfg.eps)
    g = _capture(lambda: sh.run(norm=norm))
    for i in range(REPLAYS):
        _between([sh.codes1, sh.meta1, sh.codes2[rank], sh.meta2[rank], out, rout], i)
        g.replay()
        torch.cuda.synchronize()
        where = f"replay {i}"
        assert_equal_bits(down(sh.meta1, np.uint32), ref["meta1"][rank], "own message: meta, " + where)
        assert_equal_bits(down(sh.codes1, np.uint8), ref["codes1"][rank], "own message: codes, " + where)
        assert_equal_bits(down(sh.meta2[rank], np.uint32), ref["meta2"][rank * mb:(rank + 1) * mb],
                          "own shard: meta, " + where)
        assert_equal_bits(down(sh.codes2[rank], np.uint8), ref["codes2"][rank * cb2:(rank + 1) * cb2],
                          "own shard: codes, " + where)
        assert_equal_bits(down(rout, np.uint16), ref["residual_out"], "residual_out " + where)
        assert_bf16_close(down(out, np.uint16), ref["out"], 2, "out " + where)
