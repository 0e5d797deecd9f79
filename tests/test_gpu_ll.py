"""GPU parity of the self-synchronizing slots (fc_ll_pack, fc_ll_unpack_reduce; flash-comm) against the
CPU oracle: stale flags, done flags, counters and outputs bit-exact, on the 8-rank workload with its
seeded stale mix and shuffled write order, on every kind of wrong epoch word, and across a retry."""
import numpy as np
import pytest

from tensor_all_reduce_amd import datagen as dg

pytestmark = pytest.mark.gpu
M32 = 0xFFFFFFFF


@pytest.fixture(scope="module")
def fc():
    from tensor_all_reduce_amd import _lib
    return _lib


def set_epochs_host(slots, ep):
    s = slots.copy()
    s &= np.uint64(0xFFFFFFFF)
    s |= ep.astype(np.uint64) << np.uint64(32)
    return s


def inject_gpu(slots_d, ep):
    """Harness: overwrite the epoch words of a device slot buffer (emulates blocks that have not arrived)."""
    import torch
    v = slots_d.view(torch.int32).view(-1, 2)
    v[:, 1] = torch.from_numpy(ep.view(np.int32)).to(slots_d.device)


class GpuLL:
    def __init__(self, R, n, B):
        import torch
        from gpu_helpers import counters_buf
        self.R, self.n, self.B = R, n, B
        self.nblk = n // 2 // B
        self.out = torch.zeros(n, dtype=torch.int16, device="cuda")
        self.stale = torch.full((R * self.nblk,), 0xAB, dtype=torch.uint8, device="cuda")
        self.done = torch.zeros(self.nblk, dtype=torch.uint8, device="cuda")
        self.cnt = counters_buf()

    def run(self, fc, slots_d, epoch):
        self.cnt.zero_()
        fc.fc_ll_unpack_reduce(slots_d, self.n, self.B, epoch, self.out, self.stale, self.done, self.cnt)
        from gpu_helpers import counts, down
        return (down(self.out, np.uint16), down(self.stale, np.uint8).reshape(self.R, self.nblk),
                down(self.done, np.uint8), counts(self.cnt))


def test_pack_ranks_in_one_launch(fc, orc):
    """Three peers packed in one launch, one of them in ascending order: each equals the oracle's packing."""
    import torch
    from gpu_helpers import assert_equal_bits, down, up
    B, nblk, e = 64, 29, 0xABCDEF01
    n = 2 * B * nblk
    xs = [dg.synth_bf16((B, 3, r), n) for r in range(3)]
    orders = [np.random.default_rng(r).permutation(nblk).astype(np.int32) for r in range(3)]
    slots = [torch.empty(n // 2, dtype=torch.int64, device="cuda") for _ in range(3)]
    fc.fc_ll_pack([up(x) for x in xs], B, e, slots, block_order=[up(orders[0]), None, up(orders[2])], pace=1)
    for r in range(3):
        o = None if r == 1 else orders[r]
        assert_equal_bits(down(slots[r], np.uint64), orc.ll_pack(xs[r], B, e, order=o), f"slots {r}")


@pytest.mark.parametrize("B", [32, 64, 128, 256])
def test_pack_matches_oracle(fc, orc, B):
    import torch
    from gpu_helpers import assert_equal_bits, down, up
    n = 2 * B * 77
    x = dg.synth_bf16((B,), n)
    order = np.random.default_rng(B).permutation(n // 2 // B).astype(np.int32)
    for o in (None, order):
        slots = torch.empty(n // 2, dtype=torch.int64, device="cuda")
        fc.fc_ll_pack(up(x), B, 0xC0FFEE, slots, block_order=up(o) if o is not None else None)
        assert_equal_bits(down(slots, np.uint64), orc.ll_pack(x, B, 0xC0FFEE, order=o), "slots")


def test_workload_stale_mix_and_retry(fc, orc):
    """8 ranks x [128, 8192]: blocks written in a seeded order per rank, 2% of (rank, block) copies stale
    (mostly the previous epoch; also zero, next, inverted, top bit, random words and torn blocks).
    Pass 1 flags exactly the injected pairs and completes the rest; after the late blocks arrive a second
    pass completes every pending block with the same bits as an all-on-time run."""
    from gpu_helpers import assert_equal_bits, up
    import torch
    cfg = dg.SLOTS
    R, n, B, e = cfg.R, cfg.n, cfg.block_slots, cfg.epoch
    nslots, nblk = n // 2, n // 2 // B
    xs = [dg.partial(cfg, r) for r in range(R)]
    orders = [dg.write_order(cfg, r, nblk) for r in range(R)]
    eps, masks = zip(*[dg.stale_epochs(cfg, r, nslots) for r in range(R)])
    inj = np.stack(masks)
    # device: pack (sender emulation), then mark the late blocks
    slots_d = []
    for r in range(R):
        s = torch.empty(nslots, dtype=torch.int64, device="cuda")
        fc.fc_ll_pack(up(xs[r]), B, e, s, block_order=up(orders[r]))
        slots_d.append(s)
    for r in range(R):
        inject_gpu(slots_d[r], eps[r])
    g = GpuLL(R, n, B)
    out1, st1, dn1, c1 = g.run(fc, slots_d, e)
    # oracle, from the same bf16 inputs
    good = [orc.ll_pack(xs[r], B, e, order=orders[r]) for r in range(R)]
    late = [set_epochs_host(good[r], eps[r]) for r in range(R)]
    ro, rst, rdn, rc = orc.ll_unpack_reduce(late, n, B, e)
    assert_equal_bits(st1, rst, "stale flags")
    assert_equal_bits(st1, inj, "stale flags == injected")
    assert_equal_bits(dn1, rdn, "done")
    assert_equal_bits(c1, rc, "counters")
    assert c1[1] > 0.10 * nblk  # about 1 - 0.98^8 of the blocks are pending
    assert_equal_bits(out1[np.repeat(rdn.astype(bool), 2 * B)], ro[np.repeat(rdn.astype(bool), 2 * B)], "out (done)")
    assert np.all(out1[np.repeat(~rdn.astype(bool), 2 * B)] == 0), "pending blocks must stay untouched"
    # retry after the late blocks arrive
    for r in range(R):
        inject_gpu(slots_d[r], np.full(nslots, e, np.uint32))
    out2, st2, dn2, c2 = g.run(fc, slots_d, e)
    ro2, _, rdn2, rc2 = orc.ll_unpack_reduce(good, n, B, e, out=ro.copy(), done=rdn.copy())
    full, _, _, _ = orc.ll_unpack_reduce(good, n, B, e)
    assert dn2.all() and list(c2) == [0, 0] and list(rc2) == [0, 0]
    assert_equal_bits(out2, full, "retry == all on time")
    assert_equal_bits(out2, ro2, "retry == oracle retry")


STALE_WORDS = {
    "prev": lambda e: (e - 1) & M32, "next": lambda e: (e + 1) & M32, "zero": lambda e: 0 if e else 1,
    "not": lambda e: (~e) & M32, "msb": lambda e: e ^ 0x80000000, "lowbit": lambda e: e ^ 1,
}


@pytest.mark.parametrize("e", [0, 0x2A, 0xFFFFFFFF])
@pytest.mark.parametrize("kind", sorted(STALE_WORDS) + ["torn", "rank"])
@pytest.mark.parametrize("B", [32, 256])
def test_every_stale_word(fc, orc, e, kind, B):
    import torch
    from gpu_helpers import assert_equal_bits, up
    R, nblk = 3, 40
    n = 2 * B * nblk
    xs = [dg.synth_bf16((B, r, 4), n) for r in range(R)]
    eps = [np.full(n // 2, e, np.uint32) for _ in range(R)]
    rng = np.random.default_rng(B)
    if kind == "rank":
        eps[1][:] = (e - 1) & M32
    else:
        for b in rng.choice(nblk, 5, replace=False):
            r = int(rng.integers(0, R))
            if kind == "torn":
                eps[r][b * B + int(rng.integers(0, B))] = (e - 1) & M32
            else:
                eps[r][b * B:(b + 1) * B] = STALE_WORDS[kind](e)
    slots_d = []
    for r in range(R):
        s = torch.empty(n // 2, dtype=torch.int64, device="cuda")
        fc.fc_ll_pack(up(xs[r]), B, e, s)
        inject_gpu(s, eps[r])
        slots_d.append(s)
    g = GpuLL(R, n, B)
    out, st, dn, c = g.run(fc, slots_d, e)
    late = [set_epochs_host(orc.ll_pack(xs[r], B, e), eps[r]) for r in range(R)]
    ro, rst, rdn, rc = orc.ll_unpack_reduce(late, n, B, e)
    assert_equal_bits(st, rst, "stale")
    assert_equal_bits(dn, rdn, "done")
    assert_equal_bits(c, rc, "counters")
    assert_equal_bits(out, ro, "out")


@pytest.mark.parametrize("R", [1, 2, 16])
def test_rank_counts_and_done_skip(fc, orc, R):
    """R from 1 to 16; blocks already done are skipped (flags and outputs untouched, nothing counted)."""
    import torch
    from gpu_helpers import assert_equal_bits, down, up
    B, nblk, e = 64, 33, 5
    n = 2 * B * nblk
    xs = [dg.synth_bf16((R, r, 6), n) for r in range(R)]
    slots_d = []
    for r in range(R):
        s = torch.empty(n // 2, dtype=torch.int64, device="cuda")
        fc.fc_ll_pack(up(xs[r]), B, e - 1, s)   # nothing has arrived: every copy stale
        slots_d.append(s)
    g = GpuLL(R, n, B)
    done0 = (np.arange(nblk) % 3 == 0).astype(np.uint8)
    g.done.copy_(torch.from_numpy(done0))
    g.out.fill_(77)
    out, st, dn, c = g.run(fc, slots_d, e)
    ro, rst, rdn, rc = orc.ll_unpack_reduce([orc.ll_pack(x, B, e - 1) for x in xs], n, B, e,
                                            out=np.full(n, 77, np.uint16), done=done0.copy())
    assert_equal_bits(dn, rdn, "done")
    assert_equal_bits(c, rc, "counters")
    assert_equal_bits(out, ro, "out")
    # flags: examined blocks per the oracle; skipped blocks keep the sentinel the buffer started with
    skipped = done0.astype(bool)
    assert np.all(st[:, skipped] == 0xAB)
    assert_equal_bits(st[:, ~skipped], rst[:, ~skipped], "stale (examined)")


def test_receivers_without_counters(fc, orc):
    """counters = NULL: nothing is counted and no atomic is issued; out, stale and done are the same bits
    as with counters, and as the oracle's, for the slot receiver (8-rank workload with its stale mix, both
    passes), the standalone all-gather, the polling slot receiver and the flag receiver."""
    import torch
    from gpu_helpers import assert_equal_bits, counters_buf, down, up
    cfg = dg.SLOTS
    R, n, B, e = cfg.R, cfg.n, cfg.block_slots, cfg.epoch
    nslots, nblk = n // 2, n // 2 // B
    xs = [dg.partial(cfg, r) for r in range(R)]
    orders = [dg.write_order(cfg, r, nblk) for r in range(R)]
    eps = [dg.stale_epochs(cfg, r, nslots)[0] for r in range(R)]
    slots_d = []
    for r in range(R):
        s = torch.empty(nslots, dtype=torch.int64, device="cuda")
        fc.fc_ll_pack(up(xs[r]), B, e, s, block_order=up(orders[r]))
        inject_gpu(s, eps[r])
        slots_d.append(s)
    late = [set_epochs_host(orc.ll_pack(xs[r], B, e, order=orders[r]), eps[r]) for r in range(R)]
    ro, rst, rdn, _ = orc.ll_unpack_reduce(late, n, B, e)
    res = {}
    for tag, cnt in (("counted", counters_buf()), ("uncounted", None)):
        out = torch.zeros(n, dtype=torch.int16, device="cuda")
        st = torch.full((R * nblk,), 0xAB, dtype=torch.uint8, device="cuda")
        dn = torch.zeros(nblk, dtype=torch.uint8, device="cuda")
        fc.fc_ll_unpack_reduce(slots_d, n, B, e, out, st, dn, cnt)
        torch.cuda.synchronize()
        res[tag] = (down(out, np.uint16), down(st, np.uint8).reshape(R, nblk), down(dn, np.uint8))
    for a, b, what in zip(res["counted"], res["uncounted"], ("out", "stale", "done")):
        assert_equal_bits(b, a, what + " without counters")
    assert_equal_bits(res["uncounted"][1], rst, "stale vs oracle")
    assert_equal_bits(res["uncounted"][2], rdn, "done vs oracle")
    ok = np.repeat(rdn.astype(bool), 2 * B)
    assert_equal_bits(res["uncounted"][0][ok], ro[ok], "out of completed blocks vs oracle")
    # standalone all-gather on the same slots (rank r's words = its packed payload)
    outs = [torch.zeros(nslots, dtype=torch.int32, device="cuda") for _ in range(R)]
    gst = torch.full((R * nblk,), 0xAB, dtype=torch.uint8, device="cuda")
    gdn = torch.zeros(R * nblk, dtype=torch.uint8, device="cuda")
    fc.fc_ll_gather(slots_d, nslots, B, e, outs, gst, gdn, None)
    torch.cuda.synchronize()
    rg_out, rg_st, rg_dn, _ = orc.ll_gather(late, nslots, B, e)
    assert_equal_bits(down(gst, np.uint8).ravel(), np.asarray(rg_st).ravel(), "all-gather stale without counters")
    assert_equal_bits(down(gdn, np.uint8).ravel(), np.asarray(rg_dn).ravel(), "all-gather done without counters")
    # polling slot receiver and flag receiver, every copy on time
    st2 = torch.empty(R * nblk, dtype=torch.uint8, device="cuda")
    dn2 = torch.zeros(nblk, dtype=torch.uint8, device="cuda")
    out2 = torch.zeros(n, dtype=torch.int16, device="cuda")
    good = [s.clone() for s in slots_d]
    for r in range(R):
        inject_gpu(good[r], np.full(nslots, e, np.uint32))
    fc.fc_ll_poll_unpack_reduce(good, n, B, e, out2, st2, dn2, None, max_polls=2)
    torch.cuda.synchronize()
    ro2, _, _, _ = orc.ll_unpack_reduce([orc.ll_pack(xs[r], B, e, order=orders[r]) for r in range(R)], n, B, e)
    assert_equal_bits(down(out2, np.uint16), ro2, "polling receiver out without counters")
    assert int(down(dn2, np.uint8).sum()) == nblk
    be = 2048
    pays = [torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(R)]
    fls = [torch.empty(n // be, dtype=torch.int32, device="cuda") for _ in range(R)]
    fc.fc_flag_pack([up(x) for x in xs], be, e, pays, fls)
    fb = n // be
    out3 = torch.zeros(n, dtype=torch.int16, device="cuda")
    st3 = torch.empty(R * fb, dtype=torch.uint8, device="cuda")
    dn3 = torch.zeros(fb, dtype=torch.uint8, device="cuda")
    fc.fc_flag_unpack_reduce(pays, fls, n, be, e, out3, st3, dn3, None, max_polls=1)
    torch.cuda.synchronize()
    assert_equal_bits(down(out3, np.uint16), ro2, "flag receiver out without counters")
    assert int(down(dn3, np.uint8).sum()) == fb
