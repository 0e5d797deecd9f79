"""GPU parity of the readiness encodings that are read while the senders write (flash-comm, abstract:
self-synchronizing transfers; the protocol selector picks the readiness encoding):

  * one flag word per block (fc_flag_pack, fc_flag_unpack_reduce) against the oracle's flag receiver,
  * the polling receiver of 8-byte slots (fc_ll_poll_unpack_reduce) against the oracle's slot receiver,

bit-exact in outputs, stale flags, done flags and counters, with every kind of wrong flag word, blocks
already done, 1 to 16 ranks, ragged tile counts, and a poll budget that cannot change a verdict when the
senders have finished.  Then the live case: the receiver starts first on one stream and spins (bounded)
while a paced sender on a second stream writes the blocks in a shuffled order, for two epochs in a row
on the same buffers; the result must equal the oracle's with every block on time."""
import dataclasses
import time

import numpy as np
import pytest

from tensor_all_reduce_amd import datagen as dg

pytestmark = pytest.mark.gpu
M32 = 0xFFFFFFFF


@pytest.fixture(scope="module")
def fc():
    from tensor_all_reduce_amd import _lib
    return _lib


def _bufs(R, n, nblk, out_fill=0, done0=None):
    import torch
    from gpu_helpers import counters_buf
    out = torch.full((n,), out_fill, dtype=torch.int16, device="cuda")
    stale = torch.full((R * nblk,), 0xAB, dtype=torch.uint8, device="cuda")
    done = torch.zeros(nblk, dtype=torch.uint8, device="cuda")
    if done0 is not None:
        done.copy_(torch.from_numpy(done0))
    cnt = counters_buf()
    return out, stale, done, cnt


def _down_all(out, stale, done, cnt, R, nblk):
    from gpu_helpers import counts, down
    return (down(out, np.uint16), down(stale, np.uint8).reshape(R, nblk), down(done, np.uint8),
            counts(cnt, 4))


def _tiles_polled(stale_rb, done0, group):
    """Tiles (`group` consecutive blocks) holding a block not done with a stale copy: each of them spends
    the whole poll budget when nothing changes."""
    bad = (stale_rb.any(axis=0)) & (done0 == 0)
    nt = -(-bad.size // group)
    padded = np.zeros(nt * group, bool)
    padded[:bad.size] = bad
    return int(padded.reshape(nt, group).any(axis=1).sum())


# ---------------------------------------------------------------------------------------------------
# flag encoding, senders finished before the receiver starts
# ---------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("polls", [0, 3])
@pytest.mark.parametrize("R", [1, 3, 8, 16])
@pytest.mark.parametrize("be,nblk", [(512, 37), (1024, 21), (4096, 9), (65536, 3)])
def test_flag_receiver_matches_oracle(fc, orc, be, nblk, R, polls):
    from gpu_helpers import assert_equal_bits, up
    cfg = dg.SLOTS
    n, e = be * nblk, 0xFFFFFFFF if R == 3 else 0x2A
    xs = [dg.synth_bf16((be, R, r), n) for r in range(R)]
    fls, masks = zip(*[dg.stale_flags(cfg, r, nblk, epoch=e, p=0.15, salt=be * 100 + R) for r in range(R)])
    done0 = (np.arange(nblk) % 5 == 2).astype(np.uint8)
    out, stale, done, cnt = _bufs(R, n, nblk, out_fill=77, done0=done0)
    fc.fc_flag_unpack_reduce([up(x) for x in xs], [up(f) for f in fls], n, be, e, out, stale, done, cnt,
                             max_polls=polls)
    got_out, got_st, got_dn, got_c = _down_all(out, stale, done, cnt, R, nblk)
    ro, rst, rdn, rc = orc.flag_unpack_reduce(xs, fls, n, be, e, out=np.full(n, 77, np.uint16), done=done0)
    rst = rst.reshape(R, nblk)
    assert_equal_bits(got_out, ro, "out")
    assert_equal_bits(got_dn, rdn, "done")
    assert_equal_bits(got_c[:2], rc, "counters")
    skipped = done0.astype(bool)
    assert np.all(got_st[:, skipped] == 0xAB), "blocks already done are not examined"
    assert_equal_bits(got_st[:, ~skipped], rst[:, ~skipped], "stale (examined)")
    assert_equal_bits(got_st[:, ~skipped], np.stack(masks)[:, ~skipped], "stale == injected")
    want_polls = polls * _tiles_polled(np.stack(masks).astype(bool), done0, max(1, 2048 // be))
    assert int(got_c[2]) == want_polls and int(got_c[3]) == 0



@pytest.mark.parametrize("mw", [1, 3, 7])
@pytest.mark.parametrize("be,nblk,R,polls", [(512, 37, 8, 3), (4096, 9, 3, 0), (2048, 40, 16, 2)])
def test_flag_receiver_capped_grid(fc, orc, be, nblk, R, polls, mw):
    """A grid capped below the tile count: each workgroup walks several tiles (reading the next tile's
    flags ahead), with the same outputs, stale flags and re-read count as the oracle says."""
    from gpu_helpers import assert_equal_bits, up
    cfg = dg.SLOTS
    n, e = be * nblk, 0x2A
    xs = [dg.synth_bf16((be, R, r, mw), n) for r in range(R)]
    fls, masks = zip(*[dg.stale_flags(cfg, r, nblk, epoch=e, p=0.15, salt=be * 100 + R + 7) for r in range(R)])
    done0 = (np.arange(nblk) % 7 == 3).astype(np.uint8)
    out, stale, done, cnt = _bufs(R, n, nblk, out_fill=77, done0=done0)
    fc.fc_flag_unpack_reduce([up(x) for x in xs], [up(f) for f in fls], n, be, e, out, stale, done, cnt,
                             max_polls=polls, max_workgroups=mw)
    got_out, got_st, got_dn, got_c = _down_all(out, stale, done, cnt, R, nblk)
    ro, rst, rdn, rc = orc.flag_unpack_reduce(xs, fls, n, be, e, out=np.full(n, 77, np.uint16), done=done0)
    rst = rst.reshape(R, nblk)
    assert_equal_bits(got_out, ro, "out")
    assert_equal_bits(got_dn, rdn, "done")
    assert_equal_bits(got_c[:2], rc, "counters")
    skipped = done0.astype(bool)
    assert np.all(got_st[:, skipped] == 0xAB), "blocks already done are not examined"
    assert_equal_bits(got_st[:, ~skipped], rst[:, ~skipped], "stale (examined)")
    want_polls = polls * _tiles_polled(np.stack(masks).astype(bool), done0, max(1, 2048 // be))
    assert int(got_c[2]) == want_polls and int(got_c[3]) == 0


@pytest.mark.parametrize("be,nblk", [(512, 45), (2048, 45), (512, 8192 + 3)])
def test_flag_pack_round_trip(fc, orc, be, nblk):
    """The sender writes every block (shuffled order) and its flag; the receiver completes every block.
    The last case is a message large enough for the widest fence span (256 blocks of 512 per fence) and
    ends in a ragged span."""
    import torch
    from gpu_helpers import assert_equal_bits, down, up
    R, e = 4, 9
    n = be * nblk
    xs = [dg.synth_bf16((be, 7, r), n) for r in range(R)]
    pays = [torch.zeros(n, dtype=torch.int16, device="cuda") for _ in range(R)]
    fls = [torch.full((nblk,), e - 1, dtype=torch.int32, device="cuda") for _ in range(R)]
    orders = [up(np.random.default_rng(r).permutation(nblk).astype(np.int32)) for r in range(R)]
    # ranks 0 and 1 in one launch (two peers at once), ranks 2 and 3 one launch each
    fc.fc_flag_pack([up(xs[0]), up(xs[1])], be, e, pays[:2], fls[:2], block_order=orders[:2])
    for r in (2, 3):
        fc.fc_flag_pack(up(xs[r]), be, e, pays[r], fls[r], block_order=orders[r] if r == 2 else None)
    for r in range(R):
        assert_equal_bits(down(pays[r], np.uint16), xs[r], f"payload {r}")
        assert_equal_bits(down(fls[r], np.uint32), np.full(nblk, e, np.uint32), f"flags {r}")
    out, stale, done, cnt = _bufs(R, n, nblk)
    fc.fc_flag_unpack_reduce(pays, fls, n, be, e, out, stale, done, cnt)
    got_out, got_st, got_dn, got_c = _down_all(out, stale, done, cnt, R, nblk)
    ro, rst, rdn, rc = orc.flag_unpack_reduce(xs, [np.full(nblk, e, np.uint32)] * R, n, be, e)
    assert_equal_bits(got_out, ro, "out")
    assert got_dn.all() and not got_st.any() and list(got_c) == [0, 0, 0, 0]


def test_flag_empty_is_noop(fc):
    import torch
    out, stale, done, cnt = _bufs(2, 512, 1)
    x = torch.zeros(512, dtype=torch.int16, device="cuda")
    f = torch.zeros(1, dtype=torch.int32, device="cuda")
    fc.fc_flag_unpack_reduce([x, x], [f, f], 0, 512, 1, out, stale, done, cnt)
    fc.fc_flag_pack(x, 512, 1, x, f, n=0)
    torch.cuda.synchronize()
    assert int(cnt.abs().sum()) == 0 and int(f[0]) == 0


# ---------------------------------------------------------------------------------------------------
# polling slot receiver, senders finished before the receiver starts
# ---------------------------------------------------------------------------------------------------
def _inject(slots_d, ep):
    import torch
    v = slots_d.view(torch.int32).view(-1, 2)
    v[:, 1] = torch.from_numpy(ep.view(np.int32)).to(slots_d.device)


def _set_epochs_host(slots, ep):
    s = slots.copy()
    s &= np.uint64(0xFFFFFFFF)
    s |= ep.astype(np.uint64) << np.uint64(32)
    return s


@pytest.mark.parametrize("polls", [0, 2])
@pytest.mark.parametrize("R", [1, 3, 8, 16])
@pytest.mark.parametrize("B", [32, 64, 128, 256])
def test_ll_poll_matches_oracle(fc, orc, B, R, polls):
    import torch
    from gpu_helpers import assert_equal_bits, up
    cfg = dg.SLOTS
    nblk = 8 * 9 + 3  # 75 blocks: the last tile is ragged for every block size
    n, e = 2 * B * nblk, 0 if R == 3 else 0x2A
    xs = [dg.synth_bf16((B, R, r, 1), n) for r in range(R)]
    cf = dataclasses.replace(cfg, block_slots=B)
    eps, masks = zip(*[dg.stale_epochs(cf, r, n // 2, epoch=e, p=0.12) for r in range(R)])
    done0 = (np.arange(nblk) % 7 == 3).astype(np.uint8)
    slots_d = []
    for r in range(R):
        s = torch.empty(n // 2, dtype=torch.int64, device="cuda")
        fc.fc_ll_pack(up(xs[r]), B, e, s)
        _inject(s, eps[r])
        slots_d.append(s)
    out, stale, done, cnt = _bufs(R, n, nblk, out_fill=77, done0=done0)
    fc.fc_ll_poll_unpack_reduce(slots_d, n, B, e, out, stale, done, cnt, max_polls=polls)
    got_out, got_st, got_dn, got_c = _down_all(out, stale, done, cnt, R, nblk)
    late = [_set_epochs_host(orc.ll_pack(xs[r], B, e), eps[r]) for r in range(R)]
    ro, rst, rdn, rc = orc.ll_unpack_reduce(late, n, B, e, out=np.full(n, 77, np.uint16), done=done0.copy())
    assert_equal_bits(got_out, ro, "out")
    assert_equal_bits(got_dn, rdn, "done")
    assert_equal_bits(got_c[:2], rc, "counters")
    skipped = done0.astype(bool)
    assert np.all(got_st[:, skipped] == 0xAB)
    assert_equal_bits(got_st[:, ~skipped], rst[:, ~skipped], "stale (examined)")
    want_polls = polls * _tiles_polled(np.stack(masks).astype(bool), done0, 256 // B)
    assert int(got_c[2]) == want_polls and int(got_c[3]) == 0


def test_ll_poll_equals_one_look_receiver(fc):
    """With no re-reads the polling receiver gives the one-look receiver's bits on the slot workload
    (8 ranks x [128, 8192], 2% late copies, shuffled write order), grid capped or not."""
    import torch
    from gpu_helpers import assert_equal_bits, counters_buf, down, up
    cfg = dg.SLOTS
    R, n, B, e = cfg.R, cfg.n, cfg.block_slots, cfg.epoch
    nslots, nblk = n // 2, n // 2 // B
    slots_d = []
    for r in range(R):
        s = torch.empty(nslots, dtype=torch.int64, device="cuda")
        fc.fc_ll_pack(up(dg.partial(cfg, r)), B, e, s, block_order=up(dg.write_order(cfg, r, nblk)))
        _inject(s, dg.stale_epochs(cfg, r, nslots)[0])
        slots_d.append(s)
    ref = _bufs(R, n, nblk)
    c2 = counters_buf()
    fc.fc_ll_unpack_reduce(slots_d, n, B, e, ref[0], ref[1], ref[2], c2)
    want = _down_all(ref[0], ref[1], ref[2], c2, R, nblk)
    for mw in (0, 37):
        got = _bufs(R, n, nblk)
        fc.fc_ll_poll_unpack_reduce(slots_d, n, B, e, *got, max_workgroups=mw)
        g = _down_all(*got, R, nblk)
        for a, b, what in zip(g[:3], want[:3], ("out", "stale", "done")):
            assert_equal_bits(a, b, f"{what} (max_workgroups={mw})")
        assert_equal_bits(g[3][:2], want[3][:2], "counters")
        assert int(g[3][1]) > 0


# ---------------------------------------------------------------------------------------------------
# live: the receiver spins on stream A while a paced sender writes on stream B
# ---------------------------------------------------------------------------------------------------
LIVE_POLLS = 200_000   # at ~1-2 us a re-read, a bound of well under a second per tile
LIVE_WGS = 32          # the receiver's grid and compute units; the sender has the other ones


@pytest.mark.parametrize("enc", ["flag", "ll"])
def test_live_sender_and_receiver(fc, orc, enc):
    import torch
    from gpu_helpers import assert_equal_bits, counters_buf, up
    cfg = dg.SLOTS
    R, n = cfg.R, cfg.n
    be, B = 2048, cfg.block_slots
    nblk = n // be if enc == "flag" else n // 2 // B
    from tensor_all_reduce_amd.streams import sender_receiver_streams
    # streams with disjoint compute-unit masks get hardware queues of their own: two plain streams may
    # share one queue, and then the sender would only start once the receiver's budget had run out
    sa, sb = sender_receiver_streams(receiver_cus=LIVE_WGS)
    e0 = 0x51
    # buffers hold an earlier epoch's data: every copy is stale until the sender rewrites it
    if enc == "flag":
        pays = [torch.zeros(n, dtype=torch.int16, device="cuda") for _ in range(R)]
        fls = [torch.full((nblk,), e0 - 1, dtype=torch.int32, device="cuda") for _ in range(R)]
    else:
        slots = [torch.zeros(n // 2, dtype=torch.int64, device="cuda") for _ in range(R)]
        fc.fc_ll_pack([up(dg.synth_bf16((0xDEAD, r), n)) for r in range(R)], B, e0 - 1, slots)
    torch.cuda.synchronize()
    for step in range(2):  # two epochs in a row on the same buffers
        e = e0 + step
        xs = [dg.synth_bf16((0x11FE, step, r), n) for r in range(R)]
        xd = [up(x) for x in xs]
        orders = [up(np.random.default_rng((step, r)).permutation(nblk).astype(np.int32)) for r in range(R)]
        out, stale, done, cnt = _bufs(R, n, nblk)
        torch.cuda.synchronize()
        print(f"live {enc} epoch {e:#x}: receiver on stream A, then the paced sender on stream B", flush=True)
        if enc == "flag":
            fc.fc_flag_unpack_reduce(pays, fls, n, be, e, out, stale, done, cnt, max_polls=LIVE_POLLS,
                                     max_workgroups=LIVE_WGS, stream=sa)
            time.sleep(0.002)  # the receiver is spinning before the sender starts
            fc.fc_flag_pack(xd, be, e, pays, fls, block_order=orders, pace=2, stream=sb)  # R peers at once
        else:
            fc.fc_ll_poll_unpack_reduce(slots, n, B, e, out, stale, done, cnt, max_polls=LIVE_POLLS,
                                        max_workgroups=LIVE_WGS, stream=sa)
            time.sleep(0.002)
            fc.fc_ll_pack(xd, B, e, slots, block_order=orders, pace=2, stream=sb)
        torch.cuda.synchronize()
        got = _down_all(out, stale, done, cnt, R, nblk)
        print(f"  pending after the live pass {int(got[3][1])}, re-reads {int(got[3][2])}", flush=True)
        # whatever the budget left pending is completed by a second, one-look pass
        c2 = counters_buf()
        if enc == "flag":
            fc.fc_flag_unpack_reduce(pays, fls, n, be, e, out, stale, done, c2)
            ro, _, _, _ = orc.flag_unpack_reduce(xs, [np.full(nblk, e, np.uint32)] * R, n, be, e)
        else:
            fc.fc_ll_poll_unpack_reduce(slots, n, B, e, out, stale, done, c2)
            ro, _, _, _ = orc.ll_unpack_reduce([orc.ll_pack(x, B, e) for x in xs], n, B, e)
        fin = _down_all(out, stale, done, c2, R, nblk)
        assert_equal_bits(fin[0], ro, "out == all on time")
        assert fin[2].all() and int(fin[3][1]) == 0
        # the receiver saw stale copies, waited, and completed every block while the sender was writing
        assert int(got[3][2]) > 0, "the receiver never had to wait: the sender ran first"
        assert int(got[3][1]) == 0, "blocks left pending: sender and receiver did not run concurrently"
        assert_equal_bits(got[0], ro, "out of the live pass")
    sa.close()
    sb.close()


@pytest.mark.parametrize("R,n", [(8, 8192), (8, 1 << 20), (3, 65536)])
def test_selector_driven_receiver(fc, orc, R, n):
    """SelfSyncReduce picks the encoding from the measured cost table, the senders write, the receiver
    folds: the result equals the oracle's fixed-order sum, whichever encoding was chosen."""
    import torch
    from gpu_helpers import assert_equal_bits, counts, down, up
    from tensor_all_reduce_amd.flash_allreduce import SelfSyncReduce
    xs = [dg.synth_bf16((0x5E1, R, n, r), n) for r in range(R)]
    ss = SelfSyncReduce(R, n)
    print(f"R={R} n={n}: encoding {ss.encoding}", flush=True)
    for e in (3, 4):
        ss.begin()
        ss.send([up(x) for x in xs], e)
        ss.receive(e)
        torch.cuda.synchronize()
        c = counts(ss.counters, 4)
        assert down(ss.done, np.uint8).all() and list(c) == [0, 0, 0, 0]
        if ss.encoding == "ll":
            ro, _, _, _ = orc.ll_unpack_reduce([orc.ll_pack(x, ss.B, e) for x in xs], n, ss.B, e)
        else:
            ro, _, _, _ = orc.flag_unpack_reduce(xs, [np.full(ss.nblk, e, np.uint32)] * R, n, ss.B, e)
        assert_equal_bits(down(ss.out, np.uint16), ro, f"out ({ss.encoding})")
