"""Seeded random shapes through the self-synchronizing receivers (flash-comm, abstract: readiness evidence
per block, validated by the receiver with no barrier) and the unquantized reduce + RMSNorm (TokenWeave,
abstract), against the oracle:

  * slot sender (R peers in one launch, shuffled write order) + slot receiver, counted and uncounted:
    1-16 ranks, every block size, block counts that fill the receiver's tiles and ragged ones, epochs at
    the wrap, late copies of every kind (whole blocks and torn single slots) from none to all, blocks
    already done; then the late blocks are published and a second pass must complete every block with
    the bits of an on-time pass;
  * the standalone all-gather on the same kind of slots, both passes;
  * the flag receiver: block sizes 512-65536, wrong flag words, a poll budget, capped grids;
  * the bf16 reduce + RMSNorm: 1-16 ranks, rows of 8 to 32768 elements, capped grids, with and without
    a residual.

Outputs, stale flags, done flags and counters bit-exact; normalized bf16 outputs within 2 ulp."""
import numpy as np
import pytest

from tensor_all_reduce_amd import datagen as dg

pytestmark = pytest.mark.gpu
M32 = 0xFFFFFFFF
EPOCHS = [0, 1, 0x2A, 0x7FFFFFFF, 0x80000000, M32, None]   # None: a random epoch


@pytest.fixture(scope="module")
def fc():
    from tensor_all_reduce_amd import _lib
    return _lib


def _bf16(rng, n, scale=1.0):
    v = (scale * rng.standard_normal(n)).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def _wrong(rng, e):
    """A wrong epoch word of one of several kinds (never e itself)."""
    k = int(rng.integers(7))
    w = [(e - 1) & M32, 0, (e + 1) & M32, ~e & M32, e ^ 0x80000000, int(rng.integers(1 << 32)), (e + 2) & M32][k]
    return w if w != e else e ^ 1


def _late_epochs(rng, nslots, B, e, frac):
    """Per-slot epoch words as the receiver sees one rank's blocks: about frac of the blocks late, half of
    those whole (one wrong word for every slot), half torn (one slot of the block wrong)."""
    ep = np.full(nslots, e, np.uint32)
    nblk = nslots // B
    for b in np.nonzero(rng.random(nblk) < frac)[0]:
        if rng.random() < 0.5:
            ep[b * B:(b + 1) * B] = _wrong(rng, e)
        else:
            ep[b * B + int(rng.integers(B))] = _wrong(rng, e)
    return ep


def _with_epochs(slots, ep):
    return (np.asarray(slots, np.uint64) & np.uint64(M32)) | (ep.astype(np.uint64) << np.uint64(32))


def _epoch(rng):
    e = EPOCHS[int(rng.integers(len(EPOCHS)))]
    return int(rng.integers(1 << 32)) if e is None else e


def _set_epochs_gpu(slots_d, ep):
    import torch
    slots_d.view(torch.int32).view(-1, 2)[:, 1] = torch.from_numpy(ep.view(np.int32)).to(slots_d.device)


def _nblk(rng, tile_blocks):
    """A block count: a few blocks, whole receiver tiles, or whole tiles plus a ragged tail."""
    k = int(rng.integers(3))
    if k == 0:
        return int(rng.integers(1, 2 * tile_blocks + 1))
    whole = tile_blocks * int(rng.integers(1, 9))
    return whole if k == 1 else whole + int(rng.integers(1, tile_blocks))


def _slot_cases(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        R = int(rng.integers(1, 17))
        B = int(rng.choice([32, 64, 128, 256]))
        tile = 4096 // B if B == 256 else 2048 // B   # slots per receiver workgroup / block size
        out.append((R, B, _nblk(rng, tile), _epoch(rng),
                    float(rng.choice([0.0, 0.02, 0.3, 1.0])), bool(rng.random() < 0.6), int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("R,B,nblk,e,frac,counted,seed", _slot_cases(40, 0x51075), ids=lambda v: str(v))
def test_slot_receiver_random(fc, orc, R, B, nblk, e, frac, counted, seed):
    import torch
    from gpu_helpers import assert_equal_bits, counters_buf, counts, down, up
    rng = np.random.default_rng(seed)
    nslots = B * nblk
    n = 2 * nslots
    xs = [_bf16(rng, n, 10.0 ** rng.uniform(-1, 1)) for _ in range(R)]
    orders = [rng.permutation(nblk).astype(np.int32) for _ in range(R)]
    eps = [_late_epochs(rng, nslots, B, e, frac) for _ in range(R)]
    slots_d = [torch.empty(nslots, dtype=torch.int64, device="cuda") for _ in range(R)]
    fc.fc_ll_pack([up(x) for x in xs], B, e, slots_d, block_order=[up(o) for o in orders])
    for s, ep in zip(slots_d, eps):
        _set_epochs_gpu(s, ep)
    good = [orc.ll_pack(x, B, e, order=o) for x, o in zip(xs, orders)]
    late = [_with_epochs(g, ep) for g, ep in zip(good, eps)]
    done0 = (rng.random(nblk) < 0.2).astype(np.uint8)
    fill = np.uint16(rng.integers(1 << 16))
    out = torch.full((n,), int(fill.astype(np.int16)), dtype=torch.int16, device="cuda")
    stale = torch.full((R * nblk,), 0xAB, dtype=torch.uint8, device="cuda")
    done = up(done0.copy())
    cnt = counters_buf()
    where = f"R={R} B={B} nblk={nblk} e={e:#x} late={frac} counted={counted}"

    fc.fc_ll_unpack_reduce(slots_d, n, B, e, out, stale, done, cnt if counted else None)
    torch.cuda.synchronize()
    r_out, r_done, r_cnt = np.full(n, fill, np.uint16), done0.copy(), np.zeros(2, np.uint32)
    ro, rst, rdn, rc = orc.ll_unpack_reduce(late, n, B, e, out=r_out, done=r_done, counters=r_cnt)
    st = down(stale, np.uint8).reshape(R, nblk)
    skipped = done0.astype(bool)
    assert np.all(st[:, skipped] == 0xAB), "blocks already done are not examined: " + where
    assert_equal_bits(st[:, ~skipped], np.asarray(rst).reshape(R, nblk)[:, ~skipped], "stale " + where)
    assert_equal_bits(down(done, np.uint8), rdn, "done " + where)
    assert_equal_bits(down(out, np.uint16), ro, "out " + where)
    assert_equal_bits(counts(cnt), rc if counted else np.zeros(2, np.uint32), "counters " + where)

    # the late blocks are published; the second pass completes them with the bits of an on-time pass
    fc.fc_ll_pack([up(x) for x in xs], B, e, slots_d)
    cnt.zero_()
    fc.fc_ll_unpack_reduce(slots_d, n, B, e, out, stale, done, cnt if counted else None)
    torch.cuda.synchronize()
    ro2, _, rdn2, rc2 = orc.ll_unpack_reduce(good, n, B, e, out=ro, done=rdn, counters=np.zeros(2, np.uint32))
    assert np.all(rdn2 == 1)
    assert_equal_bits(down(done, np.uint8), rdn2, "done, second pass " + where)
    assert_equal_bits(down(out, np.uint16), ro2, "out, second pass " + where)
    assert_equal_bits(counts(cnt), rc2 if counted else np.zeros(2, np.uint32), "counters, second pass " + where)
    # every block not done before the first pass now holds the on-time reduction
    full, _, _, _ = orc.ll_unpack_reduce(good, n, B, e)
    fresh = np.repeat(~skipped, 2 * B)
    assert_equal_bits(down(out, np.uint16)[fresh], full[fresh], "out vs on-time pass " + where)


def _gather_cases(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        R = int(rng.integers(1, 17))
        B = int(rng.choice([32, 64, 128, 256]))
        out.append((R, B, _nblk(rng, 2048 // B), _epoch(rng),
                    float(rng.choice([0.0, 0.05, 0.5])), bool(rng.random() < 0.5), int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("R,B,nblk,e,frac,counted,seed", _gather_cases(24, 0x6A7), ids=lambda v: str(v))
def test_all_gather_random(fc, orc, R, B, nblk, e, frac, counted, seed):
    import torch
    from gpu_helpers import assert_equal_bits, counters_buf, counts, down, up
    rng = np.random.default_rng(seed)
    nw = B * nblk
    words = [rng.integers(0, 1 << 32, nw, dtype=np.uint64) for _ in range(R)]
    eps = [_late_epochs(rng, nw, B, e, frac) for _ in range(R)]
    late = [_with_epochs(w, ep) for w, ep in zip(words, eps)]
    good = [_with_epochs(w, np.full(nw, e, np.uint32)) for w in words]
    done0 = (rng.random(R * nblk) < 0.15).astype(np.uint8)
    slots_d = [up(s) for s in late]
    outs = [torch.full((nw,), 0x5A5A5A5A, dtype=torch.int32, device="cuda") for _ in range(R)]
    stale = torch.full((R * nblk,), 0xAB, dtype=torch.uint8, device="cuda")
    done = up(done0.copy())
    cnt = counters_buf()
    where = f"R={R} B={B} nblk={nblk} e={e:#x} late={frac} counted={counted}"
    r_out = [np.full(nw, 0x5A5A5A5A, np.uint32) for _ in range(R)]
    for p, slots_h in enumerate((late, good)):
        if p:
            for s, g in zip(slots_d, good):
                s.copy_(up(g))
            cnt.zero_()
        fc.fc_ll_gather(slots_d, nw, B, e, outs, stale, done, cnt if counted else None)
        torch.cuda.synchronize()
        r_out, rst, r_dn, rc = orc.ll_gather(slots_h, nw, B, e, out=r_out, done=(done0 if p == 0 else r_dn).copy(),
                                             counters=np.zeros(2, np.uint32))
        tag = f" pass {p + 1} " + where
        for r in range(R):
            assert_equal_bits(down(outs[r], np.uint32), r_out[r], f"out[{r}]" + tag)
        assert_equal_bits(down(done, np.uint8), r_dn, "done" + tag)
        assert_equal_bits(counts(cnt), rc if counted else np.zeros(2, np.uint32), "counters" + tag)
        if p == 0:
            st = down(stale, np.uint8)
            ex = done0 == 0
            assert np.all(st[~ex] == 0xAB), "copies already done are not examined: " + where
            assert_equal_bits(st[ex], np.asarray(rst).ravel()[ex], "stale" + tag)
    assert np.all(r_dn == 1)
    for r in range(R):
        fresh = np.repeat(done0.reshape(R, nblk)[r] == 0, B)
        assert_equal_bits(down(outs[r], np.uint32)[fresh], words[r].astype(np.uint32)[fresh], f"out[{r}] payload " + where)


def _flag_cases(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        R = int(rng.integers(1, 17))
        be = int(2 ** rng.integers(9, 17))
        nblk = int(rng.integers(1, max(2, (1 << 21) // be // R)))
        out.append((R, be, nblk, _epoch(rng), int(rng.choice([0, 0, 2])),
                    int(rng.choice([0, 0, 1, 3, 11])), int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("R,be,nblk,e,polls,mw,seed", _flag_cases(24, 0xF1A6), ids=lambda v: str(v))
def test_flag_receiver_random(fc, orc, R, be, nblk, e, polls, mw, seed):
    import torch
    from gpu_helpers import assert_equal_bits, counters_buf, counts, down, up
    rng = np.random.default_rng(seed)
    n = be * nblk
    xs = [_bf16(rng, n) for _ in range(R)]
    frac = float(rng.choice([0.0, 0.1, 0.6]))
    fls = []
    for _ in range(R):
        f = np.full(nblk, e, np.uint32)
        for b in np.nonzero(rng.random(nblk) < frac)[0]:
            f[b] = _wrong(rng, e)
        fls.append(f)
    done0 = (rng.random(nblk) < 0.2).astype(np.uint8)
    out = torch.full((n,), 77, dtype=torch.int16, device="cuda")
    stale = torch.full((R * nblk,), 0xAB, dtype=torch.uint8, device="cuda")
    done = up(done0.copy())
    cnt = counters_buf()
    where = f"R={R} be={be} nblk={nblk} e={e:#x} polls={polls} max_workgroups={mw}"
    fc.fc_flag_unpack_reduce([up(x) for x in xs], [up(f) for f in fls], n, be, e, out, stale, done, cnt,
                             max_polls=polls, max_workgroups=mw)
    torch.cuda.synchronize()
    ro, rst, rdn, rc = orc.flag_unpack_reduce(xs, fls, n, be, e, out=np.full(n, 77, np.uint16), done=done0.copy())
    st = down(stale, np.uint8).reshape(R, nblk)
    skipped = done0.astype(bool)
    assert np.all(st[:, skipped] == 0xAB), "blocks already done are not examined: " + where
    assert_equal_bits(st[:, ~skipped], np.asarray(rst).reshape(R, nblk)[:, ~skipped], "stale " + where)
    assert_equal_bits(down(done, np.uint8), rdn, "done " + where)
    assert_equal_bits(down(out, np.uint16), ro, "out " + where)
    c = counts(cnt, 4)
    assert_equal_bits(c[:2], rc, "counters " + where)
    if polls == 0:
        assert c[2] == 0 and c[3] == 0, where


def _rms_cases(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        R = int(rng.integers(1, 17))
        H = 8 * int(rng.integers(1, 129)) if rng.random() < 0.5 else 8 * int(rng.integers(129, 4097))
        rows = int(rng.integers(1, max(2, min(300, (1 << 21) // H))))
        out.append((R, rows, H, int(rng.choice([0, 0, 1, 5, 64])), bool(rng.random() < 0.8),
                    int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("R,rows,H,mw,with_res,seed", _rms_cases(32, 0x7E4), ids=lambda v: str(v))
def test_reduce_rmsnorm_random(fc, orc, R, rows, H, mw, with_res, seed):
    import torch
    from gpu_helpers import assert_bf16_close, assert_equal_bits, down, up
    rng = np.random.default_rng(seed)
    n = rows * H
    parts = [_bf16(rng, n, 10.0 ** rng.uniform(-1, 1)) for _ in range(R)]
    res = _bf16(rng, n) if with_res else None
    gam = (((1.0 + 0.1 * rng.standard_normal(H)).astype(np.float32)).view(np.uint32) >> 16).astype(np.uint16)
    eps = float(rng.choice([1e-5, 1e-6]))
    o, ro, _ = orc.reduce_rmsnorm(parts, rows, H, res, gam, eps)
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    rout = torch.empty(n, dtype=torch.int16, device="cuda") if with_res else None
    fc.fc_reduce_rmsnorm([up(p) for p in parts], rows,
                         dict(residual=up(res) if with_res else None, gamma=up(gam), eps=eps, hidden=H, out=out,
                              residual_out=rout), max_workgroups=mw)
    torch.cuda.synchronize()
    where = f"R={R} rows={rows} H={H} max_workgroups={mw} residual={with_res}"
    if with_res:
        assert_equal_bits(down(rout, np.uint16), ro, "residual_out " + where)
    assert_bf16_close(down(out, np.uint16), o, 2, "out " + where)
