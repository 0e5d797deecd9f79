"""Pins of the oracle's receiver for readiness by one flag word per block.  Expected values are built here
with numpy (an fp32 left fold of small integers is exact, so the reduced block is the integer sum)."""
import numpy as np
import pytest

E = 0x2A


def _bf16(v):
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _inputs(R, n, seed):
    rng = np.random.default_rng(seed)
    vals = [rng.integers(-32, 33, n).astype(np.float32) for _ in range(R)]   # sums stay exact in bf16
    return vals, [_bf16(v) for v in vals]


@pytest.mark.parametrize("R,E_blk", [(1, 2048), (3, 2048), (8, 8192)])
def test_all_valid_reduces_every_block(orc, R, E_blk):
    n = 4 * E_blk
    vals, pay = _inputs(R, n, R)
    flags = [np.full(n // E_blk, E, np.uint32) for _ in range(R)]
    out, stale, done, cnt = orc.flag_unpack_reduce(pay, flags, n, E_blk, E)
    assert np.array_equal(out, _bf16(np.sum(vals, axis=0)))
    assert not stale.any() and done.all() and list(cnt) == [0, 0]


@pytest.mark.parametrize("bad", [E - 1, 0, E + 1, ~E & 0xFFFFFFFF, E ^ 0x80000000, 0x9E3779B9])
def test_wrong_flag_is_stale_and_its_payload_is_never_read(orc, bad):
    R, Eb, nblk = 4, 2048, 6
    n = Eb * nblk
    vals, pay = _inputs(R, n, 9)
    flags = [np.full(nblk, E, np.uint32) for _ in range(R)]
    flags[2][3] = bad
    pay[2][3 * Eb:4 * Eb] = 0x7FC0            # garbage where the flag says "not ready": a NaN if it were read
    out, stale, done, cnt = orc.flag_unpack_reduce(pay, flags, n, Eb, E)
    assert stale.reshape(R, nblk)[2, 3] == 1 and stale.sum() == 1
    assert done[3] == 0 and done.sum() == nblk - 1 and list(cnt) == [1, 1]
    assert not out[3 * Eb:4 * Eb].any()
    keep = np.ones(n, bool)
    keep[3 * Eb:4 * Eb] = False
    assert np.array_equal(out[keep], _bf16(np.sum(vals, axis=0))[keep])
    # the block arrives: the retry completes it with the on-time bits
    pay[2][3 * Eb:4 * Eb] = _bf16(vals[2][3 * Eb:4 * Eb])
    flags[2][3] = E
    out2, _, done2, cnt2 = orc.flag_unpack_reduce(pay, flags, n, Eb, E, out=out, done=done)
    assert np.array_equal(out2, _bf16(np.sum(vals, axis=0))) and done2.all() and list(cnt2) == [0, 0]


def test_done_blocks_skipped(orc):
    R, Eb, nblk = 2, 2048, 3
    n = Eb * nblk
    vals, pay = _inputs(R, n, 4)
    flags = [np.full(nblk, E, np.uint32) for _ in range(R)]
    done = np.array([0, 1, 0], np.uint8)
    out, stale, done2, cnt = orc.flag_unpack_reduce(pay, flags, n, Eb, E, done=done)
    assert not out[Eb:2 * Eb].any() and done2.all()


def test_order_of_ranks_matters_and_is_ascending(orc):
    """2^15, -2^15, 2^-10 in ranks 0, 1, 2: the ascending left fold keeps the small term (a fold starting
    elsewhere loses it to rounding)."""
    n, Eb = 2048, 2048
    pay = [_bf16(np.full(n, v, np.float32)) for v in (32768.0, -32768.0, 2.0 ** -10)]
    flags = [np.array([E], np.uint32)] * 3
    out, _, _, _ = orc.flag_unpack_reduce(pay, flags, n, Eb, E)
    assert np.all(out == _bf16(np.float32(2.0 ** -10)))
