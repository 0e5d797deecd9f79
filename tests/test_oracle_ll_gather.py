"""Pins of the oracle's standalone all-gather on epoch-tagged blocks (flash-comm, abstract: every block
carries evidence of its readiness, validated by the receiver).  Slots are built here with numpy
(word | epoch << 32), independently of the oracle's packer."""
import numpy as np
import pytest

from tensor_all_reduce_amd import datagen as dg

E = 0x2A


def _slots(words, epochs):
    return (np.asarray(words, np.uint64) & np.uint64(0xFFFFFFFF)) | (np.asarray(epochs, np.uint64) << np.uint64(32))


def _words(R, nwords, seed):
    rng = np.random.default_rng(seed)
    return [rng.integers(0, 1 << 32, nwords, dtype=np.uint64).astype(np.uint32) for _ in range(R)]


@pytest.mark.parametrize("B", [32, 64, 128, 256])
def test_all_valid_copies_every_word(orc, B):
    R, nwords = 3, 4 * 256
    ws = _words(R, nwords, B)
    out, stale, done, cnt = orc.ll_gather([_slots(w, np.full(nwords, E)) for w in ws], nwords, B, E)
    for r in range(R):
        assert np.array_equal(out[r], ws[r])
    assert not stale.any() and done.all() and list(cnt) == [0, 0]


WRONG = {"prev": lambda e: e - 1, "zero": lambda e: 0, "next": lambda e: e + 1, "not": lambda e: ~e & 0xFFFFFFFF,
         "msb": lambda e: e ^ 0x80000000, "random": lambda e: 0x9E3779B9}


@pytest.mark.parametrize("kind", sorted(WRONG) + ["torn", "whole_rank"])
def test_stale_blocks_flagged_untouched_and_completed_by_retry(orc, kind):
    R, B, nblk = 4, 64, 16
    nwords = B * nblk
    ws = _words(R, nwords, 7)
    ep = [np.full(nwords, E, np.uint64) for _ in range(R)]
    late = set()
    rng = np.random.default_rng(3)
    if kind == "whole_rank":
        ep[2][:] = E - 1
        late = {(2, b) for b in range(nblk)}
    else:
        for r, b in {(int(rng.integers(R)), int(rng.integers(nblk))) for _ in range(6)}:
            late.add((r, b))
            if kind == "torn":  # one late slot in an otherwise written block
                ep[r][b * B + int(rng.integers(B))] = E - 1
            else:
                ep[r][b * B:(b + 1) * B] = WRONG[kind](E)
    out, stale, done, cnt = orc.ll_gather([_slots(ws[r], ep[r]) for r in range(R)], nwords, B, E)
    for r in range(R):
        for b in range(nblk):
            f = r * nblk + b
            assert stale[f] == ((r, b) in late) and done[f] == ((r, b) not in late)
            blk = out[r][b * B:(b + 1) * B]
            assert np.array_equal(blk, np.zeros(B, np.uint32) if (r, b) in late else ws[r][b * B:(b + 1) * B])
    assert list(cnt) == [len(late), len(late)]
    # the late blocks arrive: the retry completes them and examines nothing else
    out2, stale2, done2, cnt2 = orc.ll_gather([_slots(ws[r], np.full(nwords, E)) for r in range(R)], nwords, B, E,
                                              out=out, done=done)
    for r in range(R):
        assert np.array_equal(out2[r], ws[r])
    assert done2.all() and list(cnt2) == [0, 0]


@pytest.mark.parametrize("pos", [0, 63])
def test_torn_block_at_either_end(orc, pos):
    """A block with a single late slot, first or last, is stale."""
    B, nwords = 64, 256
    ws = _words(1, nwords, 5)
    ep = np.full(nwords, E, np.uint64)
    ep[B + pos] = E + 1
    out, stale, done, cnt = orc.ll_gather([_slots(ws[0], ep)], nwords, B, E)
    assert list(stale) == [0, 1, 0, 0] and list(cnt) == [1, 1]
    assert not out[0][B:2 * B].any()


def test_done_blocks_are_not_rewritten(orc):
    R, B, nwords = 2, 32, 128
    ws = _words(R, nwords, 11)
    done = np.zeros(R * (nwords // B), np.uint8)
    done[[0, 5]] = 1
    out, stale, done2, cnt = orc.ll_gather([_slots(w, np.full(nwords, E)) for w in ws], nwords, B, E, done=done)
    assert not out[0][:B].any() and not out[1][B:2 * B].any()
    assert np.array_equal(out[0][B:], ws[0][B:])


def test_quantized_message_survives_the_trip(orc):
    """A shard's quantized message (codes, then meta, one contiguous buffer) carried as slot words comes out
    byte for byte, and dequantizes to the same values as the message sent."""
    L, G, bits = 4096, 128, 8
    x = dg.synth_bf16((1, 2, 3), L, sigma=1.0, outlier_p=0.01, outlier_factor=20.0)
    codes, meta = orc.quantize(x, bits, G)
    msg = np.concatenate([codes.view(np.uint8), meta.view(np.uint8)]).view(np.uint32)
    B = 32
    nw = -(-msg.size // B) * B
    words = np.zeros(nw, np.uint32)
    words[:msg.size] = msg
    out, _, done, _ = orc.ll_gather([_slots(words, np.full(nw, E))], nw, B, E)
    got = out[0][:msg.size].view(np.uint8)
    c2, m2 = got[:codes.size], got[codes.size:].view(np.uint32)
    assert np.array_equal(c2, codes) and np.array_equal(m2, meta)
    assert np.array_equal(orc.dequant(c2, m2, L, bits, G), orc.dequant(codes, meta, L, bits, G))
