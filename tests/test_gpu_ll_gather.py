"""GPU parity of the standalone all-gather on epoch-tagged blocks (fc_ll_gather) against the oracle:
payload words, stale flags, done flags and counters bit-exact, on time, with every kind of late block,
after the retry, and with blocks already done.  Then the quantized all-gather of the decode workload
carried in slots: the shards' messages validated, copied and dequantized with the residual-add +
RMSNorm epilogue, against the oracle's two-step all-reduce."""
import numpy as np
import pytest

from tensor_all_reduce_amd import datagen as dg

pytestmark = pytest.mark.gpu
E = 0x2A


@pytest.fixture(scope="module")
def fc():
    from tensor_all_reduce_amd import _lib
    return _lib


def _slots(words, epochs):
    return (np.asarray(words, np.uint64) & np.uint64(0xFFFFFFFF)) | (np.asarray(epochs, np.uint64) << np.uint64(32))


def _gpu_gather(fc, slots_h, nwords, B, out=None, done=None, counted=True):
    """counted=False passes NULL counters; the returned counters are then zeros."""
    import torch
    from gpu_helpers import counters_buf, down, up
    R = len(slots_h)
    nblk = nwords // B
    sl = [up(s) for s in slots_h]
    out = [torch.zeros(nwords, dtype=torch.int32, device="cuda") for _ in range(R)] if out is None else out
    done = torch.zeros(R * nblk, dtype=torch.uint8, device="cuda") if done is None else done
    stale = torch.full((R * nblk,), 7, dtype=torch.uint8, device="cuda")
    cnt = counters_buf()
    fc.fc_ll_gather(sl, nwords, B, E, out, stale, done, cnt if counted else None)
    torch.cuda.synchronize()
    return out, stale, done, cnt


def _late(R, nblk, B, nwords, seed, frac=0.1):
    """Per-rank slot epochs with about frac of the (rank, block) copies late, of every kind."""
    rng = np.random.default_rng(seed)
    kinds = [lambda e: e - 1, lambda e: 0, lambda e: e + 1, lambda e: ~e & 0xFFFFFFFF, lambda e: e ^ 0x80000000,
             lambda e: 0x9E3779B9, None]
    ep = [np.full(nwords, E, np.uint64) for _ in range(R)]
    for r in range(R):
        for b in range(nblk):
            if rng.random() < frac:
                k = kinds[int(rng.integers(len(kinds)))]
                if k is None:  # torn: one late slot
                    ep[r][b * B + int(rng.integers(B))] = E - 1
                else:
                    ep[r][b * B:(b + 1) * B] = k(E)
    return ep


@pytest.mark.parametrize("counted", [True, False])
@pytest.mark.parametrize("B", [32, 64, 128, 256])
@pytest.mark.parametrize("R,nblk", [(1, 7), (3, 33), (8, 64), (16, 5), (2, 3000)])
def test_ll_gather_parity_and_retry(fc, orc, B, R, nblk, counted):
    """Both tile shapes of the launcher (counted: 16 wavefronts of 4 instructions; uncounted: 8 of 2), every
    block size, ragged tile counts."""
    from gpu_helpers import assert_equal_bits, counts, down
    nwords = B * nblk
    rng = np.random.default_rng(B * 100 + R)
    ws = [rng.integers(0, 1 << 32, nwords, dtype=np.uint64).astype(np.uint32) for _ in range(R)]
    ep = _late(R, nblk, B, nwords, B + R)
    slots = [_slots(ws[r], ep[r]) for r in range(R)]
    ro, rs, rd, rc = orc.ll_gather(slots, nwords, B, E)
    out, stale, done, cnt = _gpu_gather(fc, slots, nwords, B, counted=counted)
    where = f"B={B} R={R} nblk={nblk} counted={counted}"
    for r in range(R):
        assert_equal_bits(down(out[r], np.uint32), ro[r], f"out rank {r} " + where)
    assert_equal_bits(down(stale, np.uint8), rs, "stale " + where)
    assert_equal_bits(down(done, np.uint8), rd, "done " + where)
    if counted:
        assert_equal_bits(counts(cnt), rc, "counters " + where)
    # the late blocks arrive: the retry completes them
    slots2 = [_slots(ws[r], np.full(nwords, E)) for r in range(R)]
    ro2, rs2, rd2, rc2 = orc.ll_gather(slots2, nwords, B, E, out=ro, done=rd)
    out2, stale2, done2, cnt2 = _gpu_gather(fc, slots2, nwords, B, out=out, done=done, counted=counted)
    for r in range(R):
        assert_equal_bits(down(out2[r], np.uint32), ws[r], f"retry out rank {r} " + where)
    assert_equal_bits(down(done2, np.uint8), rd2, "retry done " + where)
    if counted:
        assert_equal_bits(counts(cnt2), rc2, "retry counters " + where)
    # stale flags are written for the blocks examined in this pass only
    examined = rd == 0
    assert_equal_bits(down(stale2, np.uint8)[examined], rs2[examined], "retry stale " + where)


def test_ll_gather_done_blocks_untouched(fc, orc):
    import torch
    from gpu_helpers import assert_equal_bits, counts, down, up
    R, B, nblk = 2, 64, 9
    nwords = B * nblk
    ws = [np.arange(nwords, dtype=np.uint32) + 1000 * r for r in range(R)]
    done_h = np.zeros(R * nblk, np.uint8)
    done_h[[0, 4, 10]] = 1
    slots = [_slots(w, np.full(nwords, E)) for w in ws]
    ro, rs, rd, rc = orc.ll_gather(slots, nwords, B, E, done=done_h)
    out, stale, done, cnt = _gpu_gather(fc, slots, nwords, B, done=up(done_h))
    for r in range(R):
        assert_equal_bits(down(out[r], np.uint32), ro[r], f"rank {r}")
    assert_equal_bits(down(done, np.uint8), rd, "done")
    assert_equal_bits(counts(cnt), rc, "counters")


def test_quantized_all_gather_in_slots_end_to_end(fc, orc):
    """Decode workload: every shard's requantized message (codes then meta, one buffer) is carried in epoch
    slots with ~10% late blocks; the receiver validates and copies (pass 1 + retry), then dequantizes the
    gathered messages with the residual-add + RMSNorm epilogue."""
    import torch
    from gpu_helpers import assert_bf16_close, assert_equal_bits, counts, down, up
    cfg = dg.DECODE_8B
    R, L, G, b2 = cfg.R, cfg.L, cfg.group, cfg.bits_ag
    parts = dg.partials(cfg)
    res, gam = dg.residual(cfg), dg.gamma(cfg)
    ref = orc.two_step(parts, cfg.bits_rs, b2, G, residual=res, gamma=gam, eps=cfg.eps, hidden=cfg.H, plain=False)
    cb, mb = L * b2 // 8, L // G
    B = 64
    msg_words = (cb + 4 * mb) // 4
    nwords = -(-msg_words // B) * B
    words = []
    for s in range(R):
        m = np.zeros(nwords, np.uint32)
        m[:msg_words] = np.concatenate([ref["codes2"][s * cb:(s + 1) * cb].view(np.uint8),
                                        ref["meta2"][s * mb:(s + 1) * mb].view(np.uint8)]).view(np.uint32)
        words.append(m)
    ep = _late(R, nwords // B, B, nwords, 17)
    out, stale, done, cnt = _gpu_gather(fc, [_slots(words[s], ep[s]) for s in range(R)], nwords, B)
    assert int(counts(cnt, 4)[1]) > 0
    out, stale, done, cnt = _gpu_gather(fc, [_slots(w, np.full(nwords, E)) for w in words], nwords, B, out=out,
                                        done=done)
    assert down(done, np.uint8).all()
    shards = [(out[s].view(torch.uint8)[:cb], out[s].view(torch.uint8)[cb:cb + 4 * mb].view(torch.int32))
              for s in range(R)]
    o = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    rout = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    fc.fc_gather_dequant(shards, L, b2, G, norm=dict(residual=up(res), gamma=up(gam), eps=cfg.eps, hidden=cfg.H,
                                                    out=o, residual_out=rout))
    assert_bf16_close(down(rout, np.uint16), ref["residual_out"], 0, "residual_out")
    assert_bf16_close(down(o, np.uint16), ref["out"], 2, "out")


@pytest.mark.parametrize("counted", [True, False])
def test_all_gather_prefill_messages_as_benched(fc, orc, counted):
    """The benchmark's f3 workload: the 8 int8 shard messages of the 70B prefill (codes then meta, 1,081,344
    words each) carried in 64-slot blocks with about 2% of the copies late (every kind), pass 1 then the
    retry with every block rewritten: out, stale, done and counters of both passes equal the oracle's."""
    from gpu_helpers import assert_equal_bits, counts, down
    cfg = dg.PREFILL_70B
    R, B = cfg.R, 64
    nwords = (cfg.L * cfg.bits_ag // 8 + 4 * (cfg.L // cfg.group)) // 4
    assert nwords % B == 0
    nblk = nwords // B
    rng = np.random.default_rng(0xF3)
    words = [rng.integers(0, 1 << 32, nwords, dtype=np.uint64).astype(np.uint32) for _ in range(R)]
    ep = _late(R, nblk, B, nwords, 23, frac=0.02)
    first = [_slots(words[r], ep[r]) for r in range(R)]
    print(f"f3 prefill messages: R={R} nwords={nwords} B={B}", flush=True)
    out, stale, done, cnt = _gpu_gather(fc, first, nwords, B, counted=counted)
    ro, rst, rdn, rc = orc.ll_gather(first, nwords, B, E)
    for r in range(R):
        assert_equal_bits(down(out[r], np.uint32), ro[r], f"pass 1 words of rank {r}")
    assert_equal_bits(down(stale, np.uint8), rst, "pass 1 stale")
    assert_equal_bits(down(done, np.uint8), rdn, "pass 1 done")
    if counted:
        assert_equal_bits(counts(cnt), rc, "pass 1 counters")
    assert int(rc[1]) > 0
    again = [_slots(words[r], np.full(nwords, E)) for r in range(R)]
    out, stale, done, cnt = _gpu_gather(fc, again, nwords, B, out=out, done=done, counted=counted)
    ro2, rst2, rdn2, rc2 = orc.ll_gather(again, nwords, B, E, out=ro, done=rdn)
    for r in range(R):
        assert_equal_bits(down(out[r], np.uint32), ro2[r], f"retry words of rank {r}")
    assert_equal_bits(down(done, np.uint8), rdn2, "retry done")
    assert rdn2.all() and int(rc2[1]) == 0
    if counted:
        assert_equal_bits(counts(cnt), rc2, "retry counters")
