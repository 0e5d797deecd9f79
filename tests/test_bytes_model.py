"""CPU pins of the algorithmic byte model (host logic behind every GB/s and roofline figure) against totals
worked out by hand from the workload shapes: each input read once and each output written once at its
stored width (bf16 2 B, codes bits/8, one 4-byte meta word per group, 8-byte slots, gamma once)."""
from tensor_all_reduce_amd import bytes_model as bm
from tensor_all_reduce_amd import datagen as dg


def _whole(cfg):
    return bm.two_step_whole(cfg.R, cfg.T, cfg.H, cfg.bits_rs, cfg.bits_ag, cfg.group)


def test_decode_step_by_call():
    c = _whole(dg.DECODE_8B)  # 8 x [64, 4096], int8, G = 128
    assert c["quantize"] == dict(read=4_194_304, write=2_162_688)   # 8 x 262144 bf16 in; codes + 16384 metas out
    assert c["reduce_shard"] == dict(read=2_162_688, write=270_336)  # 8 shards x 8 chunks of 32768 codes + metas
    assert c["gather_norm"] == dict(read=802_816, write=1_048_576)   # codes 262144 + meta 8192 + residual + gamma
    assert sum(bm.total(v) for v in c.values()) == 10_641_408


def test_tiny_and_prefill_totals():
    assert sum(bm.total(v) for v in _whole(dg.TINY).values()) == 17_664
    c3 = _whole(dg.PREFILL_70B)  # int4 reduce-scatter, int8 all-gather
    assert c3["quantize"] == dict(read=536_870_912, write=142_606_336)
    assert c3["reduce_shard"] == dict(read=142_606_336, write=34_603_008)
    assert c3["gather_norm"] == dict(read=101_728_256, write=134_217_728)
    assert sum(bm.total(v) for v in c3.values()) == 1_092_632_576


def test_one_gpu_share():
    c2, c3 = dg.DECODE_8B, dg.PREFILL_70B
    for cfg, want in ((c2, 2_950_144), (c3, 343_031_808)):
        s = bm.two_step_share(cfg.R, cfg.T, cfg.H, cfg.bits_rs, cfg.bits_ag, cfg.group)
        assert sum(bm.total(v) for v in s.values()) == want


def test_slots_and_tokenweave():
    c4 = dg.SLOTS  # 8 ranks x 524288 slots of 8 B, 64-slot blocks
    a = bm.ll_unpack(c4.R, c4.n, c4.block_slots)
    # slots 33,554,432 + out 2,097,152 + stale flags 65,536 = 35,717,120, plus the done flags read and written
    assert bm.total(a) == 35_717_120 + 2 * 8192
    c5 = dg.TOKENWEAVE
    h = bm.reduce_rmsnorm(c5.R, c5.splits[0], c5.H, True, True)
    assert h == dict(read=603_996_160, write=134_217_728) and bm.total(h) == 738_213_888


def test_flag_and_allgather_formulas():
    # 8 ranks x 2^20 elements with 2048-element blocks: payload 16 MiB + 8 x 512 flag words + 512 done flags
    f = bm.flag_unpack(8, 1 << 20, 2048)
    assert f == dict(read=16_777_216 + 16_384 + 512, write=2_097_152 + 4096 + 512)
    g = bm.ll_gather(2, 1024, 64, completed_blocks=30)  # 32 (rank, block) pairs, 30 complete
    assert g == dict(read=2 * 8 * 1024 + 32, write=4 * 64 * 30 + 32 + 30)
