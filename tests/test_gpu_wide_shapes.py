"""Kernel shapes that only large inputs select, against the oracle for every code width and group size
(Flash Communication, "Core ideas": two-step all-reduce):

  * the reduce-scatter's 16-element chunks per lane (chosen once a launch has 2048 workgroups of them):
    8 ranks x 8 shards of a little over 2^20 elements, every (b1, b2) pair and group, a ragged last
    workgroup, and rank counts of 3, 5 and 16 (the rank count known only at run time); codes and meta
    bit-exact;
  * the all-gather + residual-add + RMSNorm epilogue with more than 256 rows, in every row shape that
    many rows select (256 x 1 to 1024 x 8 lanes x chunks), rows inside one shard or across shard
    boundaries, 4-bit and 8-bit payloads, several groups; y and residual_out bit-exact, out within 2 ulp;
  * the unquantized reduce + RMSNorm with more than 256 rows in each row shape, and capped grids that
    keep 2 or 4 rows in flight per workgroup.

The rank messages are drawn directly (uniform codes, fp16 scales and zero-points in a fixed range): the
oracle's dequantization defines their values whatever produced them."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fc():
    from tensor_all_reduce_amd import _lib
    return _lib


def _msg(rng, L, bits, group, scale_range=(1e-3, 5e-2), zero_range=(-4.0, 0.0)):
    codes = rng.integers(0, 256, L * bits // 8, dtype=np.uint8)
    s = rng.uniform(*scale_range, L // group).astype(np.float16).view(np.uint16).astype(np.uint32)
    z = rng.uniform(*zero_range, L // group).astype(np.float16).view(np.uint16).astype(np.uint32)
    return codes, (s | (z << 16)).astype(np.uint32)


@pytest.mark.parametrize("b1,b2", [(8, 8), (4, 8), (8, 4), (4, 4)])
@pytest.mark.parametrize("group", [32, 64, 128, 256])
def test_reduce_sixteen_element_chunks(fc, orc, b1, b2, group):
    import torch
    from gpu_helpers import assert_equal_bits, down, up
    R, n_shards = 8, 8
    L = (1 << 20) + 3 * group  # 2^16 + 3G/16 chunks of 16 per shard: more than 2048 workgroups in all
    rng = np.random.default_rng((b1, b2, group))
    host = [_msg(rng, L, b1, group) for _ in range(n_shards * R)]
    ins = [(up(c), up(m)) for c, m in host]
    outs = [(torch.empty(L * b2 // 8, dtype=torch.uint8, device="cuda"),
             torch.empty(L // group, dtype=torch.int32, device="cuda")) for _ in range(n_shards)]
    fc.fc_reduce_shard(ins, R, L, b1, b2, group, outs)
    torch.cuda.synchronize()
    for s in range(n_shards):
        chunk = host[s * R:(s + 1) * R]
        rc, rm = orc.reduce_shard([c for c, _ in chunk], [m for _, m in chunk], L, b1, b2, group)
        where = f"shard {s} bits {b1}->{b2} G={group}"
        assert_equal_bits(down(outs[s][1], np.uint32), rm, "meta " + where)
        assert_equal_bits(down(outs[s][0], np.uint8), rc, "codes " + where)


@pytest.mark.parametrize("bits,group", [(4, 32), (4, 128), (4, 256), (8, 32), (8, 256)])
def test_gather_norm_256_lane_rows(fc, orc, bits, group):
    import torch
    from gpu_helpers import assert_bf16_close, assert_equal_bits, down, up
    R, T, H = 8, 520, 8192  # 520 rows: the 256-lane x 4-chunk row shape, rows straddling no shard
    n = T * H
    L = n // R
    rng = np.random.default_rng((bits, group, 5))
    shards = [_msg(rng, L, bits, group, scale_range=(1e-2, 3e-1), zero_range=(-2.0, 0.0)) for _ in range(R)]
    res = (rng.standard_normal(n).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    gam = ((1.0 + 0.1 * rng.standard_normal(H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y_ref, out_ref, rout_ref = orc.gather([c for c, _ in shards], [m for _, m in shards], L, bits, group, plain=True,
                                          residual=res, gamma=gam, eps=1e-5, hidden=H)
    dsh = [(up(c), up(m)) for c, m in shards]
    y = torch.empty(n, dtype=torch.int16, device="cuda")
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    rout = torch.empty(n, dtype=torch.int16, device="cuda")
    fc.fc_gather_dequant(dsh, L, bits, group, y=y,
                         norm=dict(residual=up(res), gamma=up(gam), eps=1e-5, hidden=H, out=out, residual_out=rout))
    torch.cuda.synchronize()
    where = f"bits {bits} G={group}"
    assert_equal_bits(down(y, np.uint16), y_ref, "y " + where)
    assert_equal_bits(down(rout, np.uint16), rout_ref, "residual_out " + where)
    assert_bf16_close(down(out, np.uint16), out_ref, 2, "out " + where)


@pytest.mark.parametrize("R,b1,b2,group", [(16, 8, 8, 128), (16, 4, 8, 64), (5, 4, 4, 256), (3, 8, 4, 32)])
def test_reduce_sixteen_element_chunks_other_rank_counts(fc, orc, R, b1, b2, group):
    """The same chunk shape with the rank count known only at run time (two batches of loads at R = 16)."""
    import torch
    from gpu_helpers import assert_equal_bits, down, up
    n_shards = R
    L = -(-(2048 * 256 * 16) // n_shards) // group * group + group  # at least 2048 workgroups of 16-element chunks
    rng = np.random.default_rng((R, b1, b2, group))
    host = [_msg(rng, L, b1, group) for _ in range(n_shards * R)]
    ins = [(up(c), up(m)) for c, m in host]
    outs = [(torch.empty(L * b2 // 8, dtype=torch.uint8, device="cuda"),
             torch.empty(L // group, dtype=torch.int32, device="cuda")) for _ in range(n_shards)]
    fc.fc_reduce_shard(ins, R, L, b1, b2, group, outs)
    torch.cuda.synchronize()
    for s in (0, n_shards // 2, n_shards - 1):
        chunk = host[s * R:(s + 1) * R]
        rc, rm = orc.reduce_shard([c for c, _ in chunk], [m for _, m in chunk], L, b1, b2, group)
        where = f"R={R} shard {s} bits {b1}->{b2} G={group}"
        assert_equal_bits(down(outs[s][1], np.uint32), rm, "meta " + where)
        assert_equal_bits(down(outs[s][0], np.uint8), rc, "codes " + where)


@pytest.mark.parametrize("R,T,H,bits,group", [(8, 300, 2048, 8, 128), (8, 300, 4096, 4, 64), (4, 260, 16384, 8, 256),
                                              (8, 264, 32768, 4, 128), (2, 258, 65536, 8, 32), (8, 300, 12288, 8, 128)])
def test_gather_norm_many_rows(fc, orc, R, T, H, bits, group):
    """More than 256 rows in each row shape (256 x 1, 256 x 2, 512 x 4, 1024 x 4, 1024 x 8 lanes x chunks);
    T = 300 with 8 ranks puts rows across shard boundaries (the pointer table staged in LDS)."""
    import torch
    from gpu_helpers import assert_bf16_close, assert_equal_bits, down, up
    n = T * H
    L = n // R
    rng = np.random.default_rng((R, T, H, bits, group))
    shards = [_msg(rng, L, bits, group, scale_range=(1e-2, 3e-1), zero_range=(-2.0, 0.0)) for _ in range(R)]
    res = (rng.standard_normal(n).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    gam = ((1.0 + 0.1 * rng.standard_normal(H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y_ref, out_ref, rout_ref = orc.gather([c for c, _ in shards], [m for _, m in shards], L, bits, group, plain=True,
                                          residual=res, gamma=gam, eps=1e-5, hidden=H)
    dsh = [(up(c), up(m)) for c, m in shards]
    y = torch.empty(n, dtype=torch.int16, device="cuda")
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    rout = torch.empty(n, dtype=torch.int16, device="cuda")
    fc.fc_gather_dequant(dsh, L, bits, group, y=y,
                         norm=dict(residual=up(res), gamma=up(gam), eps=1e-5, hidden=H, out=out, residual_out=rout))
    torch.cuda.synchronize()
    where = f"R={R} T={T} H={H} bits {bits} G={group}"
    assert_equal_bits(down(y, np.uint16), y_ref, "y " + where)
    assert_equal_bits(down(rout, np.uint16), rout_ref, "residual_out " + where)
    assert_bf16_close(down(out, np.uint16), out_ref, 2, "out " + where)


@pytest.mark.parametrize("R,rows,H,mw", [(8, 300, 2048, 0), (16, 300, 4096, 0), (3, 260, 16384, 0), (8, 264, 32768, 0),
                                         (2, 258, 65536, 0), (8, 400, 1024, 50), (8, 300, 8192, 64), (5, 520, 4096, 100),
                                         (8, 300, 256, 32)])
def test_reduce_rmsnorm_many_rows(fc, orc, R, rows, H, mw):
    """The unquantized reduce + RMSNorm (TokenWeave, abstract) with more than 256 rows in each row shape,
    and capped grids that keep 2 or 4 rows in flight per workgroup."""
    import torch
    from gpu_helpers import assert_bf16_close, assert_equal_bits, down, up
    n = rows * H
    rng = np.random.default_rng((R, rows, H, mw))
    bf = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    parts = [bf(rng.standard_normal(n)) for _ in range(R)]
    res, gam = bf(rng.standard_normal(n)), bf(1.0 + 0.1 * rng.standard_normal(H))
    o, ro, _ = orc.reduce_rmsnorm(parts, rows, H, res, gam, 1e-5)
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    rout = torch.empty(n, dtype=torch.int16, device="cuda")
    fc.fc_reduce_rmsnorm([up(p) for p in parts], rows,
                         dict(residual=up(res), gamma=up(gam), eps=1e-5, hidden=H, out=out, residual_out=rout),
                         max_workgroups=mw)
    torch.cuda.synchronize()
    where = f"R={R} rows={rows} H={H} max_workgroups={mw}"
    assert_equal_bits(down(rout, np.uint16), ro, "residual_out " + where)
    assert_bf16_close(down(out, np.uint16), o, 2, "out " + where)
