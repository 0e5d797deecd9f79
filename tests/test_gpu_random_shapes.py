"""Seeded random shapes through the whole quantized two-step all-reduce (batched quantize, every shard's
reduce, gather + residual-add + RMSNorm) and, where shards hold whole rows, the norm-first path, against
the oracle: rank counts 1-16, every code width pair and group size, rows of 32 to 24576 elements, rows
that straddle shards, ragged row counts.  Rank messages, payloads, y and residual_out bit-exact; out
within 2 bf16 ulp; the norm-first path bit-exact in the kernels' sum-of-squares order."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _cases(count=64, seed=0x5EED):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        R = int(rng.integers(1, 17))
        group = int(rng.choice([32, 64, 128, 256]))
        b1, b2 = [(8, 8), (4, 8), (8, 4), (4, 4)][int(rng.integers(4))]
        # short rows (one or a few chunks per lane) and long ones (up to 24576: several chunks per lane,
        # and the norm-first path's chunk-per-lane kernel past 16384)
        H = group * int(rng.integers(1, 9)) if rng.random() < 0.7 else 1024 * int(rng.integers(1, 25))
        if rng.random() < 0.5:
            T = R * int(rng.integers(1, 6))          # shards of whole rows
        else:
            T = int(rng.integers(1, 4 * R + 1))      # rows may straddle shards
        if (T * H) % (R * group):
            continue
        out.append((R, T, H, b1, b2, group, int(rng.integers(1 << 30))))
    return out


def _bf16(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("R,T,H,b1,b2,group,seed", _cases(), ids=lambda v: str(v))
def test_random_shape(orc, R, T, H, b1, b2, group, seed):
    import torch
    from gpu_helpers import assert_bf16_close, assert_equal_bits, down, up
    from tensor_all_reduce_amd.flash_allreduce import TwoStepAllReduce
    rng = np.random.default_rng(seed)
    n = T * H
    scale = 10.0 ** rng.uniform(-2, 2)
    parts = [_bf16(scale * rng.standard_normal(n)) for _ in range(R)]
    res = _bf16(rng.standard_normal(n))
    gam = _bf16(1.0 + 0.1 * rng.standard_normal(H))
    eps = 1e-5
    ref = orc.two_step(parts, b1, b2, group, residual=res, gamma=gam, eps=eps, hidden=H)
    p = TwoStepAllReduce(R, T, H, b1, b2, group, parts=up(np.stack(parts)))
    y = torch.empty(n, dtype=torch.int16, device="cuda")
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    rout = torch.empty(n, dtype=torch.int16, device="cuda")
    p.run(y=y, norm=p.make_norm(up(gam), out, residual=up(res), residual_out=rout, eps=eps))
    torch.cuda.synchronize()
    where = f"R={R} T={T} H={H} bits={b1}/{b2} G={group}"
    assert_equal_bits(down(p.codes1, np.uint8).ravel(), ref["codes1"].ravel(), "codes1 " + where)
    assert_equal_bits(down(p.meta1, np.uint32).ravel(), ref["meta1"].ravel(), "meta1 " + where)
    assert_equal_bits(down(p.codes2, np.uint8), ref["codes2"], "codes2 " + where)
    assert_equal_bits(down(p.meta2, np.uint32), ref["meta2"], "meta2 " + where)
    assert_equal_bits(down(y, np.uint16), ref["y"], "y " + where)
    assert_equal_bits(down(rout, np.uint16), ref["residual_out"], "residual_out " + where)
    assert_bf16_close(down(out, np.uint16), ref["out"], 2, "out " + where)
    if (n // R) % H == 0:  # the norm-first path needs shards of whole rows
        nf = orc.two_step_normfirst(parts, b1, b2, group, res, gam, eps, H, order="tree")
        q = TwoStepAllReduce(R, T, H, b1, b2, group, parts=up(np.stack(parts)))
        y2 = torch.empty(n, dtype=torch.int16, device="cuda")
        rout2 = torch.empty(n, dtype=torch.int16, device="cuda")
        q.run_norm_first(y2, q.make_norm(up(gam), None, residual=up(res), residual_out=rout2, eps=eps))
        torch.cuda.synchronize()
        assert_equal_bits(down(q.codes2, np.uint8), nf["codes2"], "norm-first codes2 " + where)
        assert_equal_bits(down(q.meta2, np.uint32), nf["meta2"], "norm-first meta2 " + where)
        assert_equal_bits(down(rout2, np.uint16), nf["residual_out"], "norm-first residual_out " + where)
        assert_equal_bits(down(y2, np.uint16), nf["y"], "norm-first y " + where)
