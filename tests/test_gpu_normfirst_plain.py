"""GPU parity of the norm-before-all-gather path (fc_quantize -> fc_reduce_shard_norm -> fc_gather_dequant)
against the oracle's plain reading of it (TokenWeave, abstract: RMSNorm moved relative to the all-reduce),
whose sum of squares is the epilogue's left fold of the rounded squares.  The kernels add the squares in
their own fixed tree order; tests/normfirst_bound.py states what that allows: residual_out and every
group the order cannot decide otherwise bit-exact, the rest within one requantization step.  Both
workloads in full."""
import numpy as np
import pytest

from tensor_all_reduce_amd import datagen as dg

pytestmark = pytest.mark.gpu


def _run(orc, cfg):
    import torch
    from gpu_helpers import down, up
    from normfirst_bound import compare
    from tensor_all_reduce_amd.flash_allreduce import TwoStepAllReduce
    print(f"[f1 plain] {cfg.name}", flush=True)
    parts = dg.partials(cfg)
    res, gam = dg.residual(cfg), dg.gamma(cfg)
    p = TwoStepAllReduce(cfg.R, cfg.T, cfg.H, cfg.bits_rs, cfg.bits_ag, cfg.group, parts=up(np.stack(parts)))
    y = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    rout = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    p.run_norm_first(y, p.make_norm(up(gam), None, residual=up(res), residual_out=rout, eps=cfg.eps))
    torch.cuda.synchronize()
    got = dict(codes1=down(p.codes1, np.uint8), meta1=down(p.meta1, np.uint32), residual_out=down(rout, np.uint16),
               codes2=down(p.codes2, np.uint8), meta2=down(p.meta2, np.uint32), y=down(y, np.uint16))
    del p, y, rout
    compare(orc, cfg, parts, res, gam, got, log=lambda m: print("[f1 plain] " + m, flush=True))


def test_decode_in_full_against_plain_order(orc):
    _run(orc, dg.DECODE_8B)


@pytest.mark.timeout(300)
def test_prefill_in_full_against_plain_order(orc):
    _run(orc, dg.PREFILL_70B)


# Other launch paths of the same reading: rows longer than 16384 elements (the k_rows producer, whose tree
# runs over lanes, wavefronts, then a lane's chunks), a chunk count that is not a power of two (the tree
# pads with zeros), 4-bit codes out, group sizes 32 and 256.  Seeds use workload numbers of their own.
EXTRA = [
    dg.Config(31, "norm-first R=4 T=8 H=20480 int8/int8 G=128", "two_step", R=4, T=8, H=20480, sigma=1.0,
              outlier_p=0.01, outlier_factor=20.0, bits_rs=8, bits_ag=8, group=128),
    dg.Config(32, "norm-first R=2 T=12 H=1056 int4/int8 G=32", "two_step", R=2, T=12, H=1056, sigma=0.7,
              outlier_p=0.02, outlier_factor=30.0, bits_rs=4, bits_ag=8, group=32),
    dg.Config(33, "norm-first R=8 T=64 H=4096 int8/int4 G=256", "two_step", R=8, T=64, H=4096, sigma=0.5,
              outlier_p=0.005, outlier_factor=30.0, bits_rs=8, bits_ag=4, group=256),
]


@pytest.mark.parametrize("cfg", EXTRA, ids=lambda c: c.name)
def test_other_shapes_against_plain_order(orc, cfg):
    _run(orc, cfg)
