"""GPU parity of the reduce-scatter receive side with the norm before the all-gather
(fc_reduce_shard_norm) against the CPU oracle: every shard's fixed-order sum, residual add and RMSNorm
(fixed-order sum of squares), then the quantized normalized rows.  Codes, meta and residual_out
bit-exact; the gathered bf16 rows bit-exact too (they are the dequantized codes).  Inputs of every
step are the oracle's own outputs of the previous step."""
import numpy as np
import pytest

from tensor_all_reduce_amd import datagen as dg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fc():
    from tensor_all_reduce_amd import _lib
    return _lib


def _run_shards(orc, R, n_shards, rows, H, b1, b2, G, with_residual=True, seed=0):
    import torch
    from gpu_helpers import assert_equal_bits, down, up
    from tensor_all_reduce_amd import _lib
    L = rows * H
    rng = np.random.default_rng(seed)
    ins_host = []
    for s in range(n_shards):
        for r in range(R):
            x = dg.synth_bf16((s, r, b1, G, H, seed), L, sigma=0.5 + r, outlier_p=0.01, outlier_factor=30.0)
            ins_host.append(orc.quantize(x, b1, G))
    res = orc.f32_to_bf16(rng.standard_normal(n_shards * L).astype(np.float32)) if with_residual else None
    gam = orc.f32_to_bf16(rng.normal(1.0, 0.1, H).astype(np.float32))
    ins = [(up(c), up(m)) for c, m in ins_host]
    outs = [(torch.empty(L * b2 // 8, dtype=torch.uint8, device="cuda"),
             torch.empty(L // G, dtype=torch.int32, device="cuda")) for _ in range(n_shards)]
    rout = torch.empty(n_shards * L, dtype=torch.int16, device="cuda") if with_residual else None
    norm = dict(residual=up(res) if with_residual else None, gamma=up(gam), eps=1e-5, hidden=H, residual_out=rout)
    _lib.fc_reduce_shard_norm(ins, R, L, b1, b2, G, norm, outs)
    torch.cuda.synchronize()
    for s in range(n_shards):
        chunk = ins_host[s * R:(s + 1) * R]
        rc, rm, rro, _ = orc.reduce_norm_quant([c for c, _ in chunk], [m for _, m in chunk], L, b1, b2, G,
                                               res[s * L:(s + 1) * L] if with_residual else None, gam, 1e-5, H,
                                               order="tree")
        where = f"R={R} shard {s}/{n_shards} rows={rows} H={H} b={b1}/{b2} G={G}"
        assert_equal_bits(down(outs[s][1], np.uint32), rm, "meta " + where)
        assert_equal_bits(down(outs[s][0], np.uint8), rc, "codes " + where)
        if with_residual:
            assert_equal_bits(down(rout[s * L:(s + 1) * L], np.uint16), rro, "residual_out " + where)


@pytest.mark.parametrize("b1,b2", [(8, 8), (4, 8), (8, 4), (4, 4)])
@pytest.mark.parametrize("G", [32, 64, 128, 256])
def test_reduce_norm_bits_groups(fc, orc, b1, b2, G):
    _run_shards(orc, 8, 2, 3, 4096, b1, b2, G, seed=b1 * 100 + b2 * 10 + G)


# row shapes: 32 chunks (64 lanes), 128 chunks, 512 and 1024 chunks one per lane, 1536 chunks two per lane,
# 2560 chunks four per lane (a padded tree), many rows (256 lanes x 2 or 4 chunks)
@pytest.mark.parametrize("R,n_shards,rows,H", [(1, 1, 2, 256), (2, 3, 1, 1024), (8, 1, 2, 4096), (16, 2, 1, 8192),
                                               (3, 2, 1, 12288), (2, 1, 2, 20480), (2, 2, 150, 4096),
                                               (2, 2, 130, 8192), (4, 9, 1, 1024)])
def test_reduce_norm_shapes(fc, orc, R, n_shards, rows, H):
    _run_shards(orc, R, n_shards, rows, H, 8, 8, 128, seed=R * 7 + rows + H)


# 16-element slots per lane: a row of 6 slots (lanes past it hold a clamped copy and store nothing, whole
# 2-lane groups of them), 1022 slots (an unaligned wavefront tail; from 2 ranks, the chunk-per-lane
# kernel), 1024 slots (the largest one-slot row), and 1026 slots (past it: the chunk-per-lane kernel)
@pytest.mark.parametrize("R,rows,H", [(3, 5, 96), (8, 1, 16352), (2, 1, 16352), (8, 2, 16384), (2, 1, 16416)])
def test_reduce_norm_slot_edges(fc, orc, R, rows, H):
    _run_shards(orc, R, 2, rows, H, 8, 4, 32, seed=R * 5 + H)


# many short rows (over 8000 one-row workgroups of 64 lanes); 16 ranks add a second batch of rank loads
@pytest.mark.parametrize("R,rows,H,b1", [(3, 4500, 96, 8), (16, 4200, 256, 4)])
def test_reduce_norm_many_rows(fc, orc, R, rows, H, b1):
    _run_shards(orc, R, 2, rows, H, b1, 8, 32, seed=R + rows)


def test_reduce_norm_without_residual(fc, orc):
    _run_shards(orc, 4, 2, 2, 4096, 8, 8, 128, with_residual=False, seed=11)


@pytest.mark.parametrize("workload", ["tiny-r2-t4-h256", "llama3-8b-decode"])
def test_norm_first_end_to_end(fc, orc, workload):
    """Quantize all ranks, every shard's reduce + norm + quantization, gather of the normalized rows,
    against the oracle's whole norm-first all-reduce."""
    import torch
    from gpu_helpers import assert_equal_bits, down, up
    from tensor_all_reduce_amd.flash_allreduce import TwoStepAllReduce
    cfg = dg.WORKLOADS[workload]
    parts = dg.partials(cfg)
    res, gam = dg.residual(cfg), dg.gamma(cfg)
    ref = orc.two_step_normfirst(parts, cfg.bits_rs, cfg.bits_ag, cfg.group, res, gam, cfg.eps, cfg.H, order="tree")
    p = TwoStepAllReduce(cfg.R, cfg.T, cfg.H, cfg.bits_rs, cfg.bits_ag, cfg.group, parts=up(np.stack(parts)))
    y = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    rout = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    p.run_norm_first(y, p.make_norm(up(gam), None, residual=up(res), residual_out=rout, eps=cfg.eps))
    assert_equal_bits(down(p.codes1, np.uint8).ravel(), ref["codes1"].ravel(), "rank messages: codes")
    assert_equal_bits(down(p.meta2, np.uint32), ref["meta2"], "normalized payload: meta")
    assert_equal_bits(down(p.codes2, np.uint8), ref["codes2"], "normalized payload: codes")
    assert_equal_bits(down(rout, np.uint16), ref["residual_out"], "residual_out")
    assert_equal_bits(down(y, np.uint16), ref["y"], "gathered normalized rows")


def test_norm_first_70b_prefill_sampled(fc, orc):
    """8 x [4096, 8192], int4 reduce-scatter, int8 normalized all-gather, in the benchmark's launch
    configuration; sampled rows recomputed by the oracle from the partial sums (a row's groups and norm
    need only that row)."""
    import torch
    from gpu_helpers import assert_equal_bits, down, up
    from tensor_all_reduce_amd.flash_allreduce import TwoStepAllReduce
    cfg = dg.PREFILL_70B
    R, T, H, G, b1, b2 = cfg.R, cfg.T, cfg.H, cfg.group, cfg.bits_rs, cfg.bits_ag
    parts = dg.partials(cfg)
    res, gam = dg.residual(cfg), dg.gamma(cfg)
    p = TwoStepAllReduce(R, T, H, b1, b2, G, parts=up(np.stack(parts)))
    y = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    rout = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    p.run_norm_first(y, p.make_norm(up(gam), None, residual=up(res), residual_out=rout, eps=cfg.eps))
    torch.cuda.synchronize()
    rps = T // R
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, T - 1], np.arange(R) * rps, np.arange(1, R + 1) * rps - 1,
                                     rng.integers(0, T, 12)]))
    codes2, meta2 = p.codes2.cpu().numpy(), p.meta2.cpu().numpy().view(np.uint32)
    y_h, rout_h = down(y, np.uint16), down(rout, np.uint16)
    gpr = H // G
    for t in rows:
        sl = slice(t * H, (t + 1) * H)
        msgs = [orc.quantize(parts[r][sl], b1, G) for r in range(R)]
        c2, m2, ro, _ = orc.reduce_norm_quant([c for c, _ in msgs], [m for _, m in msgs], H, b1, b2, G, res[sl],
                                              gam, cfg.eps, H, order="tree")
        assert_equal_bits(codes2[t * H * b2 // 8:(t + 1) * H * b2 // 8], c2, f"row {t} payload codes")
        assert_equal_bits(meta2[t * gpr:(t + 1) * gpr], m2, f"row {t} payload meta")
        assert_equal_bits(rout_h[sl], ro, f"row {t} residual_out")
        yo = orc.gather([c2], [m2], H, b2, G, plain=True)
        assert_equal_bits(y_h[sl], yo[0] if isinstance(yo, tuple) else yo, f"row {t} gathered")
