"""GPU parity of the two-step all-reduce (fc_reduce_shard, fc_gather_dequant) against the CPU oracle.

Each step is fed the oracle's own output of the previous step (so inputs never come from the HIP
path), then the whole GPU pipeline is compared end to end on the decode workloads and, element by
element, on the 70B prefill workload (8 x [4096, 8192], int4 reduce-scatter, int8 all-gather).  Codes
and meta bit-exact; bf16 outputs within 2 ulp."""
import numpy as np
import pytest

from tensor_all_reduce_amd import datagen as dg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fc():
    from tensor_all_reduce_amd import _lib
    return _lib


def _qmsgs_on_gpu(msgs):
    from gpu_helpers import up
    return [(up(c), up(m)) for c, m in msgs]


@pytest.mark.parametrize("b1,b2", [(8, 8), (4, 8), (8, 4), (4, 4)])
@pytest.mark.parametrize("group", [32, 64, 128, 256])
@pytest.mark.parametrize("R,n_shards", [(1, 1), (2, 2), (3, 1), (8, 8), (8, 1), (16, 16)])
def test_reduce_shard_parity(fc, orc, b1, b2, group, R, n_shards):
    import torch
    from gpu_helpers import assert_equal_bits, down
    L = group * (37 if R < 16 else 9)  # ragged: not a multiple of a workgroup's elements
    ins_host = []
    for s in range(n_shards):
        for r in range(R):
            x = dg.synth_bf16((s, r, b1, group), L, sigma=1.0 + r, outlier_p=0.01, outlier_factor=30.0)
            ins_host.append(orc.quantize(x, b1, group))
    ins = _qmsgs_on_gpu(ins_host)
    outs = [(torch.empty(L * b2 // 8, dtype=torch.uint8, device="cuda"),
             torch.empty(L // group, dtype=torch.int32, device="cuda")) for _ in range(n_shards)]
    fc.fc_reduce_shard(ins, R, L, b1, b2, group, outs)
    for s in range(n_shards):
        chunk = ins_host[s * R:(s + 1) * R]
        rc, rm = orc.reduce_shard([c for c, _ in chunk], [m for _, m in chunk], L, b1, b2, group)
        assert_equal_bits(down(outs[s][1], np.uint32), rm, f"meta shard {s}")
        assert_equal_bits(down(outs[s][0], np.uint8), rc, f"codes shard {s}")


def test_reduce_order_cancellation(fc, orc):
    """Ranks 0, 1, 2 dequantize to 2^15, -2^15, 2^-10: only the ascending fold keeps 2^-10."""
    import torch
    from gpu_helpers import down
    G, L = 32, 32 * 64
    msgs = [orc.quantize(dg.f32_to_bf16_bits(np.full(L, v, np.float32)), 8, G)
            for v in (2.0 ** 15, -(2.0 ** 15), 2.0 ** -10)]
    ins = _qmsgs_on_gpu(msgs)
    out = (torch.empty(L, dtype=torch.uint8, device="cuda"), torch.empty(L // G, dtype=torch.int32, device="cuda"))
    fc.fc_reduce_shard(ins, 3, L, 8, 8, G, [out])
    y = orc.dequant(down(out[0], np.uint8), down(out[1], np.uint32), L, 8, G)
    assert np.all(y == np.float32(2.0 ** -10))


def _shard_msgs(orc, R, L, bits, group, seed, sigma=6.0):
    """Requantized shards as the oracle makes them from fp32 sums (the all-gather payload)."""
    return [orc.quantize(dg.synth_f32((seed, s), L, sigma), bits, group) for s in range(R)]


# (R, T, H) shapes, each with every group that splits its shards into whole groups
_GATHER_SHAPES = [(2, 4, 256), (8, 64, 4096), (8, 3, 4096), (4, 16, 8192), (3, 6, 2048), (8, 1, 4096), (1, 5, 12288),
                  (16, 2, 1024), (5, 8, 1000), (2, 2, 65536)]
_GATHER_CASES = [(G, R, T, H) for R, T, H in _GATHER_SHAPES for G in (32, 64, 128, 256)
                 if (T * H) % R == 0 and (T * H // R) % G == 0]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group,R,T,H", _GATHER_CASES)
def test_gather_parity(fc, orc, bits, group, R, T, H):
    """Plain dequantize and the fused residual-add + RMSNorm epilogue; includes rows that straddle shards
    (T*H/R not a multiple of H, e.g. one decode token) and row lengths needing 1..4 chunks per lane."""
    import torch
    from gpu_helpers import assert_bf16_close, assert_equal_bits, down, up
    n = T * H
    L = n // R
    shards = _shard_msgs(orc, R, L, bits, group, seed=(R, T, H, bits))
    dsh = _qmsgs_on_gpu(shards)
    res = dg.synth_bf16((7, R, T, H), n)
    gam = dg.f32_to_bf16_bits(dg.synth_f32((8, H), H, 0.1) + 1.0)
    y_ref, out_ref, rout_ref = orc.gather([c for c, _ in shards], [m for _, m in shards], L, bits, group, plain=True,
                                          residual=res, gamma=gam, eps=1e-5, hidden=H)
    # plain
    y = torch.empty(n, dtype=torch.int16, device="cuda")
    fc.fc_gather_dequant(dsh, L, bits, group, y=y)
    assert_equal_bits(down(y, np.uint16), y_ref, "y")
    # norm with residual, separate residual_out
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    rout = torch.empty(n, dtype=torch.int16, device="cuda")
    dres, dgam = up(res), up(gam)
    fc.fc_gather_dequant(dsh, L, bits, group, norm=dict(residual=dres, gamma=dgam, eps=1e-5, hidden=H, out=out,
                                                         residual_out=rout))
    assert_bf16_close(down(out, np.uint16), out_ref, 2, "out")
    assert_bf16_close(down(rout, np.uint16), rout_ref, 0, "residual_out")
    # in place: residual_out == residual, and y in the same call
    y2 = torch.empty(n, dtype=torch.int16, device="cuda")
    out2 = torch.empty(n, dtype=torch.int16, device="cuda")
    fc.fc_gather_dequant(dsh, L, bits, group, y=y2, norm=dict(residual=dres, gamma=dgam, eps=1e-5, hidden=H, out=out2,
                                                               residual_out=dres))
    assert_equal_bits(down(y2, np.uint16), y_ref, "y (with norm)")
    assert_equal_bits(down(out2, np.uint16), down(out, np.uint16), "out in place")
    assert_equal_bits(down(dres, np.uint16), down(rout, np.uint16), "residual updated in place")
    # no residual
    _, out_nr, _ = orc.gather([c for c, _ in shards], [m for _, m in shards], L, bits, group, plain=False,
                              residual=None, gamma=gam, eps=1e-5, hidden=H)
    out3 = torch.empty(n, dtype=torch.int16, device="cuda")
    fc.fc_gather_dequant(dsh, L, bits, group, norm=dict(gamma=dgam, eps=1e-5, hidden=H, out=out3))
    assert_bf16_close(down(out3, np.uint16), out_nr, 2, "out (no residual)")


def _pipeline(cfg, parts_np):
    import torch
    from gpu_helpers import up
    from tensor_all_reduce_amd.flash_allreduce import TwoStepAllReduce
    p = TwoStepAllReduce(cfg.R, cfg.T, cfg.H, cfg.bits_rs, cfg.bits_ag, cfg.group, device="cuda",
                         parts=up(np.stack(parts_np)))
    return p


@pytest.mark.parametrize("workload", ["tiny-r2-t4-h256", "llama3-8b-decode"])
def test_two_step_end_to_end(fc, orc, workload):
    """The whole GPU pipeline (batched quantize, all shards' reduce-scatter, gather + epilogue) against the
    oracle's whole two-step all-reduce, stage by stage."""
    import torch
    from gpu_helpers import assert_bf16_close, assert_equal_bits, down, up
    cfg = dg.WORKLOADS[workload]
    parts = dg.partials(cfg)
    res, gam = dg.residual(cfg), dg.gamma(cfg)
    ref = orc.two_step(parts, cfg.bits_rs, cfg.bits_ag, cfg.group, residual=res, gamma=gam, eps=cfg.eps, hidden=cfg.H)
    p = _pipeline(cfg, parts)
    y = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    out = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    rout = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    norm = p.make_norm(up(gam), out, residual=up(res), residual_out=rout, eps=cfg.eps)
    p.run(y=y, norm=norm)
    assert_equal_bits(down(p.meta1, np.uint32).ravel(), ref["meta1"].ravel(), "rank messages: meta")
    assert_equal_bits(down(p.codes1, np.uint8).ravel(), ref["codes1"].ravel(), "rank messages: codes")
    assert_equal_bits(down(p.meta2, np.uint32), ref["meta2"], "all-gather payload: meta")
    assert_equal_bits(down(p.codes2, np.uint8), ref["codes2"], "all-gather payload: codes")
    assert_equal_bits(down(y, np.uint16), ref["y"], "y")
    assert_bf16_close(down(rout, np.uint16), ref["residual_out"], 0, "residual_out")
    assert_bf16_close(down(out, np.uint16), ref["out"], 2, "out")
    # one GPU's real share: reducing only shard s reproduces that shard's payload
    p.codes2.zero_()
    p.meta2.zero_()
    s = cfg.R - 1
    p.reduce_scatter(shard=s)
    c2, m2 = p.shard_msg(s)
    cb, mb = cfg.L * cfg.bits_ag // 8, cfg.L // cfg.group
    assert_equal_bits(down(c2, np.uint8), ref["codes2"][s * cb:(s + 1) * cb], "shard-only codes")
    assert_equal_bits(down(m2, np.uint32), ref["meta2"][s * mb:(s + 1) * mb], "shard-only meta")
    assert np.all(down(p.meta2, np.uint32)[:s * mb] == 0)


@pytest.mark.timeout(300)
def test_two_step_70b_prefill_full(fc, orc):
    """8 x [4096, 8192]: int4 reduce-scatter, int8 all-gather, residual-add + RMSNorm, in the launch
    configuration the benchmark times, against the oracle's whole run: every code and meta word of the
    rank messages and of the all-gather payload, every residual_out and out element."""
    import torch
    from gpu_helpers import assert_bf16_close, assert_equal_bits, down, up
    cfg = dg.PREFILL_70B
    print(f"[full] {cfg.name}", flush=True)
    parts = dg.partials(cfg)
    res, gam = dg.residual(cfg), dg.gamma(cfg)
    p = _pipeline(cfg, parts)
    out = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    rout = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
    norm = p.make_norm(up(gam), out, residual=up(res), residual_out=rout, eps=cfg.eps)
    p.run(norm=norm)
    torch.cuda.synchronize()
    got = dict(codes1=down(p.codes1, np.uint8), meta1=down(p.meta1, np.uint32), codes2=down(p.codes2, np.uint8),
               meta2=down(p.meta2, np.uint32), out=down(out, np.uint16), residual_out=down(rout, np.uint16))
    del p, out, rout, norm
    torch.cuda.empty_cache()
    ref = orc.two_step(parts, cfg.bits_rs, cfg.bits_ag, cfg.group, residual=res, gamma=gam, eps=cfg.eps,
                       hidden=cfg.H, plain=False)
    assert_equal_bits(got["meta1"].ravel(), ref["meta1"].ravel(), "rank messages: meta")
    assert_equal_bits(got["codes1"].ravel(), ref["codes1"].ravel(), "rank messages: codes")
    assert_equal_bits(got["meta2"], ref["meta2"], "all-gather payload: meta")
    assert_equal_bits(got["codes2"], ref["codes2"], "all-gather payload: codes")
    assert_equal_bits(got["residual_out"], ref["residual_out"], "residual_out")
    exact = assert_bf16_close(got["out"], ref["out"], 2, "out")
    print(f"[full] {cfg.name}: {cfg.n} outputs, {100 * exact:.3f}% bit-identical, the rest within 2 ulp", flush=True)


def test_two_step_deterministic_repeat(fc):
    """The same inputs give the same bits on every call (no atomics, fixed order)."""
    import torch
    from gpu_helpers import up
    cfg = dg.DECODE_8B
    parts = dg.partials(cfg)
    p = _pipeline(cfg, parts)
    outs = []
    for _ in range(3):
        y = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
        out = torch.empty(cfg.n, dtype=torch.int16, device="cuda")
        norm = p.make_norm(up(dg.gamma(cfg)), out, residual=up(dg.residual(cfg)), eps=cfg.eps)
        p.run(y=y, norm=norm)
        outs.append((y.cpu(), out.cpu(), p.codes2.cpu().clone()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a, b)


@pytest.mark.parametrize("b1,b2", [(8, 8), (4, 8)])
@pytest.mark.parametrize("log2_L", [17, 19])
def test_reduce_shard_large_shards(fc, orc, b1, b2, log2_L):
    """Shards large enough for the 8-element (2^17) and 16-element (2^19) lane chunks of the launcher
    (8 shards x 8 ranks x (2^k + 384) elements, a ragged tail), compared in full; smaller shards of
    8-bit codes use 4-element chunks and are covered by the parity test above."""
    import torch
    from gpu_helpers import assert_equal_bits, down
    R, G = 8, 128
    L = (1 << log2_L) + 3 * G
    ins_host = []
    for s in range(R):
        for r in range(R):
            x = dg.synth_bf16((s, r, b1, 999), L, sigma=1.0, outlier_p=0.001, outlier_factor=50.0)
            ins_host.append(orc.quantize(x, b1, G))
    ins = _qmsgs_on_gpu(ins_host)
    outs = [(torch.empty(L * b2 // 8, dtype=torch.uint8, device="cuda"),
             torch.empty(L // G, dtype=torch.int32, device="cuda")) for _ in range(R)]
    fc.fc_reduce_shard(ins, R, L, b1, b2, G, outs)
    for s in (0, R - 1):
        chunk = ins_host[s * R:(s + 1) * R]
        rc, rm = orc.reduce_shard([c for c, _ in chunk], [m for _, m in chunk], L, b1, b2, G)
        assert_equal_bits(down(outs[s][1], np.uint32), rm, f"meta shard {s}")
        assert_equal_bits(down(outs[s][0], np.uint8), rc, f"codes shard {s}")
