"""GPU parity of fc_reduce_rmsnorm (unquantized fused all-reduce + residual-add + RMSNorm, TokenWeave)
against the CPU oracle, the compute-unit cap (max_workgroups) and the wave-aware token split."""
import numpy as np
import pytest

from tensor_all_reduce_amd import datagen as dg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fc():
    from tensor_all_reduce_amd import _lib
    return _lib


def _run(fc, parts_d, rows, H, gam_d, res_d=None, rout_d=None, max_wg=0, eps=1e-5):
    import torch
    out = torch.empty(rows * H, dtype=torch.int16, device="cuda")
    fc.fc_reduce_rmsnorm(parts_d, rows, dict(residual=res_d, gamma=gam_d, eps=eps, hidden=H, out=out,
                                             residual_out=rout_d), max_workgroups=max_wg)
    return out


@pytest.mark.parametrize("R", [1, 2, 5, 8, 16])
@pytest.mark.parametrize("rows,H", [(3, 256), (5, 4096), (7, 8192), (2, 12288), (4, 1024), (2, 20480), (3, 1000),
                                    (2, 65536)])
def test_reduce_rmsnorm_parity(fc, orc, R, rows, H):
    import torch
    from gpu_helpers import assert_bf16_close, down, up
    n = rows * H
    parts = [dg.synth_bf16((R, rows, H, r), n, sigma=1.0) for r in range(R)]
    res = dg.synth_bf16((R, rows, H, 99), n)
    gam = dg.f32_to_bf16_bits(dg.synth_f32((H, 3), H, 0.1) + 1.0)
    out_ref, rout_ref, _ = orc.reduce_rmsnorm(parts, rows, H, res, gam, 1e-5)
    pd = [up(p) for p in parts]
    rout = torch.empty(n, dtype=torch.int16, device="cuda")
    out = _run(fc, pd, rows, H, up(gam), up(res), rout)
    assert_bf16_close(down(rout, np.uint16), rout_ref, 0, "residual_out")
    assert_bf16_close(down(out, np.uint16), out_ref, 2, "out")
    # no residual
    out_nr, _, _ = orc.reduce_rmsnorm(parts, rows, H, None, gam, 1e-5)
    assert_bf16_close(down(_run(fc, pd, rows, H, up(gam)), np.uint16), out_nr, 2, "out (no residual)")


def test_identical_partials_sum_exactly(fc, orc):
    """R identical bf16 partials: residual_out (no residual) is exactly R*x."""
    import torch
    from gpu_helpers import down, up
    rows, H, R = 4, 4096, 8
    x = dg.synth_bf16((1,), rows * H)
    rout = torch.empty(rows * H, dtype=torch.int16, device="cuda")
    zero = up(np.zeros(rows * H, np.uint16))
    _run(fc, [up(x)] * R, rows, H, up(dg.f32_to_bf16_bits(np.ones(H, np.float32))), zero, rout)
    got = dg.bf16_bits_to_f32(down(rout, np.uint16)).astype(np.float64)
    assert np.array_equal(got, R * dg.bf16_bits_to_f32(x).astype(np.float64))


def test_max_workgroups_and_split_invariance(fc):
    """Capping the grid (compute-unit footprint) or splitting the rows into two calls changes no bit."""
    import torch
    from gpu_helpers import up
    R, rows, H = 8, 96, 8192
    parts = [up(dg.synth_bf16((5, r), rows * H)) for r in range(R)]
    gam = up(dg.f32_to_bf16_bits(dg.synth_f32((6,), H, 0.1) + 1.0))
    res = up(dg.synth_bf16((7,), rows * H))
    base = _run(fc, parts, rows, H, gam, res)
    for mw in (1, 2, 8, 40, 96, 1000):
        assert torch.equal(_run(fc, parts, rows, H, gam, res, max_wg=mw), base), mw
    # token split: rows [0, 40) then [40, 96), on views of the same buffers
    a = 40
    out_a = _run(fc, [p[:a * H] for p in parts], a, H, gam, res[:a * H])
    out_b = _run(fc, [p[a * H:] for p in parts], rows - a, H, gam, res[a * H:])
    assert torch.equal(torch.cat([out_a, out_b]), base)


@pytest.mark.timeout(300)
def test_tokenweave_workload_full(fc, orc):
    """8 x [8192, 8192] bf16 split into two wave-aware halves of 4096 rows, each reduced on its own (as
    the benchmark does); the halves equal the unsplit call bit for bit, and every out and residual_out
    element of both halves matches the oracle's whole run."""
    import torch
    from gpu_helpers import assert_bf16_close, assert_equal_bits, down, up
    cfg = dg.TOKENWEAVE
    R, T, H = cfg.R, cfg.T, cfg.H
    print(f"[full] {cfg.name}", flush=True)
    parts_h = [dg.partial(cfg, r) for r in range(R)]
    res_h, gam_h = dg.residual(cfg), dg.gamma(cfg)
    parts = [up(p) for p in parts_h]
    gam, res = up(gam_h), up(res_h)
    rout = torch.empty(T * H, dtype=torch.int16, device="cuda")
    whole = _run(fc, parts, T, H, gam, res, rout)
    a = cfg.splits[0]
    halves = []
    for lo, hi in ((0, a), (a, T)):
        halves.append(_run(fc, [p[lo * H:hi * H] for p in parts], hi - lo, H, gam, res[lo * H:hi * H]))
    assert torch.equal(torch.cat(halves), whole)
    out_h = np.concatenate([down(h, np.uint16) for h in halves])
    rout_h = down(rout, np.uint16)
    del parts, halves, whole, rout
    torch.cuda.empty_cache()
    o, ro, _ = orc.reduce_rmsnorm(parts_h, T, H, res_h, gam_h, cfg.eps)
    assert_equal_bits(rout_h, ro, "residual_out")
    exact = assert_bf16_close(out_h, o, 2, "out")
    print(f"[full] {cfg.name}: {T * H} outputs, {100 * exact:.3f}% bit-identical, the rest within 2 ulp", flush=True)
