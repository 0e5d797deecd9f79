"""GPU parity of fc_quantize against the CPU oracle: codes and meta bit-exact.

Sizes span several workgroups with a ragged last one; edge-case groups (constants, signed zeros, fp16
subnormal range, top of the fp16 range, half-step ties, huge outliers); the workload shapes in full
where the oracle is quick, the 70B-prefill shape (8 ranks x 4096 x 8192, int4) on sampled groups, and
inputs large enough for the several-chunks-per-lane kernel shape in full for every code width and group."""
import numpy as np
import pytest

from tensor_all_reduce_amd import datagen as dg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fc():
    from tensor_all_reduce_amd import _lib
    return _lib


def run_quantize(fc, xb, bits, group):
    import torch
    from gpu_helpers import up, down
    n = xb.size
    x = up(xb)
    codes = torch.empty(n * bits // 8, dtype=torch.uint8, device=x.device)
    meta = torch.empty(n // group, dtype=torch.int32, device=x.device)
    fc.fc_quantize(x, bits, group, codes, meta)
    return down(codes, np.uint8), down(meta, np.uint32)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group", [32, 64, 128, 256])
def test_quantize_ragged_random(fc, orc, bits, group):
    from gpu_helpers import assert_equal_bits
    n = group * 1037  # 1037 groups: several workgroups, last one partial
    xb = dg.synth_bf16((bits, group), n, sigma=1.0, outlier_p=0.01, outlier_factor=40.0)
    c, m = run_quantize(fc, xb, bits, group)
    rc, rm = orc.quantize(xb, bits, group)
    assert_equal_bits(m, rm, f"meta bits={bits} G={group}")
    assert_equal_bits(c, rc, f"codes bits={bits} G={group}")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group", [32, 128, 256])
def test_quantize_edge_groups(fc, orc, bits, group):
    from gpu_helpers import assert_equal_bits
    xb = dg.adversarial_groups(group, seed=bits)
    c, m = run_quantize(fc, xb, bits, group)
    rc, rm = orc.quantize(xb, bits, group)
    assert_equal_bits(m, rm, "meta")
    assert_equal_bits(c, rc, "codes")


@pytest.mark.parametrize("group", [32, 128])
def test_quantize_single_group_and_tiny(fc, orc, group):
    from gpu_helpers import assert_equal_bits
    for ngroups in (1, 2, 3, 7):
        for bits in (4, 8):
            xb = dg.synth_bf16((ngroups, bits, group, 9), group * ngroups, sigma=2.0)
            c, m = run_quantize(fc, xb, bits, group)
            rc, rm = orc.quantize(xb, bits, group)
            assert_equal_bits(m, rm, f"meta n={ngroups}")
            assert_equal_bits(c, rc, f"codes n={ngroups}")


@pytest.mark.parametrize("workload", ["tiny-r2-t4-h256", "llama3-8b-decode"])
def test_quantize_workloads_full(fc, orc, workload):
    """All ranks of the workload quantized in one batched call, compared in full."""
    from gpu_helpers import assert_equal_bits
    cfg = dg.WORKLOADS[workload]
    parts = np.concatenate(dg.partials(cfg))
    c, m = run_quantize(fc, parts, cfg.bits_rs, cfg.group)
    rc, rm = orc.quantize(parts, cfg.bits_rs, cfg.group)
    assert_equal_bits(m, rm, "meta")
    assert_equal_bits(c, rc, "codes")


def test_quantize_70b_prefill_sampled(fc, orc):
    """8 ranks x [4096, 8192] bf16, int4 groups of 128, one batched launch (the benchmark's launch);
    2048 sampled groups plus the first and last group of every rank are recomputed by the oracle."""
    cfg = dg.PREFILL_70B
    from gpu_helpers import assert_equal_bits
    R, n, G, bits = cfg.R, cfg.n, cfg.group, cfg.bits_rs
    parts = [dg.partial(cfg, r) for r in range(R)]
    allp = np.concatenate(parts)
    c, m = run_quantize(fc, allp, bits, G)
    ngroups = R * n // G
    rng = np.random.default_rng(33)
    idx = np.unique(np.concatenate([rng.integers(0, ngroups, 2048), np.arange(R) * (n // G),
                                    np.arange(1, R + 1) * (n // G) - 1]))
    xs = allp.reshape(ngroups, G)[idx].ravel()
    rc, rm = orc.quantize(xs, bits, G)
    assert_equal_bits(m[idx], rm, "meta (sampled)")
    cb = G * bits // 8
    assert_equal_bits(c.reshape(ngroups, cb)[idx].ravel(), rc, "codes (sampled)")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group", [32, 64, 128, 256])
def test_quantize_many_chunks_full(fc, orc, bits, group):
    """Inputs of at least 4096 x 1024 chunks of 8 take the kernel shape with several chunks per lane (2 for
    4-bit codes, 4 for 8-bit), whose per-group step runs in one lane per group and slot and is broadcast
    back to the group's lanes: every group width, with whole groups past the last full tile.  Compared in
    full (33.6 M elements)."""
    from gpu_helpers import assert_equal_bits
    n = 4096 * 1024 * 8 + group * 37
    xb = dg.synth_bf16((bits, group, 77), n, sigma=1.0, outlier_p=0.01, outlier_factor=40.0)
    c, m = run_quantize(fc, xb, bits, group)
    rc, rm = orc.quantize(xb, bits, group)
    assert_equal_bits(m, rm, f"meta bits={bits} G={group}")
    assert_equal_bits(c, rc, f"codes bits={bits} G={group}")
