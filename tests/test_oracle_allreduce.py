"""Pins for the oracle's two-step all-reduce (Flash Communication, summary "Core ideas of the solution":
reduce-scatter then all-gather over low-bit messages), its fixed reduction order (flash-comm,
abstract: transport order decoupled from reduction order) and the residual-add + RMSNorm epilogue
(TokenWeave, abstract: fused AllReduce-RMSNorm).

Pins: exact sums where every partial sum is exactly representable, a crafted cancellation that only
the ascending-rank left fold gets right, an end-to-end error bound from the quantization steps, exact
identity at R = 1 on exact grids, closed-form RMSNorm of constant rows, and RMSNorm in double
precision."""
import numpy as np
import pytest

from tensor_all_reduce_amd import datagen as dg


def bf16(x):
    return dg.f32_to_bf16_bits(np.asarray(x, np.float32))


def f32(b):
    return dg.bf16_bits_to_f32(b)


def ulp_dist(a, b):
    """Distance in bf16 units in the last place (sign-magnitude bits mapped to a monotone line)."""
    def ordv(u):
        u = u.astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u & 0x7FFF)
    return np.abs(ordv(np.asarray(a, np.uint16)) - ordv(np.asarray(b, np.uint16)))


def rank_chunks(res, R, L, bits, group, shard):
    c = [res["codes1"][r][shard * L * bits // 8:(shard + 1) * L * bits // 8] for r in range(R)]
    m = [res["meta1"][r][shard * L // group:(shard + 1) * L // group] for r in range(R)]
    return c, m


def grid_partial(rng, n, group, bits, R=1):
    """bf16 values on an exact per-group grid z + k*s with zero-points >= 0 small enough that sums of up
    to 8 ranks stay exact in fp32 and the scales stay fp16-exact when multiplied by R."""
    qmax = (1 << bits) - 1
    x = np.empty(n, np.float32)
    for g in range(n // group):
        s = 2.0 ** int(rng.integers(-4, 1))
        # bf16 has 8 significant bits: an 8-bit grid k*s uses them all, a 4-bit grid leaves room for a
        # small integer offset
        z = 0.0 if bits == 8 else float(rng.integers(0, 8))
        k = rng.integers(0, qmax + 1, size=group)
        k[0], k[-1] = 0, qmax
        x[g * group:(g + 1) * group] = z + k * s
    b = bf16(x)
    assert np.array_equal(f32(b), x)
    return b


# ---------------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("R", [2, 4, 8])
def test_identical_ranks_sum_to_R_times(orc, R):
    """R identical buffers reduce to exactly R times the dequantized value (here every partial sum k*d is
    exact: the grid values have few significant bits)."""
    rng = np.random.default_rng(R)
    group, bits, n = 32, 8, 32 * 16 * R
    p = grid_partial(rng, n, group, bits)
    res = orc.two_step([p] * R, bits, bits, group)
    L = n // R
    for s in range(R):
        c, m = rank_chunks(res, R, L, bits, group, s)
        _, _, S = orc.reduce_shard(c, m, L, bits, bits, group, want_sum=True)
        assert np.array_equal(S.astype(np.float64), R * f32(p[s * L:(s + 1) * L]).astype(np.float64))
    # the requantized grid is the R-scaled grid, so the gathered output is exactly R*x
    assert np.array_equal(f32(res["y"]).astype(np.float64), R * f32(p).astype(np.float64))


def test_fixed_ascending_rank_order(orc):
    """Dequantized values 2^15, -2^15, 2^-10 at one position of ranks 0, 1, 2: the ascending left fold
    gives (2^15 - 2^15) + 2^-10 = 2^-10, whereas summing rank 2 into rank 1 first loses it
    (-2^15 + 2^-10 rounds back to -2^15 in fp32).  Constant groups dequantize exactly."""
    G, L = 32, 32
    vals = [2.0 ** 15, -(2.0 ** 15), 2.0 ** -10]
    cs, ms = [], []
    for v in vals:
        c, m = orc.quantize(bf16(np.full(L, v)), 8, G)
        cs.append(c)
        ms.append(m)
    _, _, S = orc.reduce_shard(cs, ms, L, 8, 8, G, want_sum=True)
    assert np.all(S == np.float32(2.0 ** -10))
    # the order is the rank order, not the argument order reversed
    _, _, S2 = orc.reduce_shard(cs[::-1], ms[::-1], L, 8, 8, G, want_sum=True)
    assert np.all(S2 == np.float32(0.0))


def test_two_step_folds_every_shard_in_ascending_rank_order(orc):
    """The cancellation above at every position of a three-rank two-step run: ranks 0, 1 and 2 hold 2^15,
    -2^15 and 2^-10 everywhere (constant fp16-exact groups dequantize exactly), so every shard's ascending
    fold is exactly 2^-10 and so is every gathered value.  A shard that folded the ranks' chunks in
    another order, or took another rank's chunk, would lose the 2^-10 or double a term."""
    G, R = 32, 3
    n = R * 2 * G
    parts = [bf16(np.full(n, v)) for v in (2.0 ** 15, -(2.0 ** 15), 2.0 ** -10)]
    res = orc.two_step(parts, 8, 8, G)
    assert np.all(f32(res["y"]) == np.float32(2.0 ** -10))


def test_requantization_takes_the_fp32_sums(orc):
    """The all-gather payload is quantized from the fp32 sums themselves, not from their bf16 rounding.
    Two ranks with 8-bit codes, fp16 scale 2^-10 and zero-point 1 dequantize exactly to 1 + q*2^-10, and
    their sums 2 + (q0 + q1)*2^-10 are exact in fp32 but need up to 11 significant bits, more than bf16's
    8.  The requantized message must be the quantizer (pinned on its own) applied to the exact sums,
    computed here in double, and that differs from the quantizer applied to their bf16 rounding."""
    G, L = 128, 512
    rng = np.random.default_rng(77)
    word = int(np.float16(2.0 ** -10).view(np.uint16)) | (int(np.float16(1.0).view(np.uint16)) << 16)
    meta = np.full(L // G, word, np.uint32)
    codes = [rng.integers(0, 256, L).astype(np.uint8) for _ in range(2)]
    exact = (1.0 + codes[0] * 2.0 ** -10) + (1.0 + codes[1] * 2.0 ** -10)
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)
    oc, om = orc.reduce_shard(codes, [meta, meta], L, 8, 8, G)
    wc, wm = orc.quantize(exact.astype(np.float32), 8, G)
    assert np.array_equal(om, wm) and np.array_equal(oc, wc)
    bc, bm = orc.quantize(f32(bf16(exact)), 8, G)
    assert not (np.array_equal(bc, wc) and np.array_equal(bm, wm))


@pytest.mark.parametrize("R", [1, 2])
@pytest.mark.parametrize("bits", [4, 8])
def test_grid_identity_small_R(orc, R, bits):
    """At R = 1 the two-step path returns the input exactly when it lies on an exact grid; at R = 2 with
    identical ranks it returns exactly twice the input."""
    rng = np.random.default_rng(50 + bits)
    group, n = 64, 64 * 8
    p = grid_partial(rng, n, group, bits)
    res = orc.two_step([p] * R, bits, bits, group)
    assert np.array_equal(f32(res["y"]).astype(np.float64), R * f32(p).astype(np.float64))


@pytest.mark.parametrize("workload", ["tiny-r2-t4-h256", "llama3-8b-decode"])
@pytest.mark.parametrize("bits1,bits2", [(8, 8), (4, 8), (4, 4), (8, 4)])
def test_two_step_error_bound(orc, workload, bits1, bits2):
    """End-to-end: |y - sum_r x_r| <= sum_r s_r/2 + s'/2 + fp32 slack, where s_r are the rank-message
    scales of each element's group and s' the requantized scale (half-step bound of each quantization,
    exact sum in double).  A dropped rank, a wrong shard or group index, or a wrong sign breaks it."""
    cfg = dg.WORKLOADS[workload]
    R, n, G = cfg.R, cfg.n, cfg.group
    if cfg is dg.DECODE_8B:
        n = 8 * 4096  # 8 rows keep the test quick
    parts = [dg.partial(cfg, r, n) for r in range(R)]
    res = orc.two_step(parts, bits1, bits2, G)
    exact = np.sum([f32(p).astype(np.float64) for p in parts], axis=0)
    s1 = np.zeros(n)
    for r in range(R):
        s1 += np.repeat((res["meta1"][r] & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64), G)
    s2 = np.repeat((res["meta2"] & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64), G)
    y = f32(res["y"]).astype(np.float64)
    bound = s1 / 2 * (1 + 2**-10) + s2 / 2 * (1 + 2**-10) + (R + 2) * np.abs(exact) * 2**-22 + np.abs(y) * 2**-8
    assert np.all(np.abs(y - exact) <= bound)
    # and it is not vacuous: the error is of the order of the quantization step somewhere
    assert np.max(np.abs(y - exact) / (s1 + s2)) > 0.05


# ---------------------------------------------------------------------------------------------------------
def test_rmsnorm_constant_rows_closed_form(orc):
    """A row with h = c everywhere: out_j = c * gamma_j / sqrt(c^2 + eps), within 1 bf16 ulp of the
    double-precision closed form."""
    H = 512
    rng = np.random.default_rng(3)
    g = bf16(rng.standard_normal(H) * 0.1 + 1)
    for c in [1.0, -2.5, 3e-3, 1e-4, 250.0, 0.0]:
        for eps in [1e-5, 1e-2]:
            y = np.full(H, c, np.float32)
            out, _ = orc.rmsnorm(y, None, g, eps, H)
            ref = np.float64(c) * f32(g).astype(np.float64) / np.sqrt(np.float64(c) ** 2 + np.float64(np.float32(eps)))
            assert np.all(ulp_dist(out, bf16(ref)) <= 1), (c, eps)


def test_rmsnorm_matches_double_and_residual(orc):
    """Residual add then RMSNorm; within 2 bf16 ulp of a double-precision evaluation, residual_out within
    1 ulp of the exactly rounded sum (double rounding through fp32 may differ by one)."""
    rng = np.random.default_rng(4)
    rows, H = 16, 1024
    y = (rng.standard_normal(rows * H) * 3).astype(np.float32)
    res = bf16(rng.standard_normal(rows * H))
    g = bf16(rng.standard_normal(H) * 0.1 + 1)
    eps = 1e-5
    out, rout = orc.rmsnorm(y, res, g, eps, H)
    h = y.astype(np.float64) + f32(res).astype(np.float64)
    hr = h.reshape(rows, H)
    r = 1 / np.sqrt((hr ** 2).mean(axis=1, keepdims=True) + np.float32(eps))
    ref = (hr * r * f32(g).astype(np.float64)).ravel()
    assert np.max(ulp_dist(out, bf16(ref))) <= 2
    assert np.max(ulp_dist(rout, bf16(h))) <= 1
    assert np.mean(rout == bf16(h)) > 0.999
    # without a residual, out is the RMSNorm of y itself
    out2, rout2 = orc.rmsnorm(y, None, g, eps, H)
    assert rout2 is None
    yr = y.astype(np.float64).reshape(rows, H)
    ref2 = (yr / np.sqrt((yr ** 2).mean(axis=1, keepdims=True) + np.float32(eps)) * f32(g)).ravel()
    assert np.max(ulp_dist(out2, bf16(ref2))) <= 2


def test_rmsnorm_eps_dominates_tiny_rows(orc):
    """For |h| << sqrt(eps), out ~= h * gamma / sqrt(eps): eps sits inside the square root."""
    H = 256
    y = np.full(H, 1e-5, np.float32)
    g = bf16(np.ones(H))
    out, _ = orc.rmsnorm(y, None, g, 1e-2, H)
    ref = 1e-5 / np.sqrt(1e-10 + np.float64(np.float32(1e-2)))
    assert np.all(ulp_dist(out, bf16(np.full(H, ref))) <= 1)


@pytest.mark.parametrize("R", [1, 2, 4, 8])
def test_reduce_rmsnorm_identical_partials(orc, R):
    """Unquantized reduce: R identical bf16 partials sum exactly to R*x (bf16 has 8 significant bits, so
    every partial sum is exact in fp32); the norm of R*x + residual matches double within 2 ulp."""
    rng = np.random.default_rng(9 + R)
    rows, H = 4, 2048
    p = bf16(rng.standard_normal(rows * H))
    res = bf16(rng.standard_normal(rows * H))
    g = bf16(rng.standard_normal(H) * 0.1 + 1)
    out, rout, y = orc.reduce_rmsnorm([p] * R, rows, H, res, g, 1e-5, want_y=True)
    assert np.array_equal(f32(y).astype(np.float64), R * f32(p).astype(np.float64))
    h = (R * f32(p).astype(np.float64) + f32(res)).reshape(rows, H)
    ref = (h / np.sqrt((h ** 2).mean(axis=1, keepdims=True) + np.float32(1e-5)) * f32(g)).ravel()
    assert np.max(ulp_dist(out, bf16(ref))) <= 2
    assert np.max(ulp_dist(rout, bf16(h.ravel()))) <= 1


def test_reduce_rmsnorm_generic_sum(orc):
    """Generic partials: the fp32 ascending fold is within R fp32 roundings of the exact sum."""
    cfg = dg.TOKENWEAVE
    rows, H, R = 2, cfg.H, cfg.R
    parts = [dg.partial(cfg, r, rows * H) for r in range(R)]
    res = dg.residual(cfg, rows * H)
    g = dg.gamma(cfg)
    out, rout, y = orc.reduce_rmsnorm(parts, rows, H, res, g, 1e-5, want_y=True)
    exact = np.sum([f32(p).astype(np.float64) for p in parts], axis=0)
    assert np.max(ulp_dist(y, bf16(exact))) <= 1


def test_two_rank_sum_is_one_ieee_add(orc):
    """At R = 2 the fold is a single fp32 addition: the exactly rounded sum of the two dequantized values
    (the double sum of two fp32 values is exact, so one rounding to fp32 gives the IEEE result)."""
    rng = np.random.default_rng(21)
    G, L = 128, 128 * 64
    xs = [bf16(rng.standard_normal(L) * 3) for _ in range(2)]
    cm = [orc.quantize(x, 8, G) for x in xs]
    d = [orc.dequant(c, m, L, 8, G).astype(np.float64) for c, m in cm]
    _, _, S = orc.reduce_shard([c for c, _ in cm], [m for _, m in cm], L, 8, 8, G, want_sum=True)
    assert np.array_equal(S, (d[0] + d[1]).astype(np.float32))


@pytest.mark.parametrize("H", [2, 4, 8, 16])
def test_rmsnorm_small_rows_closed_form(orc, H):
    """Short rows where mean(h^2) is known exactly: rows built from (3, 4) pairs have mean 12.5, so
    out_j = h_j * gamma_j / sqrt(12.5 + eps); checked within 1 ulp of double."""
    y = np.tile(np.array([3.0, -4.0], np.float32), H // 2)
    g = bf16(np.linspace(0.5, 1.5, H))
    out, _ = orc.rmsnorm(y, None, g, 1e-5, H)
    ref = y.astype(np.float64) * f32(g) / np.sqrt(12.5 + np.float64(np.float32(1e-5)))
    assert np.all(ulp_dist(out, bf16(ref)) <= 1)
