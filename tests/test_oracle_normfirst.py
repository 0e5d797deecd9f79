"""Pins of the oracle's norm-before-all-gather variant (TokenWeave, abstract: the RMSNorm moved relative to
the communication, applied to each reduce-scattered shard; the normalized rows are then quantized for the
all-gather).

The row's sum of squares uses a fixed order (8-element chunk folds, then a pairwise tree over the chunks)
because the normalized values decide integer codes.  The pins: exact sums on integer data, hand-derived
values where the order changes the result, bit-identity with the standard epilogue whenever every sum
is exact, a closed form for constant rows, and the quantization round trip."""
import numpy as np
import pytest

from tensor_all_reduce_amd import datagen as dg


def _bf16(x):
    """Exact bf16 values of a float array of bf16-representable numbers, as uint16 bits."""
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("H", [8, 24, 1000, 4096, 8192])
def test_sumsq_tree_exact_on_integers(orc, H):
    rng = np.random.default_rng(H)
    h = rng.integers(-16, 17, H).astype(np.float32)   # every partial sum < 2^24: exact in fp32
    assert orc.sumsq_tree(h) == np.float32(np.sum(h.astype(np.int64) ** 2))


def test_sumsq_tree_order():
    """Chunk partials [2^24, 1, 1, 1]: the pairwise tree gives (2^24 + 1) + (1 + 1) = 2^24 + 2, a sequential
    fold would give 2^24.  Inside a chunk the fold is sequential: [4096, 1, 1, 1] gives 2^24 (a tree would
    give 2^24 + 2).  Five chunks [2^24, 1, 1, 1, 1] pad to eight: ((2^24 + 1) + (1 + 1)) + ((1 + 0) + 0)
    = (2^24 + 2) + 1, a tie rounded to even: 2^24 + 4."""
    import oracle as orc
    h = np.zeros(32, np.float32)
    h[[0, 8, 16, 24]] = [4096, 1, 1, 1]
    assert orc.sumsq_tree(h) == np.float32(16777218)
    h = np.zeros(8, np.float32)
    h[:4] = [4096, 1, 1, 1]
    assert orc.sumsq_tree(h) == np.float32(16777216)
    h = np.zeros(40, np.float32)
    h[[0, 8, 16, 24, 32]] = [4096, 1, 1, 1, 1]
    assert orc.sumsq_tree(h) == np.float32(16777220)


def _rn32(x):
    """Round an exact rational to the nearest fp32, ties to even."""
    from fractions import Fraction
    v = np.float32(float(x))
    cands = [np.nextafter(v, np.float32(-np.inf)), v, np.nextafter(v, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - x), int(np.float32(c).view(np.uint32)) & 1))


def test_sumsq_tree_chunk_fold_rounds_each_square(orc):
    """Inside a chunk every square is rounded before it is added (no fused multiply-add): for the chunk
    [1, b, 0, ...] with b = 1 + 3370 * 2^-23, fl(1 + fl(b*b)) and fl(1 + b*b) differ."""
    from fractions import Fraction
    b = np.float32(1.0 + 3370 * 2.0 ** -23)
    unfused = _rn32(Fraction(1) + Fraction(float(_rn32(Fraction(float(b)) ** 2))))
    fused = _rn32(Fraction(1) + Fraction(float(b)) ** 2)
    assert unfused != fused
    h = np.zeros(8, np.float32)
    h[:2] = [1.0, b]
    assert orc.sumsq_tree(h) == unfused


def test_sumsq_tree_close_to_exact_sum(orc):
    rng = np.random.default_rng(7)
    for H in (256, 4096, 8192):
        h = rng.standard_normal(H).astype(np.float32)
        exact = np.sum(h.astype(np.float64) ** 2)
        assert abs(float(orc.sumsq_tree(h)) - exact) <= exact * 2.0 ** -18


@pytest.mark.parametrize("H", [256, 1024, 4096])
def test_norm_matches_standard_epilogue_when_sums_are_exact(orc, H):
    """With integer-valued y and residual every sum of squares is exact in any order, so the fp32
    normalized values rounded to bf16 must equal the standard epilogue's output bit for bit."""
    rng = np.random.default_rng(H + 1)
    rows = 3
    y = rng.integers(-8, 9, rows * H).astype(np.float32)
    res = _bf16(rng.integers(-8, 9, rows * H).astype(np.float32))
    gam = _bf16(rng.integers(1, 5, H).astype(np.float32) * 0.25)
    o, rout = orc.norm_rows_f32(y, res, gam, 1e-5, H)
    out_std, rout_std = orc.rmsnorm(y, res, gam, 1e-5, H)
    assert np.array_equal(orc.f32_to_bf16(o), out_std)
    assert np.array_equal(rout, rout_std)


def test_norm_constant_row_closed_form(orc):
    """h = c on the whole row: sum of squares H*c^2 exactly (c a power of two), o_j = (c / sqrt(c^2 + eps))
    * gamma_j up to three fp32 roundings."""
    H, eps = 4096, 1e-5
    rng = np.random.default_rng(3)
    gam = orc.f32_to_bf16(rng.normal(1.0, 0.1, H).astype(np.float32))
    gf = (gam.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for c in (0.125, 1.0, 4.0, -2.0):
        o, _ = orc.norm_rows_f32(np.full(H, c, np.float32), None, gam, eps, H)
        ref = c / np.sqrt(c * c + np.float64(np.float32(eps))) * gf
        assert np.max(np.abs(o - ref) / np.abs(ref)) <= 4 * 2.0 ** -24


@pytest.mark.parametrize("b1,b2", [(8, 8), (4, 8), (8, 4)])
def test_reduce_norm_quant_round_trip(orc, b1, b2):
    """The shard's sums, residual-add and norm, then quantization: every dequantized value lies within half
    a scale of the normalized value (plus the fp32 slack of the quantizer), and residual_out is
    bf16(sum + residual)."""
    R, H, G, rows = 4, 512, 128, 3
    L = rows * H
    rng = np.random.default_rng(b1 * 10 + b2)
    msgs = [orc.quantize(dg.synth_bf16((r, b1, 5), L, sigma=1.0, outlier_p=0.01, outlier_factor=20.0), b1, G)
            for r in range(R)]
    res = orc.f32_to_bf16(rng.standard_normal(L).astype(np.float32))
    gam = orc.f32_to_bf16(rng.normal(1.0, 0.1, H).astype(np.float32))
    codes, meta, rout, o = orc.reduce_norm_quant([c for c, _ in msgs], [m for _, m in msgs], L, b1, b2, G, res,
                                                 gam, 1e-5, H)
    _, _, S = orc.reduce_shard([c for c, _ in msgs], [m for _, m in msgs], L, b1, b1, G, want_sum=True)
    resf = (res.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(rout, orc.f32_to_bf16(S + resf))
    # the quantizer's input is the fp32 normalized value, not its bf16 rounding
    qc, qm = orc.quantize(o, b2, G)
    assert np.array_equal(codes, qc) and np.array_equal(meta, qm)
    bc, _ = orc.quantize(((orc.f32_to_bf16(o).astype(np.uint32)) << 16).view(np.float32), b2, G)
    assert not np.array_equal(codes, bc)
    d = orc.dequant(codes, meta, L, b2, G).astype(np.float64)
    scale = orc.f16_to_f32((meta & 0xFFFF).astype(np.uint16)).astype(np.float64)
    s_el = np.repeat(scale, G)
    assert np.all(np.abs(d - o) <= s_el / 2 + s_el * ((1 << b2) - 1) * 2.0 ** -22)


def test_two_step_normfirst_close_to_standard_path(orc):
    """Norm first, then an 8-bit quantized all-gather, versus the standard path (all-gather of the sums,
    then the norm): the same rows up to one 8-bit quantization step of the normalized values, and the
    same residual stream up to the quantization of the sums."""
    cfg = dg.TINY
    parts = dg.partials(cfg)
    res, gam = dg.residual(cfg), dg.gamma(cfg)
    nf = orc.two_step_normfirst(parts, cfg.bits_rs, cfg.bits_ag, cfg.group, res, gam, cfg.eps, cfg.H)
    st = orc.two_step(parts, cfg.bits_rs, cfg.bits_ag, cfg.group, residual=res, gamma=gam, eps=cfg.eps,
                      hidden=cfg.H, plain=False)
    f = lambda u: (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    o_nf, o_st = f(nf["y"]).reshape(-1, cfg.group), f(st["out"]).reshape(-1, cfg.group)
    rng_g = o_st.max(axis=1, keepdims=True) - o_st.min(axis=1, keepdims=True)
    assert np.all(np.abs(o_nf - o_st) <= rng_g / 255 * 2 + np.abs(o_st) * 2.0 ** -6)
    assert np.max(np.abs(f(nf["residual_out"]) - f(st["residual_out"]))) < 0.1


# ---- the plain order (the reading the GPU's fixed tree order is compared against) ----------------------
def test_sumsq_seq_is_the_left_fold_of_rounded_squares(orc):
    """Squares [2^24, 1, 1, 1] (placed at any positions): the left fold rounds each +1 back to 2^24 (a tie,
    to even), so the plain order gives 2^24 where the tree gives 2^24 + 2; [1, 1, 1, 2^24] gives 2^24 + 4 in
    the left fold (3 + 2^24 rounds to even, up)."""
    h = np.zeros(32, np.float32)
    h[[0, 8, 16, 24]] = [4096, 1, 1, 1]
    assert orc.sumsq_seq(h) == np.float32(16777216)
    assert orc.sumsq_tree(h) == np.float32(16777218)
    h[[0, 8, 16, 24]] = [1, 1, 1, 4096]
    assert orc.sumsq_seq(h) == np.float32(16777220)


@pytest.mark.parametrize("H", [8, 1000, 8192])
def test_sumsq_seq_exact_on_integers(orc, H):
    rng = np.random.default_rng(H + 5)
    h = rng.integers(-16, 17, H).astype(np.float32)
    assert orc.sumsq_seq(h) == np.float32(np.sum(h.astype(np.int64) ** 2))


def test_sumsq_seq_rounds_each_square(orc):
    """As the tree's chunk fold: fl(1 + fl(b*b)), not a fused fl(1 + b*b)."""
    from fractions import Fraction
    b = np.float32(1.0 + 3370 * 2.0 ** -23)
    unfused = _rn32(Fraction(1) + Fraction(float(_rn32(Fraction(float(b)) ** 2))))
    h = np.zeros(5, np.float32)
    h[[0, 4]] = [1.0, b]
    assert orc.sumsq_seq(h) == unfused


@pytest.mark.parametrize("H", [256, 4096, 8192])
def test_plain_norm_rounds_to_the_standard_epilogue(orc, H):
    """The plain-order normalized rows are the standard epilogue's values before their bf16 rounding: on
    Gaussian rows (sums of squares not exact) bf16(o) equals the epilogue's output bit for bit, and
    residual_out is the same."""
    rng = np.random.default_rng(H + 9)
    rows = 4
    y = (rng.standard_normal(rows * H) * 3).astype(np.float32)
    res = orc.f32_to_bf16(rng.standard_normal(rows * H).astype(np.float32))
    gam = orc.f32_to_bf16(rng.normal(1.0, 0.1, H).astype(np.float32))
    o, rout = orc.norm_rows_f32(y, res, gam, 1e-5, H, order="seq")
    out_std, rout_std = orc.rmsnorm(y, res, gam, 1e-5, H)
    assert np.array_equal(orc.f32_to_bf16(o), out_std)
    assert np.array_equal(rout, rout_std)


def test_plain_and_tree_orders_differ_where_the_sum_does():
    """A row whose squares are [2^24, 1, 1, 1] at chunk starts: the two orders give different sums, hence
    different normalized values; on integer rows with exact sums they agree."""
    import oracle as orc
    H = 32
    y = np.zeros(H, np.float32)
    y[[0, 8, 16, 24]] = [4096, 1, 1, 1]
    gam = orc.f32_to_bf16(np.ones(H, np.float32))
    o_s, _ = orc.norm_rows_f32(y, None, gam, 1e-5, H, order="seq")
    o_t, _ = orc.norm_rows_f32(y, None, gam, 1e-5, H, order="tree")
    assert not np.array_equal(o_s, o_t)
    y = np.arange(H, dtype=np.float32) - 16
    assert np.array_equal(orc.norm_rows_f32(y, None, gam, 1e-5, H, order="seq")[0],
                          orc.norm_rows_f32(y, None, gam, 1e-5, H, order="tree")[0])


def test_two_step_normfirst_orders_share_every_other_step():
    """The whole norm-first path in both orders: identical reduce-scatter messages and residual stream (the
    order only enters the norm), and gathered rows within one 8-bit step of each other."""
    import oracle as orc
    cfg = dg.DECODE_8B
    parts = dg.partials(cfg)
    res, gam = dg.residual(cfg), dg.gamma(cfg)
    a = orc.two_step_normfirst(parts, cfg.bits_rs, cfg.bits_ag, cfg.group, res, gam, cfg.eps, cfg.H, order="seq")
    b = orc.two_step_normfirst(parts, cfg.bits_rs, cfg.bits_ag, cfg.group, res, gam, cfg.eps, cfg.H, order="tree")
    assert np.array_equal(a["codes1"], b["codes1"]) and np.array_equal(a["meta1"], b["meta1"])
    assert np.array_equal(a["residual_out"], b["residual_out"])
    scale = orc.f16_to_f32((a["meta2"] & 0xFFFF).astype(np.uint16)).astype(np.float64)
    f = lambda u: (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    d = np.abs(f(a["y"]) - f(b["y"]))
    assert np.all(d <= np.repeat(scale, cfg.group) * 1.01 + np.abs(f(a["y"])) * 2.0 ** -7)


def test_order_bound_holds_for_the_tree_order(orc):
    """The comparison the GPU test makes (tests/normfirst_bound.py), run with the oracle's tree order in the
    kernels' place (its depth is the one the bound assumes): every decided group is bit-exact against the
    plain order, the rest within the bound, and few groups are undecided."""
    import sys
    import os
    sys.path.insert(0, os.path.dirname(__file__))
    from normfirst_bound import compare
    cfg = dg.DECODE_8B
    parts = dg.partials(cfg)
    res, gam = dg.residual(cfg), dg.gamma(cfg)
    tree = orc.two_step_normfirst(parts, cfg.bits_rs, cfg.bits_ag, cfg.group, res, gam, cfg.eps, cfg.H, order="tree")
    flip, total = compare(orc, cfg, parts, res, gam, tree, log=lambda m: None)
    assert flip < 0.1 * total


def test_order_bound_catches_a_wrong_code(orc):
    """The same comparison rejects a result with one code of a decided group changed."""
    import sys
    import os
    sys.path.insert(0, os.path.dirname(__file__))
    from normfirst_bound import compare
    cfg = dg.DECODE_8B
    parts = dg.partials(cfg)
    res, gam = dg.residual(cfg), dg.gamma(cfg)
    tree = orc.two_step_normfirst(parts, cfg.bits_rs, cfg.bits_ag, cfg.group, res, gam, cfg.eps, cfg.H, order="tree")
    tree["codes2"] = tree["codes2"].copy()
    tree["codes2"][5] ^= 1
    with pytest.raises(AssertionError):
        compare(orc, cfg, parts, res, gam, tree, log=lambda m: None)


@pytest.mark.parametrize("H,G,b2", [(1056, 32, 8), (4096, 256, 4)])
def test_order_bound_holds_on_other_shapes(orc, H, G, b2):
    """The comparison of tests/normfirst_bound.py with the oracle's tree order on shapes whose chunk count is
    not a power of two, and with 4-bit codes out."""
    import sys
    import os
    sys.path.insert(0, os.path.dirname(__file__))
    from normfirst_bound import compare
    cfg = dg.Config(34, f"bound H={H}", "two_step", R=2, T=12, H=H, sigma=0.7, outlier_p=0.02, outlier_factor=30.0,
                    bits_rs=8, bits_ag=b2, group=G)
    parts = dg.partials(cfg)
    res, gam = dg.residual(cfg), dg.gamma(cfg)
    tree = orc.two_step_normfirst(parts, cfg.bits_rs, cfg.bits_ag, cfg.group, res, gam, cfg.eps, cfg.H, order="tree")
    flip, total = compare(orc, cfg, parts, res, gam, tree, log=lambda m: None)
    assert flip < 0.1 * total
