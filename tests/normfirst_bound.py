"""Comparison of a norm-before-all-gather result with the oracle's plain reading of it, up to the order of
the rows' sums of squares (used by the GPU parity test and, with the oracle's tree order standing in for
the kernels, by a CPU test of the comparison itself).

A result that adds the squares in a fixed order in which no square passes through more than
d = 7 + ceil(log2(H/8)) additions (an 8-element chunk fold, then a pairwise tree over the chunks) has a
sum within gamma_d = d*u/(1 - d*u) (u = 2^-24) of the exact sum of the rounded squares; the plain left
fold is known exactly.  Every later step is a monotone fp32 function of the sum (r = 1/sqrt(ss/H + eps))
and, element by element, of r (o = fl(fl(h*r)*gamma)), and the quantizer's zero, scale and codes are
monotone in the group's values.  So quantizing the normalized rows at both ends of the interval of r
decides exactly which groups can come out differently from any sum in that interval:
  * residual_out does not depend on the order: bit-exact;
  * a group whose codes and meta agree at both ends must be bit-exact, and its gathered values with it;
  * in the other groups every gathered value must lie within one requantization step of its group (the
    larger of the two scales) plus the width of its normalized value's interval plus 2 bf16 ulp."""
import math

import numpy as np

U = 2.0 ** -24


def f32(u16):
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32)


def rinv(ss, H, eps):
    """The epilogue's fp32 reciprocal RMS of a sum of squares (numpy float32 ops are IEEE, nearest-even)."""
    ss = np.asarray(ss, np.float32)
    return np.float32(1.0) / np.sqrt(ss / np.float32(H) + np.float32(eps))


def depth(H):
    return 7 + max(0, math.ceil(math.log2(max(1, H // 8))))


def flip_analysis(orc, S, res, gam, eps, H, bits, G):
    """S: the oracle's fp32 shard sums of whole rows (flat); res, gam: bf16 bits.  Returns (fixed, o_lo, o_hi,
    (codes, meta)): fixed[g] = group g's codes and meta are the same for every sum of squares in the
    interval; o_lo, o_hi bound each normalized value; codes, meta: the quantized rows at one end."""
    h = S.astype(np.float32) + (f32(res) if res is not None else np.float32(0))
    rows = h.size // H
    h2 = h.reshape(rows, H)
    sq = (h2 * h2).astype(np.float64)                  # each square rounded to fp32 first, then exact in f64
    exact = sq.sum(axis=1)                             # pairwise in f64: within 2^-40 relative of exact
    gd = depth(H) * U / (1 - depth(H) * U) + 2.0 ** -40
    lo = np.nextafter(np.float32(exact * (1 - gd)), np.float32(-np.inf))
    hi = np.nextafter(np.float32(exact * (1 + gd)), np.float32(np.inf))
    plain = np.array([orc.sumsq_seq(r) for r in h2], np.float32)
    lo, hi = np.minimum(lo, plain), np.maximum(hi, plain)
    g = f32(gam)[None, :]
    oa = ((h2 * rinv(hi, H, eps)[:, None]) * g).ravel()
    ob = ((h2 * rinv(lo, H, eps)[:, None]) * g).ravel()
    o_lo, o_hi = np.minimum(oa, ob), np.maximum(oa, ob)
    ca, ma = orc.quantize(o_lo, bits, G)
    cb, mb = orc.quantize(o_hi, bits, G)
    cpg = G * bits // 8
    fixed = (ma == mb) & np.all(ca.reshape(-1, cpg) == cb.reshape(-1, cpg), axis=1)
    return fixed, o_lo, o_hi, (ca, ma)


def compare(orc, cfg, parts, res, gam, got, log=print):
    """got: dict(codes1, meta1, residual_out, codes2, meta2, y) of a norm-first all-reduce of `parts` (the
    rank messages flat per rank).  Asserts the rules above against the oracle's plain order and returns
    (groups that could flip, groups)."""
    R, H, G, b1, b2, L = cfg.R, cfg.H, cfg.group, cfg.bits_rs, cfg.bits_ag, cfg.L
    ref = orc.two_step_normfirst(parts, b1, b2, G, res, gam, cfg.eps, H, order="seq")
    assert np.array_equal(np.ravel(got["codes1"]), ref["codes1"].ravel()), "rank messages: codes"
    assert np.array_equal(np.ravel(got["meta1"]), ref["meta1"].ravel()), "rank messages: meta"
    assert np.array_equal(got["residual_out"], ref["residual_out"]), "residual_out"
    cpg = G * b2 // 8
    ngroups = nfix = 0
    for s in range(R):
        sl = slice(s * L, (s + 1) * L)
        cin = [ref["codes1"][r][s * L * b1 // 8:(s + 1) * L * b1 // 8] for r in range(R)]
        min_ = [ref["meta1"][r][s * (L // G):(s + 1) * (L // G)] for r in range(R)]
        _, _, S = orc.reduce_shard(cin, min_, L, b1, b1, G, want_sum=True)
        fixed, o_lo, o_hi, (qa, ma) = flip_analysis(orc, S, res[sl], gam, cfg.eps, H, b2, G)
        gs = slice(s * (L // G), (s + 1) * (L // G))
        cs = slice(s * L * b2 // 8, (s + 1) * L * b2 // 8)
        mg, mp = got["meta2"][gs], ref["meta2"][gs]
        cg, cp = got["codes2"][cs].reshape(-1, cpg), ref["codes2"][cs].reshape(-1, cpg)
        # the plain result is the decided value in every decided group
        assert np.array_equal(mp[fixed], ma[fixed]) and np.array_equal(cp[fixed], qa.reshape(-1, cpg)[fixed])
        bad = np.nonzero((mg != mp)[fixed] | np.any(cg != cp, axis=1)[fixed])[0]
        assert bad.size == 0, f"shard {s}: {bad.size} decided groups differ, first {np.nonzero(fixed)[0][bad[:5]]}"
        el = np.repeat(fixed, G)
        yg, yp = got["y"][sl], ref["y"][sl]
        assert np.array_equal(yg[el], yp[el]), f"shard {s}: gathered values of decided groups differ"
        sc = lambda m: orc.f16_to_f32((m & 0xFFFF).astype(np.uint16)).astype(np.float64)
        step = np.repeat(np.maximum(sc(mg), sc(mp)), G)
        a, b = f32(yg).astype(np.float64), f32(yp).astype(np.float64)
        mag = np.maximum(np.abs(a), np.abs(b))
        ulp = np.ldexp(1.0, np.frexp(np.maximum(mag, 2.0 ** -126))[1] - 8)
        tol = step + (o_hi.astype(np.float64) - o_lo.astype(np.float64)) + 2 * ulp
        far = np.nonzero(np.abs(a - b) > tol)[0]
        assert far.size == 0, f"shard {s}: {far.size} gathered values beyond the bound, first {far[:5]}"
        ngroups += fixed.size
        nfix += int(fixed.sum())
        differ = int(np.sum(~(np.all(cg == cp, axis=1) & (mg == mp))))
        log(f"shard {s}: {fixed.size - int(fixed.sum())} of {fixed.size} groups could flip, {differ} differ")
    log(f"{cfg.name}: {ngroups - nfix} of {ngroups} groups could flip ({100.0 * (ngroups - nfix) / ngroups:.2f}%)")
    assert nfix >= 0.9 * ngroups, "the bound leaves too few groups decided for the check to mean anything"
    return ngroups - nfix, ngroups
