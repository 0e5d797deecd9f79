"""Pins for the oracle's group quantizer and dequantizer (Flash Communication, abstract and summary
"Core ideas of the solution": low-bit fine-grained quantization of activations).

The pages print no worked example, so the pins come from mathematics: hand-derived cases in
``golden/quant_cases.json``, brute force over every code in exact (double / rational) arithmetic, the
defining properties of the fp16 zero-point and scale checked against a table of all fp16 values, and
the invariants a correct asymmetric quantizer must satisfy (round-trip error at most half a step, one
code for a constant group, exact codes on an exact grid, monotone codes)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from tensor_all_reduce_amd import datagen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_cases.json")

F16_TAB = None


def f16_table():
    global F16_TAB
    if F16_TAB is None:
        v = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
        F16_TAB = np.unique(v[np.isfinite(v)])
    return F16_TAB


def f16v(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def bf16_exact(vals):
    f = np.asarray(vals, np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(datagen.bf16_bits_to_f32(b), f), "golden value not exact in bf16"
    return b


def unpack_codes(codes, n, bits):
    """Independent reading of the documented code layout: int8 byte i = code i; int4 byte i = code 2i
    (low nibble) | code 2i+1 (high nibble)."""
    c = np.asarray(codes, np.uint8)
    if bits == 8:
        return c[:n].astype(np.int64)
    out = np.empty(n, np.int64)
    out[0::2] = c & 0x0F
    out[1::2] = c >> 4
    return out


# ---------------------------------------------------------------------------------------------------------
def test_golden_cases(orc):
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        G, bits = c["group"], c["bits"]
        x = list(c["x"]) + [c.get("rest", 0.0)] * (G - len(c["x"]))
        xb = bf16_exact(x)
        codes, meta = orc.quantize(xb, bits, G)
        assert meta[0] == int(c["meta"], 16), (c["name"], hex(meta[0]))
        want = list(c["codes"]) + [c.get("rest_code", 0)] * (G - len(c["codes"]))
        assert list(unpack_codes(codes, G, bits)) == want, c["name"]
    # explicit byte layouts written in the fixtures
    c0 = cases[0]
    codes, _ = orc.quantize(bf16_exact(c0["x"]), 4, 32)
    assert list(codes[:8]) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    c5 = next(c for c in cases if c["name"] == "int4 ties to even")
    x = list(c5["x"]) + [0.0] * (32 - len(c5["x"]))
    codes, _ = orc.quantize(bf16_exact(x), 4, 32)
    assert list(codes[:3]) == [0xF0, 0x20, 0xE2]


# ---------------------------------------------------------------------------------------------------------
def _groups(rng, G, ngroups, kind):
    if kind == "normal":
        x = rng.standard_normal(G * ngroups)
    elif kind == "outlier":
        x = rng.standard_normal(G * ngroups)
        x[rng.random(x.size) < 0.03] *= 40
    elif kind == "positive":
        x = np.abs(rng.standard_normal(G * ngroups)) * 3 + 0.5
    elif kind == "tiny":  # fp16 subnormal range: zero-points are not fp16-exact here
        x = rng.standard_normal(G * ngroups) * 3e-6
    elif kind == "huge":
        x = rng.standard_normal(G * ngroups) * 8000
    elif kind == "fp32sum":  # fp32 sums (the requantization input): min not fp16-exact in general
        x = (rng.standard_normal(G * ngroups) * 7.3).astype(np.float32).astype(np.float64)
    return x


KINDS = ["normal", "outlier", "positive", "tiny", "huge", "fp32sum"]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("G", [32, 128])
@pytest.mark.parametrize("kind", KINDS)
def test_meta_and_codes_brute_force(orc, bits, G, kind):
    """zero = the largest fp16 <= min; scale = the smallest fp16 that covers the range in qmax steps (up to
    the rounding of one fp32 division); each code = the exactly nearest grid point, ties to even."""
    rng = np.random.default_rng([bits, G, KINDS.index(kind)])
    ngroups = 64
    qmax = (1 << bits) - 1
    xv = _groups(rng, G, ngroups, kind)
    if kind == "fp32sum":
        x = xv.astype(np.float32)
        codes, meta = orc.quantize(x, bits, G)
        xd = x.astype(np.float64)
    else:
        xb = datagen.f32_to_bf16_bits(xv.astype(np.float32))
        codes, meta = orc.quantize(xb, bits, G)
        xd = datagen.bf16_bits_to_f32(xb).astype(np.float64)
    q = unpack_codes(codes, xd.size, bits).reshape(ngroups, G)
    xd = xd.reshape(ngroups, G)
    s = f16v((meta & 0xFFFF).astype(np.uint16))
    z = f16v((meta >> 16).astype(np.uint16))
    tab = f16_table()
    for g in range(ngroups):
        lo, hi = xd[g].min(), xd[g].max()
        # zero-point: largest fp16 <= lo
        assert z[g] <= lo
        i = np.searchsorted(tab, z[g])
        assert tab[i] == z[g] and (i + 1 == tab.size or tab[i + 1] > lo)
        rng_g = hi - z[g]
        if rng_g == 0:
            assert s[g] == 0 and np.all(q[g] == 0)
            continue
        # scale: covers the range (up to one fp32 rounding of range/qmax) and is minimal
        assert s[g] > 0
        assert s[g] * qmax >= rng_g * (1 - 2**-23)
        j = np.searchsorted(tab, s[g])
        prev = tab[j - 1]
        assert prev <= 0 or prev * qmax < rng_g * (1 + 2**-23)
        # codes: exact nearest grid point; near-ties may go either way by fp32 rounding of (x-z)*(1/s)
        for k in range(G):
            u = Fraction(float(xd[g, k])) - Fraction(float(z[g]))
            u = u / Fraction(float(s[g]))
            fl = u.numerator // u.denominator
            frac = u - fl
            if abs(frac - Fraction(1, 2)) > Fraction(1, 2**18) * max(1, fl + 1):
                want = fl + (1 if frac > Fraction(1, 2) else 0)
                want = min(max(want, 0), qmax)
                assert q[g, k] == want, (g, k, float(u))
            else:
                assert q[g, k] in (fl, fl + 1)
                # An exact tie is an fp32 tie only when 1/s is exact (s a power of two) and x - z is
                # exact in fp32; then the code must be the even neighbour.
                sg = float(s[g])
                pow2 = sg == 2.0 ** np.floor(np.log2(sg))
                d32 = np.float32(xd[g, k]) - np.float32(z[g])
                exact_d = Fraction(float(d32)) == Fraction(float(xd[g, k])) - Fraction(float(z[g]))
                if frac == Fraction(1, 2) and pow2 and exact_d:
                    assert q[g, k] % 2 == 0


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("kind", KINDS)
def test_round_trip_bound_and_monotone(orc, bits, kind):
    """|x - dequant(code)| <= scale/2 (+ the fp32 slack of the code computation), and codes never decrease
    as x increases within a group; hi -> qmax when the scale is a normal fp16; lo -> 0 when lo is an fp16."""
    rng = np.random.default_rng(100 + bits + 7 * KINDS.index(kind))
    G, ngroups = 128, 256
    qmax = (1 << bits) - 1
    xv = _groups(rng, G, ngroups, kind)
    if kind == "fp32sum":
        x = xv.astype(np.float32)
        xd = x.astype(np.float64)
    else:
        x = datagen.f32_to_bf16_bits(xv.astype(np.float32))
        xd = datagen.bf16_bits_to_f32(x).astype(np.float64)
    codes, meta = orc.quantize(x, bits, G)
    y = orc.dequant(codes, meta, xd.size, bits, G).astype(np.float64)
    s = np.repeat(f16v((meta & 0xFFFF).astype(np.uint16)), G)
    z = np.repeat(f16v((meta >> 16).astype(np.uint16)), G)
    err = np.abs(xd - y)
    bound = s / 2 + s * qmax * 2.0**-22 + np.abs(y) * 2.0**-24
    assert np.all(err <= bound), float(np.max(err / np.maximum(bound, 1e-300)))
    q = unpack_codes(codes, xd.size, bits).reshape(ngroups, G)
    xg = xd.reshape(ngroups, G)
    for g in range(ngroups):
        o = np.argsort(xg[g], kind="stable")
        assert np.all(np.diff(q[g][o]) >= 0)
        sg, zg = s[g * G], z[g * G]
        lo, hi = xg[g].min(), xg[g].max()
        if sg >= 2.0**-14:
            assert q[g][np.argmax(xg[g])] == qmax
        if zg == lo:
            assert q[g][np.argmin(xg[g])] == 0


def test_constant_group_single_code(orc):
    """A constant group maps to a single code; for an fp16-exact value the scale is 0, the code 0 and the
    dequantized value the input itself."""
    vals = [1.0, -3.25, 1e-3, 65280.0, -65280.0, 2.0**-14, 0.0, 123.0]
    for v in vals:
        xb = datagen.f32_to_bf16_bits(np.full(64, v, np.float32))
        vb = float(datagen.bf16_bits_to_f32(xb[:1])[0])
        for bits in (4, 8):
            codes, meta = orc.quantize(xb, bits, 64)
            q = unpack_codes(codes, 64, bits)
            assert np.all(q == q[0])
            y = orc.dequant(codes, meta, 64, bits, 64)
            if float(np.float16(vb)) == vb:
                assert (meta[0] & 0xFFFF) == 0 and q[0] == 0 and np.all(y == np.float32(vb))
    # fp32 constants that are not fp16 values (requantization of sums): still one code
    for v in [0.1, -7.77, 3.3e-6, 1234.5678]:
        x = np.full(32, v, np.float32)
        for bits in (4, 8):
            codes, meta = orc.quantize(x, bits, 32)
            q = unpack_codes(codes, 32, bits)
            assert np.all(q == q[0])
            y = orc.dequant(codes, meta, 32, bits, 32).astype(np.float64)
            s = float(f16v(np.uint16(meta[0] & 0xFFFF)))
            assert np.all(np.abs(y - np.float64(np.float32(v))) <= s / 2 + abs(v) * 2**-23)


@pytest.mark.parametrize("bits", [4, 8])
def test_exact_grid_gives_exact_codes(orc, bits):
    """Values z + k*s on an exactly representable grid (fp16 s and z) quantize to codes k and dequantize
    to themselves."""
    rng = np.random.default_rng(11 + bits)
    qmax = (1 << bits) - 1
    G = 64
    for trial in range(200):
        s = float(np.float16(2.0 ** rng.integers(-8, 2) * (1 + rng.integers(0, 1024) / 1024)))
        z = float(np.float16(rng.integers(-64, 64) * 0.25))
        k = rng.integers(0, qmax + 1, size=G)
        k[0], k[1] = 0, qmax
        x = (z + k * s).astype(np.float32)
        assert np.array_equal(x.astype(np.float64), z + k * s)  # grid exact in fp32
        codes, meta = orc.quantize(x, bits, G)
        assert np.array_equal(unpack_codes(codes, G, bits), k)
        assert f16v(np.uint16(meta[0] >> 16)) == z and f16v(np.uint16(meta[0] & 0xFFFF)) == s
        y = orc.dequant(codes, meta, G, bits, G)
        assert np.array_equal(y, x)


def test_dequant_is_single_rounding_exhaustive(orc):
    """dequant(q) = fl(q*scale + zero) with one rounding (q*scale is exact in fp32), for every code
    0..255 and every positive finite fp16 scale, at several zero-points; reference in exact double."""
    h = np.arange(1, 0x7C00, dtype=np.uint32).astype(np.uint16)  # all positive finite fp16 scales
    q = np.arange(256, dtype=np.uint8)
    codes = np.tile(q, h.size)
    for zbits in (0x0000, 0xC248, 0x3555, 0x8001, 0x7BFF, 0xFBFF):
        meta = (h.astype(np.uint32) | (np.uint32(zbits) << 16)).astype(np.uint32)
        y = orc.dequant(codes, meta, codes.size, 8, 256)
        sd = np.repeat(f16v(h), 256)
        zd = float(f16v(np.uint16(zbits)))
        ref = (np.tile(q.astype(np.float64), h.size) * sd + zd).astype(np.float32)
        ok = np.isfinite(ref)
        assert np.array_equal(y[ok], ref[ok])


def test_int4_and_int8_agree_on_shared_grid(orc):
    """The same 16-level grid quantized at 4 and at 8 bits: the 4-bit codes are the 8-bit codes / 17
    (scale_8 = scale_4 / 17 exactly when scale_4 is a multiple of 17 quanta)."""
    G = 32
    s4 = 17.0 / 16.0  # fp16-exact, and s4/17 = 1/16 is fp16-exact
    k = np.arange(G) % 16
    x = (k * s4).astype(np.float32)
    c4, m4 = orc.quantize(x, 4, G)
    c8, m8 = orc.quantize(x, 8, G)
    assert np.array_equal(unpack_codes(c4, G, 4), k)
    assert np.array_equal(unpack_codes(c8, G, 8), k * 17)
