"""Pins for the oracle's number-format conversions (fp32 -> fp16 nearest/down/up, fp16 -> fp32,
fp32 -> bf16), against references that share nothing with it: numpy's float16 conversion (a library
routine), a sorted table of every finite fp16 value searched with numpy, and a nearest-neighbour
definition of bf16 rounding evaluated in double precision."""
import numpy as np
import pytest

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _all_f16():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return h, h.view(np.float16).astype(np.float64)


def _probe_values(rng):
    """Every finite fp16 value, its fp32 neighbours, every midpoint between consecutive fp16 values and
    the midpoints' fp32 neighbours, plus random fp32 values over the whole fp16 range and beyond."""
    _, v = _all_f16()
    fin = np.unique(v[np.isfinite(v)])
    mids = (fin[:-1] + fin[1:]) / 2.0
    base = np.concatenate([fin, mids]).astype(np.float32)
    up = np.nextafter(base, np.float32(np.inf))
    dn = np.nextafter(base, np.float32(-np.inf))
    rnd = rng.standard_normal(200_000).astype(np.float32) * np.float32(1000.0)
    tiny = (rng.standard_normal(200_000) * 1e-6).astype(np.float32)
    wide = rng.integers(0, 2**32, size=300_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    wide = wide[np.isfinite(wide)]
    edge = np.array([65504, 65519.996, 65520, 65536, 1e30, -65504, -65520, -1e30, 2**-24, 2**-25, 2**-26,
                     -(2**-25), 5.9604645e-08, 3e-8, 0.0, -0.0], np.float32)
    return np.concatenate([base, up, dn, rnd, tiny, wide, edge])


def test_f16_to_f32_exhaustive(orc):
    h, v = _all_f16()
    got = orc.f16_to_f32(h).astype(np.float64)
    fin = np.isfinite(v)
    assert np.array_equal(got[fin], v[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(v[fin]))
    assert np.all(np.isinf(got[np.isinf(v)])) and np.all(np.isnan(got[np.isnan(v)]))


def test_f32_to_f16_nearest_even_matches_numpy(orc):
    x = _probe_values(np.random.default_rng(1))
    got = orc.f32_to_f16(x, 0)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    nan = orc.f32_to_f16(np.array([np.nan], np.float32), 0)
    assert (nan[0] & 0x7C00) == 0x7C00 and (nan[0] & 0x3FF) != 0


def _directed_ref(x, mode):
    """Largest fp16 <= x (mode 1) or smallest fp16 >= x (mode 2), as a float64 value (+-inf past the
    finite range), from a sorted table of every finite fp16 value."""
    _, v = _all_f16()
    tab = np.unique(v[np.isfinite(v)])  # -65504 .. 65504, one zero
    xd = x.astype(np.float64)
    if mode == 1:
        i = np.searchsorted(tab, xd, side="right") - 1
        out = np.where(i >= 0, tab[np.clip(i, 0, None)], -np.inf)
    else:
        i = np.searchsorted(tab, xd, side="left")
        out = np.where(i < tab.size, tab[np.clip(i, None, tab.size - 1)], np.inf)
    return out


@pytest.mark.parametrize("mode", [1, 2])
def test_f32_to_f16_directed_rounding_table(orc, mode):
    x = _probe_values(np.random.default_rng(2 + mode))
    got = orc.f16_to_f32(orc.f32_to_f16(x, mode)).astype(np.float64)
    ref = _directed_ref(x, mode)
    assert np.array_equal(got, ref), np.nonzero(got != ref)[0][:10]
    # the direction itself
    xd = x.astype(np.float64)
    assert np.all(got <= xd) if mode == 1 else np.all(got >= xd)


def test_f32_to_f16_directed_zero_steps(orc):
    # From a zero the step goes to the smallest subnormal of the right sign.
    x = np.array([1e-30, -1e-30], np.float32)
    assert list(orc.f32_to_f16(x, 1)) == [0x0000, 0x8001]
    assert list(orc.f32_to_f16(x, 2)) == [0x0001, 0x8000]
    # exact zeros keep their sign
    z = np.array([0.0, -0.0], np.float32)
    assert list(orc.f32_to_f16(z, 1)) == [0x0000, 0x8000]
    assert list(orc.f32_to_f16(z, 2)) == [0x0000, 0x8000]


def _bf16_nearest_ref(x):
    """bf16 by definition: the two bf16 neighbours bracketing x (truncation and one step away from zero),
    the nearer one in exact double arithmetic, ties to the even bit pattern."""
    u = x.view(np.uint32).astype(np.uint64)
    t = (u & 0xFFFF0000).astype(np.uint64)
    a = t + 0x10000
    tv = (t.astype(np.uint32)).view(np.float32).astype(np.float64)
    av_bits = a.astype(np.uint32)
    av = np.where((a & 0x7FFFFFFF) >= 0x7F800000, np.copysign(np.inf, tv),
                  av_bits.view(np.float32).astype(np.float64))
    xd = x.astype(np.float64)
    # bf16's largest finite magnitude is (2 - 2^-7) * 2^127; past the halfway point to 2^128 rounds to inf
    dt = np.abs(xd - tv)
    da = np.where(np.isinf(av), np.abs(np.abs(xd) - 2.0**128), np.abs(xd - av))
    even_t = ((t >> 16) & 1) == 0
    pick_a = (da < dt) | ((da == dt) & ~even_t)
    return np.where(pick_a, (a >> 16), (t >> 16)).astype(np.uint16)


def test_f32_to_bf16_nearest_even(orc):
    rng = np.random.default_rng(7)
    x = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # every tie pattern and its neighbours for a spread of exponents
    hi = rng.integers(0, 2**16, size=100_000, dtype=np.uint64).astype(np.uint32) << 16
    ties = np.concatenate([hi | 0x8000, hi | 0x7FFF, hi | 0x8001, hi, hi | 0xFFFF])
    x = np.concatenate([x, ties, np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0xFF7FFFFF, 0x00000001,
                                           0x80008000, 0x00018000], np.uint32)])
    f = x.view(np.float32)
    f = f[np.isfinite(f)]
    got = orc.f32_to_bf16(f)
    ref = _bf16_nearest_ref(f)
    assert np.array_equal(got, ref), np.nonzero(got != ref)[0][:10]
    sp = orc.f32_to_bf16(np.array([np.inf, -np.inf, np.nan], np.float32))
    assert sp[0] == 0x7F80 and sp[1] == 0xFF80 and (sp[2] & 0x7F80) == 0x7F80 and (sp[2] & 0x7F) != 0
