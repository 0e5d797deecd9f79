"""GPU parity at the largest sizes the C ABI accepts, on sampled groups, rows and blocks that the oracle
recomputes one by one (they are independent): the quantizer past one launch piece (2^33 elements), the
reduce of a 2^31 - 128 element shard, the gather + epilogue of 2^31 - 8192 elements, the slot receiver
on 2^31 - 128 elements per rank, the unquantized reduce + RMSNorm of 2^31 - 8192 elements, the flag
receiver with 65536-element blocks, the all-gather of 2^31 - 64 words, and the norm before the all-gather
on the largest shard and on shards whose rows together pass 2^31 elements.  These exercise the 32-bit element indexes and the 64-bit byte offsets
at their limits.  Inputs are seeded on the GPU (torch generators; the oracle gets the sampled bytes)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu
KMAX = (1 << 31) - 16  # largest per-rank element count of the reduce, gather and slot calls


@pytest.fixture(scope="module")
def fc():
    from tensor_all_reduce_amd import _lib
    return _lib


@pytest.fixture(autouse=True)
def _free():
    import torch
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _gen(seed):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def _bf16(n, seed):
    import torch
    return torch.randn(n, generator=_gen(seed), device="cuda", dtype=torch.bfloat16).view(torch.int16)


def _meta(ngroups, seed):
    """Valid (scale, zero) words: fp16 scale in [2^-8, 2^-5], fp16 zero in [-2, 2]."""
    import torch
    g = _gen(seed)
    s = (torch.rand(ngroups, generator=g, device="cuda") * (2 ** -5 - 2 ** -8) + 2 ** -8).half()
    z = (torch.rand(ngroups, generator=g, device="cuda") * 4 - 2).half()
    s16 = s.view(torch.int16).to(torch.int64) & 0xFFFF
    z16 = z.view(torch.int16).to(torch.int64) & 0xFFFF
    m = (z16 << 16) | s16
    return (m - (m >= (1 << 31)).to(torch.int64) * (1 << 32)).to(torch.int32)


def _codes(nbytes, seed):
    import torch
    return torch.randint(0, 256, (nbytes,), generator=_gen(seed), device="cuda", dtype=torch.uint8)


def _samples(count, rng, extra=()):
    """Sorted unique indices: the first two, the last two, `extra`, and random ones."""
    idx = {0, 1, count - 2, count - 1, *extra}
    idx |= set(int(i) for i in rng.integers(0, count, 40))
    return sorted(i for i in idx if 0 <= i < count)


def _host(t, lo, hi, dtype):
    return t[lo:hi].cpu().numpy().view(dtype)


@pytest.mark.parametrize("bits", [8, 4])
def test_quantize_past_one_launch_piece(fc, orc, bits):
    import torch
    from gpu_helpers import assert_equal_bits
    G = 128
    n = (1 << 33) + (1 << 20)  # two launch pieces of 2^30 chunks
    x = _bf16(n, 11 + bits)
    codes = torch.empty(n * bits // 8, dtype=torch.uint8, device="cuda")
    meta = torch.empty(n // G, dtype=torch.int32, device="cuda")
    fc.fc_quantize(x, bits, G, codes, meta)
    torch.cuda.synchronize()
    edge = (1 << 33) // G
    for g in _samples(n // G, np.random.default_rng(bits), extra=(edge - 1, edge)):
        xs = _host(x, g * G, (g + 1) * G, np.uint16)
        rc, rm = orc.quantize(xs, bits, G)
        assert_equal_bits(_host(meta, g, g + 1, np.uint32), rm, f"meta of group {g}")
        assert_equal_bits(_host(codes, g * G * bits // 8, (g + 1) * G * bits // 8, np.uint8), rc, f"codes of group {g}")


@pytest.mark.parametrize("b1", [8, 4])
def test_reduce_largest_shard(fc, orc, b1):
    import torch
    from gpu_helpers import assert_equal_bits
    G, R, b2 = 128, 2, 8
    L = KMAX // G * G  # 2^31 - 128
    ins = [(_codes(L * b1 // 8, 20 + r), _meta(L // G, 30 + r)) for r in range(R)]
    out = (torch.empty(L * b2 // 8, dtype=torch.uint8, device="cuda"),
           torch.empty(L // G, dtype=torch.int32, device="cuda"))
    fc.fc_reduce_shard(ins, R, L, b1, b2, G, [out])
    torch.cuda.synchronize()
    for g in _samples(L // G, np.random.default_rng(b1)):
        cs = [_host(c, g * G * b1 // 8, (g + 1) * G * b1 // 8, np.uint8) for c, _ in ins]
        ms = [_host(m, g, g + 1, np.uint32) for _, m in ins]
        rc, rm = orc.reduce_shard(cs, ms, G, b1, b2, G)
        assert_equal_bits(_host(out[1], g, g + 1, np.uint32), rm, f"meta of group {g}")
        assert_equal_bits(_host(out[0], g * G, (g + 1) * G, np.uint8), rc, f"codes of group {g}")


def test_gather_norm_largest(fc, orc):
    import torch
    from gpu_helpers import assert_bf16_close, assert_equal_bits
    G, H, bits = 128, 8192, 8
    L = KMAX // H * H  # 2^31 - 8192, one shard of whole rows
    codes, meta = _codes(L, 40), _meta(L // G, 41)
    res = _bf16(L, 42)
    gam = _bf16(H, 43)
    out = torch.empty(L, dtype=torch.int16, device="cuda")
    rout = torch.empty(L, dtype=torch.int16, device="cuda")
    fc.fc_gather_dequant([(codes, meta)], L, bits, G,
                         norm=dict(residual=res, gamma=gam, eps=1e-5, hidden=H, out=out, residual_out=rout))
    torch.cuda.synchronize()
    gh = gam.cpu().numpy().view(np.uint16)
    for row in _samples(L // H, np.random.default_rng(3)):
        lo, hi = row * H, (row + 1) * H
        _, ro, rr = orc.gather([_host(codes, lo, hi, np.uint8)], [_host(meta, lo // G, hi // G, np.uint32)], H, bits,
                               G, plain=False, residual=_host(res, lo, hi, np.uint16), gamma=gh, eps=1e-5, hidden=H)
        assert_equal_bits(_host(rout, lo, hi, np.uint16), rr, f"residual_out of row {row}")
        assert_bf16_close(_host(out, lo, hi, np.uint16), ro, 2, f"out of row {row}")


def test_slot_receiver_largest(fc, orc):
    import torch
    from gpu_helpers import assert_equal_bits, counters_buf, counts
    R, B, e = 2, 64, 0x5EED
    n = KMAX // (2 * B) * (2 * B)  # 2^31 - 128 elements, 2^30 - 64 slots per rank
    nslots, nblk = n // 2, n // 2 // B
    slots = []
    for r in range(R):
        w = torch.randint(0, 1 << 31, (nslots,), generator=_gen(50 + r), device="cuda", dtype=torch.int64)
        w = w & 0x3F7F3F7F  # bf16 pairs below 2 in magnitude: their sums stay finite
        slots.append(w | (e << 32))
        del w
    late = [nblk - 1, nblk // 2, 3]
    for b in late:  # rank 1's copies of a few blocks carry the previous epoch, one of them only in its last slot
        if b == nblk // 2:
            slots[1][b * B + B - 1] = (slots[1][b * B + B - 1] & 0xFFFFFFFF) | ((e - 1) << 32)
        else:
            slots[1][b * B:(b + 1) * B] = (slots[1][b * B:(b + 1) * B] & 0xFFFFFFFF) | ((e - 1) << 32)
    out = torch.zeros(n, dtype=torch.int16, device="cuda")
    stale = torch.zeros(R * nblk, dtype=torch.uint8, device="cuda")
    done = torch.zeros(nblk, dtype=torch.uint8, device="cuda")
    cnt = counters_buf()
    fc.fc_ll_unpack_reduce(slots, n, B, e, out, stale, done, cnt)
    torch.cuda.synchronize()
    assert list(counts(cnt)) == [len(late), len(late)]
    for b in _samples(nblk, np.random.default_rng(4), extra=late):
        ss = [_host(s, b * B, (b + 1) * B, np.uint64) for s in slots]
        ro, rst, rdn, _ = orc.ll_unpack_reduce(ss, 2 * B, B, e)
        assert_equal_bits(_host(done, b, b + 1, np.uint8), rdn, f"done of block {b}")
        assert_equal_bits(np.array([_host(stale, r * nblk + b, r * nblk + b + 1, np.uint8)[0] for r in range(R)]),
                          rst[:, 0], f"stale flags of block {b}")
        got = _host(out, 2 * B * b, 2 * B * (b + 1), np.uint16)
        assert_equal_bits(got, ro if rdn[0] else np.zeros(2 * B, np.uint16), f"out of block {b}")


def test_reduce_rmsnorm_largest(fc, orc):
    import torch
    from gpu_helpers import assert_bf16_close, assert_equal_bits
    R, H = 2, 8192
    rows = KMAX // H
    n = rows * H
    parts = [_bf16(n, 60 + r) for r in range(R)]
    res, gam = _bf16(n, 62), _bf16(H, 63)
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    rout = torch.empty(n, dtype=torch.int16, device="cuda")
    fc.fc_reduce_rmsnorm(parts, rows, dict(residual=res, gamma=gam, eps=1e-5, hidden=H, out=out, residual_out=rout))
    torch.cuda.synchronize()
    gh = gam.cpu().numpy().view(np.uint16)
    for row in _samples(rows, np.random.default_rng(6)):
        lo, hi = row * H, (row + 1) * H
        ro, rr, _ = orc.reduce_rmsnorm([_host(p, lo, hi, np.uint16) for p in parts], 1, H,
                                       _host(res, lo, hi, np.uint16), gh, 1e-5)
        assert_equal_bits(_host(rout, lo, hi, np.uint16), rr, f"residual_out of row {row}")
        assert_bf16_close(_host(out, lo, hi, np.uint16), ro, 2, f"out of row {row}")


def test_flag_receiver_largest(fc, orc):
    import torch
    from gpu_helpers import assert_equal_bits, counters_buf, counts
    R, be, e = 2, 65536, 0xF1A6
    n = KMAX // be * be
    nblk = n // be
    pays = [_bf16(n, 70 + r) for r in range(R)]
    fls = [torch.full((nblk,), e, dtype=torch.int32, device="cuda") for _ in range(R)]
    late = [nblk - 1, 0]
    for b in late:
        fls[1][b] = e - 1
    out = torch.zeros(n, dtype=torch.int16, device="cuda")
    stale = torch.zeros(R * nblk, dtype=torch.uint8, device="cuda")
    done = torch.zeros(nblk, dtype=torch.uint8, device="cuda")
    cnt = counters_buf()
    fc.fc_flag_unpack_reduce(pays, fls, n, be, e, out, stale, done, cnt)
    torch.cuda.synchronize()
    assert list(counts(cnt, 4)) == [len(late), len(late), 0, 0]
    for b in _samples(nblk, np.random.default_rng(7), extra=late):
        lo, hi = b * be, (b + 1) * be
        ro, rst, rdn, _ = orc.flag_unpack_reduce([_host(p, lo, hi, np.uint16) for p in pays],
                                                 [_host(f, b, b + 1, np.uint32) for f in fls], be, be, e)
        assert_equal_bits(_host(done, b, b + 1, np.uint8), rdn, f"done of block {b}")
        assert_equal_bits(np.array([_host(stale, r * nblk + b, r * nblk + b + 1, np.uint8)[0] for r in range(R)]),
                          rst, f"stale flags of block {b}")
        assert_equal_bits(_host(out, lo, hi, np.uint16), ro if rdn[0] else np.zeros(be, np.uint16), f"out of block {b}")


def test_allgather_largest(fc, orc):
    import torch
    from gpu_helpers import assert_equal_bits, counters_buf, counts
    R, B, e = 1, 64, 0x6A7
    nwords = KMAX // B * B
    nblk = nwords // B
    w = torch.randint(0, 1 << 31, (nwords,), generator=_gen(80), device="cuda", dtype=torch.int64)
    slots = [w | (e << 32)]
    del w
    late = [nblk - 1, 5]
    for b in late:
        slots[0][b * B] = (slots[0][b * B] & 0xFFFFFFFF) | ((e + 1) << 32)
    out = [torch.zeros(nwords, dtype=torch.int32, device="cuda")]
    stale = torch.zeros(R * nblk, dtype=torch.uint8, device="cuda")
    done = torch.zeros(R * nblk, dtype=torch.uint8, device="cuda")
    cnt = counters_buf()
    fc.fc_ll_gather(slots, nwords, B, e, out, stale, done, cnt)
    torch.cuda.synchronize()
    assert list(counts(cnt)) == [len(late), len(late)]
    for b in _samples(nblk, np.random.default_rng(8), extra=late):
        ro, rst, rdn, _ = orc.ll_gather([_host(slots[0], b * B, (b + 1) * B, np.uint64)], B, B, e)
        assert_equal_bits(_host(done, b, b + 1, np.uint8), rdn, f"done of block {b}")
        assert_equal_bits(_host(stale, b, b + 1, np.uint8), rst, f"stale of block {b}")
        assert_equal_bits(_host(out[0], b * B, (b + 1) * B, np.uint32), ro[0], f"words of block {b}")


@pytest.mark.parametrize("n_shards,L", [(1, KMAX // 8192 * 8192), (3, (1 << 30) - 8192)])
def test_reduce_norm_first_largest(fc, orc, n_shards, L):
    """The norm before the all-gather at the largest shard, and 3 shards whose rows together pass 2^31
    elements (the launcher splits them into launches below that)."""
    import torch
    from gpu_helpers import assert_equal_bits
    R, H, G, b1, b2 = 2, 8192, 128, 8, 8
    ins = [(_codes(L, 90 + 10 * s + r), _meta(L // G, 95 + 10 * s + r)) for s in range(n_shards) for r in range(R)]
    res, gam = _bf16(n_shards * L, 99), _bf16(H, 98)
    rout = torch.empty(n_shards * L, dtype=torch.int16, device="cuda")
    outs = [(torch.empty(L, dtype=torch.uint8, device="cuda"), torch.empty(L // G, dtype=torch.int32, device="cuda"))
            for _ in range(n_shards)]
    fc.fc_reduce_shard_norm(ins, R, L, b1, b2, G, dict(residual=res, gamma=gam, eps=1e-5, hidden=H, residual_out=rout),
                            outs)
    torch.cuda.synchronize()
    gh = gam.cpu().numpy().view(np.uint16)
    for s in range(n_shards):
        for row in _samples(L // H, np.random.default_rng(10 + s)):
            lo, hi = row * H, (row + 1) * H
            cs = [_host(ins[s * R + r][0], lo, hi, np.uint8) for r in range(R)]
            ms = [_host(ins[s * R + r][1], lo // G, hi // G, np.uint32) for r in range(R)]
            oc, om, rr, _ = orc.reduce_norm_quant(cs, ms, H, b1, b2, G, _host(res, s * L + lo, s * L + hi, np.uint16),
                                                   gh, 1e-5, H, order="tree")
            assert_equal_bits(_host(outs[s][1], lo // G, hi // G, np.uint32), om, f"meta, shard {s} row {row}")
            assert_equal_bits(_host(outs[s][0], lo, hi, np.uint8), oc, f"codes, shard {s} row {row}")
            assert_equal_bits(_host(rout, s * L + lo, s * L + hi, np.uint16), rr, f"residual_out, shard {s} row {row}")
