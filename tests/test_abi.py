"""CPU tests of the C ABI boundary: libfc.so loads, exports every function include/fc.h declares, shares
PyTorch's HIP runtime, and rejects invalid arguments on the host before any HIP call (so these run
without a GPU; the device addresses used here are never dereferenced)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fc.h")

A = 1 << 20  # a fake, 16-byte aligned "device address" base; never dereferenced by validation


@pytest.fixture(scope="module")
def L():
    from tensor_all_reduce_amd import _lib
    return _lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fc_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert {"fc_quantize", "fc_reduce_shard", "fc_reduce_shard_norm", "fc_gather_dequant", "fc_reduce_rmsnorm",
            "fc_ll_unpack_reduce", "fc_ll_poll_unpack_reduce", "fc_flag_unpack_reduce", "fc_flag_pack",
            "fc_ll_pack", "fc_copy", "fc_bandwidth_probe", "fc_status_string", "fc_last_hip_error", "fc_abi_version"} <= set(names)
    for n in names:
        assert hasattr(L.lib, n), n
    assert L.fc_abi_version() == 5


def test_counter_layout_matches_the_header(L):
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define (FC_COUNTER_\w+) (\d+)", text))
    assert int(defs["FC_COUNTER_GROUPS"]) == L.COUNTER_GROUPS and int(defs["FC_COUNTER_STRIDE"]) == L.COUNTER_STRIDE
    assert L.COUNTER_WORDS == L.COUNTER_GROUPS * L.COUNTER_STRIDE and L.COUNTER_BYTES == 4 * L.COUNTER_WORDS
    # groups 512 bytes apart, so that each 64-bit count pair sits on its own cache lines
    assert 4 * L.COUNTER_STRIDE == 512


def test_single_hip_runtime(L):
    assert len(L._hip_runtimes_mapped()) <= 1


def test_status_strings(L):
    for s in range(6):
        assert L.lib.fc_status_string(s).startswith(b"FC_")


def q(codes, meta):
    from tensor_all_reduce_amd._lib import QMsg
    return QMsg(codes, meta)


def test_quantize_validation(L):
    f = L.lib.fc_quantize
    ok = q(A + 0x100000, A + 0x200000)
    assert f(A, 1024, 5, 32, ok, None) == L.FC_E_ARG          # bits
    assert f(A, 1024, 8, 48, ok, None) == L.FC_E_ARG          # group
    assert f(A, -32, 8, 32, ok, None) == L.FC_E_ARG
    assert f(A, 1000, 8, 32, ok, None) == L.FC_E_SHAPE        # ragged group
    assert f(A, 0, 8, 32, ok, None) == L.FC_OK                # empty: nothing to do, no launch
    assert f(None, 1024, 8, 32, ok, None) == L.FC_E_NULL
    assert f(A, 1024, 8, 32, q(None, A), None) == L.FC_E_NULL
    assert f(A + 2, 1024, 8, 32, ok, None) == L.FC_E_ALIGN
    assert f(A, 1024, 8, 32, q(A + 0x100008, A + 0x200000), None) == L.FC_E_ALIGN
    assert f(A, 1024, 8, 32, q(A + 0x100000, A + 0x200002), None) == L.FC_E_ALIGN
    assert f(A, 1024, 8, 32, q(A + 1024, A + 0x200000), None) == L.FC_E_ARG   # codes overlap x
    assert f(A, 1024, 8, 32, q(A + 0x100000, A + 0x100000 + 512), None) == L.FC_E_ARG  # meta overlaps codes


def test_reduce_shard_validation(L):
    f = L.lib.fc_reduce_shard
    QA = L.QMsg * 4
    ins = QA(*[q(A + 0x10000 * i, A + 0x400000 + 0x1000 * i) for i in range(4)])
    outs = (L.QMsg * 2)(q(A + 0x800000, A + 0x900000), q(A + 0x810000, A + 0x910000))
    assert f(ins, 0, 1024, 2, 8, 8, 32, outs, None) == L.FC_E_ARG
    assert f(ins, 17, 1024, 2, 8, 8, 32, outs, None) == L.FC_E_ARG
    assert f(ins, 2, 1024, 2, 3, 8, 32, outs, None) == L.FC_E_ARG
    assert f(ins, 2, 1024, 2, 8, 8, 100, outs, None) == L.FC_E_ARG
    assert f(ins, 2, 1000, 2, 8, 8, 32, outs, None) == L.FC_E_SHAPE
    assert f(ins, 2, 0, 2, 8, 8, 32, outs, None) == L.FC_OK
    assert f(None, 2, 1024, 2, 8, 8, 32, outs, None) == L.FC_E_NULL
    bad = QA(*[q(A + 0x10000 * i + (8 if i == 3 else 0), A + 0x400000 + 0x1000 * i) for i in range(4)])
    assert f(bad, 2, 1024, 2, 8, 8, 32, outs, None) == L.FC_E_ALIGN
    alias = (L.QMsg * 2)(q(A + 0x10000, A + 0x900000), q(A + 0x810000, A + 0x910000))  # output = an input
    assert f(ins, 2, 1024, 2, 8, 8, 32, alias, None) == L.FC_E_ARG
    twin = (L.QMsg * 2)(q(A + 0x800000, A + 0x900000), q(A + 0x800000, A + 0x910000))  # two shards, one buffer
    assert f(ins, 2, 1024, 2, 8, 8, 32, twin, None) == L.FC_E_ARG


def test_reduce_shard_norm_validation(L):
    """The reduce with the norm first: the reduce's checks, whole rows per shard, groups inside rows, no bf16
    out, and no output overlapping an input or another output."""
    f = L.lib.fc_reduce_shard_norm
    QA = L.QMsg * 4
    ins = QA(*[q(A + 0x10000 * i, A + 0x400000 + 0x1000 * i) for i in range(4)])
    outs = (L.QMsg * 2)(q(A + 0x800000, A + 0x900000), q(A + 0x810000, A + 0x910000))

    def nm(**kw):
        d = dict(residual=A + 0xA00000, gamma=A + 0xB00000, eps=1e-5, hidden=256, out=None, residual_out=A + 0xC00000)
        d.update(kw)
        return L.Norm(d["residual"], d["gamma"], d["eps"], d["hidden"], d["out"], d["residual_out"])
    g = lambda R=2, Lx=1024, b1=8, b2=8, G=32, n=None, o=outs, i=ins: f(i, R, Lx, 2, b1, b2, G,
                                                                         C.byref(n if n is not None else nm()), o, None)
    assert g(R=17) == L.FC_E_ARG
    assert g(b2=5) == L.FC_E_ARG
    assert f(ins, 2, 1024, 2, 8, 8, 32, None, outs, None) == L.FC_E_NULL
    assert g(n=nm(gamma=None)) == L.FC_E_NULL
    assert g(n=nm(out=A + 0xD00000)) == L.FC_E_ARG          # the normalized rows go to the messages only
    assert g(n=nm(eps=0.0)) == L.FC_E_ARG
    assert g(n=nm(hidden=100)) == L.FC_E_SHAPE                # not a multiple of 8
    assert g(n=nm(hidden=384)) == L.FC_E_SHAPE                # 1024 is not whole rows of 384
    assert g(G=256, n=nm(hidden=128)) == L.FC_E_SHAPE         # a group would straddle rows
    assert g(Lx=0) == L.FC_OK
    assert g(n=nm(gamma=A + 0xB00008)) == L.FC_E_ALIGN
    assert g(n=nm(residual_out=A + 0x10000)) == L.FC_E_ARG   # residual_out over an input message
    assert g(n=nm(residual_out=A + 0x800000)) == L.FC_E_ARG  # residual_out over an output message
    alias = (L.QMsg * 2)(q(A + 0x10000, A + 0x900000), q(A + 0x810000, A + 0x910000))
    assert g(o=alias) == L.FC_E_ARG
    over_res = (L.QMsg * 2)(q(A + 0xA00000, A + 0x900000), q(A + 0x810000, A + 0x910000))
    assert g(o=over_res) == L.FC_E_ARG                        # an output over the residual rows


def norm(L, **kw):
    d = dict(residual=A + 0x100000, gamma=A + 0x200000, eps=1e-5, hidden=256, out=A + 0x300000,
             residual_out=A + 0x400000)
    d.update(kw)
    return L.Norm(d["residual"], d["gamma"], d["eps"], d["hidden"], d["out"], d["residual_out"])


def test_gather_validation(L):
    f = L.lib.fc_gather_dequant
    sh = (L.QMsg * 2)(q(A + 0x800000, A + 0x900000), q(A + 0x810000, A + 0x910000))
    assert f(sh, 2, 512, 8, 32, None, None, None) == L.FC_E_NULL          # neither output
    assert f(sh, 2, 500, 8, 32, A, None, None) == L.FC_E_SHAPE
    assert f(sh, 2, 512, 8, 32, A + 8, None, None) == L.FC_E_ALIGN
    assert f(sh, 2, 512, 8, 32, A + 0x800000 - 64, None, None) == L.FC_E_ARG  # y overlaps shard codes
    n = norm(L, hidden=100)
    assert f(sh, 2, 512, 8, 32, None, C.byref(n), None) == L.FC_E_SHAPE   # hidden % 8
    n = norm(L, hidden=96)
    assert f(sh, 2, 512, 8, 32, None, C.byref(n), None) == L.FC_E_SHAPE   # n % hidden
    n = norm(L, eps=0.0)
    assert f(sh, 2, 512, 8, 32, None, C.byref(n), None) == L.FC_E_ARG
    n = norm(L, eps=float("nan"))
    assert f(sh, 2, 512, 8, 32, None, C.byref(n), None) == L.FC_E_ARG
    n = norm(L, gamma=None)
    assert f(sh, 2, 512, 8, 32, None, C.byref(n), None) == L.FC_E_NULL
    n = norm(L, residual_out=A + 0x300000 + 512)   # overlaps out
    assert f(sh, 2, 512, 8, 32, None, C.byref(n), None) == L.FC_E_ARG
    n = norm(L, residual_out=A + 0x100000 + 16)    # partially overlaps residual
    assert f(sh, 2, 512, 8, 32, None, C.byref(n), None) == L.FC_E_ARG
    n = norm(L, out=A + 0x300002)
    assert f(sh, 2, 512, 8, 32, None, C.byref(n), None) == L.FC_E_ALIGN
    n = norm(L)
    assert f(sh, 0, 512, 8, 32, None, C.byref(n), None) == L.FC_E_ARG
    assert f(sh, 2, 0, 8, 32, None, C.byref(n), None) == L.FC_OK


def test_reduce_rmsnorm_validation(L):
    f = L.lib.fc_reduce_rmsnorm
    parts = (C.c_void_p * 2)(A + 0x1000000, A + 0x2000000)
    n = norm(L)
    assert f(parts, 2, 4, None, 0, None) == L.FC_E_NULL
    assert f(parts, 2, 4, C.byref(n), -1, None) == L.FC_E_ARG
    assert f(parts, 0, 4, C.byref(n), 0, None) == L.FC_E_ARG
    assert f(parts, 2, 0, C.byref(n), 0, None) == L.FC_OK
    n2 = norm(L, hidden=131072)
    assert f(parts, 2, 4, C.byref(n2), 0, None) == L.FC_E_SHAPE
    bad = (C.c_void_p * 2)(A + 0x1000000, A + 0x2000004)
    assert f(bad, 2, 4, C.byref(n), 0, None) == L.FC_E_ALIGN
    over = (C.c_void_p * 2)(A + 0x1000000, A + 0x300000)   # a partial is the output
    assert f(over, 2, 4, C.byref(n), 0, None) == L.FC_E_ARG
    nul = (C.c_void_p * 2)(A + 0x1000000, None)
    assert f(nul, 2, 4, C.byref(n), 0, None) == L.FC_E_NULL


def test_ll_validation(L):
    f = L.lib.fc_ll_unpack_reduce
    sl = (C.c_void_p * 2)(A + 0x1000000, A + 0x2000000)
    args = dict(out=A + 0x3000000, stale=A + 0x4000000, done=A + 0x5000000, cnt=A + 0x6000000)
    g = lambda R=2, n=4096, B=64, **kw: f(sl, R, n, B, 7, kw.get("out", args["out"]), kw.get("stale", args["stale"]),
                                          kw.get("done", args["done"]), kw.get("cnt", args["cnt"]), None)
    assert g(B=48) == L.FC_E_ARG
    assert g(n=4096 + 64) == L.FC_E_SHAPE
    assert g(n=0) == L.FC_OK
    assert g(out=None) == L.FC_E_NULL
    assert g(out=A + 0x3000008) == L.FC_E_ALIGN
    assert g(cnt=A + 0x6000002) == L.FC_E_ALIGN
    assert g(cnt=A + 0x6000004) == L.FC_E_ALIGN    # both counts take one 64-bit atomic: 8-byte aligned
    assert g(cnt=A + 0x5000000 - 4 * L.COUNTER_WORDS + 8) == L.FC_E_ARG  # the last counter group reaches into done
    # counters may be NULL (nothing counted); every other check still applies (no call here launches)
    assert g(cnt=None, n=0) == L.FC_OK
    assert g(cnt=None, done=None) == L.FC_E_NULL
    assert g(cnt=None, out=A + 0x1000000 + 64) == L.FC_E_ARG
    assert g(done=A + 0x4000000 + 8) == L.FC_E_ARG   # done inside the stale flags
    assert g(out=A + 0x1000000 + 64) == L.FC_E_ARG   # out inside rank 0's slots
    p = L.lib.fc_ll_pack
    one = lambda *v: (C.c_void_p * len(v))(*v)
    X, S = one(A), one(A + 0x1000000)
    assert p(X, 1, 4096, 60, 7, None, 0, S, None) == L.FC_E_ARG
    assert p(X, 0, 4096, 64, 7, None, 0, S, None) == L.FC_E_ARG                # R
    assert p(X, 1, 4096, 64, 7, None, -1, S, None) == L.FC_E_ARG               # pace
    assert p(X, 1, 4096, 64, 7, None, 65537, S, None) == L.FC_E_ARG
    assert p(X, 1, 4000, 64, 7, None, 0, S, None) == L.FC_E_SHAPE
    assert p(X, 1, 0, 64, 7, None, 0, S, None) == L.FC_OK                     # empty: no launch
    assert p(X, 1, 4096, 64, 7, None, 0, one(A + 8), None) == L.FC_E_ALIGN
    assert p(X, 1, 4096, 64, 7, None, 0, one(A + 1024), None) == L.FC_E_ARG     # slots over the input
    assert p(X, 1, 4096, 64, 7, one(A + 0x1000000 + 64), 0, S, None) == L.FC_E_ARG  # order inside the slots
    X2 = one(A, A + 0x100000)
    assert p(X2, 2, 4096, 64, 7, None, 0, one(A + 0x1000000, None), None) == L.FC_E_NULL
    assert p(X2, 2, 4096, 64, 7, None, 0, one(A + 0x1000000, A + 0x1000000 + 4096), None) == L.FC_E_ARG
    assert p(X2, 2, 4096, 64, 7, None, 0, one(A + 0x1000000, A + 0x100000 + 16), None) == L.FC_E_ARG  # over x[1]


def test_ll_poll_validation(L):
    f = L.lib.fc_ll_poll_unpack_reduce
    sl = (C.c_void_p * 2)(A + 0x1000000, A + 0x2000000)
    d = dict(out=A + 0x3000000, stale=A + 0x4000000, done=A + 0x5000000, cnt=A + 0x6000000)
    g = lambda R=2, n=4096, B=64, polls=0, mw=0, s=sl, **kw: f(
        s, R, n, B, 7, polls, mw, kw.get("out", d["out"]), kw.get("stale", d["stale"]), kw.get("done", d["done"]),
        kw.get("cnt", d["cnt"]), None)
    assert g(B=48) == L.FC_E_ARG
    assert g(R=17) == L.FC_E_ARG
    assert g(polls=-1) == L.FC_E_ARG
    assert g(polls=(1 << 20) + 1) == L.FC_E_ARG
    assert g(mw=-1) == L.FC_E_ARG
    assert g(n=4096 + 64) == L.FC_E_SHAPE
    assert g(n=0) == L.FC_OK
    # counters may be NULL (nothing counted); every other check still applies (no call here launches)
    assert g(cnt=None, n=0) == L.FC_OK
    assert g(cnt=None, out=None) == L.FC_E_NULL
    assert g(cnt=None, out=A + 0x3000008) == L.FC_E_ALIGN
    assert g(cnt=A + 0x6000004) == L.FC_E_ALIGN
    assert g(out=A + 0x3000008) == L.FC_E_ALIGN
    assert g(s=(C.c_void_p * 2)(A + 0x1000008, A + 0x2000000)) == L.FC_E_ALIGN
    assert g(cnt=A + 0x5000000 - 8) == L.FC_E_ARG                    # the counter groups reach into done
    assert g(cnt=A + 0x5000000 - 4 * L.COUNTER_WORDS + 8) == L.FC_E_ARG
    assert g(out=A + 0x2000000 + 64) == L.FC_E_ARG                   # out inside rank 1's slots


def test_flag_validation(L):
    f = L.lib.fc_flag_unpack_reduce
    pl = (C.c_void_p * 2)(A + 0x1000000, A + 0x2000000)
    fl = (C.c_void_p * 2)(A + 0x7000000, A + 0x7100000)
    d = dict(out=A + 0x3000000, stale=A + 0x4000000, done=A + 0x5000000, cnt=A + 0x6000000)
    g = lambda R=2, n=8192, be=1024, polls=0, mw=0, p=pl, fg=fl, **kw: f(
        p, fg, R, n, be, 7, polls, mw, kw.get("out", d["out"]), kw.get("stale", d["stale"]),
        kw.get("done", d["done"]), kw.get("cnt", d["cnt"]), None)
    for be in (256, 768, 1 << 17):
        assert g(be=be) == L.FC_E_ARG                               # block: a power of two, 512 .. 65536
    assert g(R=0) == L.FC_E_ARG
    assert g(polls=-1) == L.FC_E_ARG
    assert g(mw=-1) == L.FC_E_ARG
    assert g(n=8192 + 512) == L.FC_E_SHAPE
    assert g(n=0) == L.FC_OK
    assert g(fg=(C.c_void_p * 2)(A + 0x7000000, None)) == L.FC_E_NULL
    assert g(fg=(C.c_void_p * 2)(A + 0x7000002, A + 0x7100000)) == L.FC_E_ALIGN   # flag words: 4-byte aligned
    assert g(p=(C.c_void_p * 2)(A + 0x1000004, A + 0x2000000)) == L.FC_E_ALIGN
    assert g(cnt=A + 0x6000004) == L.FC_E_ALIGN
    assert g(fg=(C.c_void_p * 2)(A + 0x7000000, A + 0x3000000 + 16)) == L.FC_E_ARG  # flags inside out
    assert g(done=A + 0x2000000 + 8) == L.FC_E_ARG                                  # done inside a payload
    pk = L.lib.fc_flag_pack
    one = lambda *v: (C.c_void_p * len(v))(*v)
    X, P, F = one(A), one(A + 0x1000000), one(A + 0x2000000)
    assert pk(X, 1, 8192, 1000, 7, None, 0, P, F, None) == L.FC_E_ARG
    assert pk(X, 17, 8192, 1024, 7, None, 0, P, F, None) == L.FC_E_ARG
    assert pk(X, 1, 8192, 1024, 7, None, -1, P, F, None) == L.FC_E_ARG
    assert pk(X, 1, 8192 + 16, 1024, 7, None, 0, P, F, None) == L.FC_E_SHAPE
    assert pk(X, 1, 0, 1024, 7, None, 0, P, F, None) == L.FC_OK                  # empty: no launch
    assert pk(X, 1, 8192, 1024, 7, None, 0, P, one(A + 0x2000002), None) == L.FC_E_ALIGN
    assert pk(X, 1, 8192, 1024, 7, None, 0, P, one(A + 0x1000000 + 64), None) == L.FC_E_ARG    # flags in payload
    assert pk(X, 1, 8192, 1024, 7, one(A + 0x1000000), 0, P, F, None) == L.FC_E_ARG            # order in payload
    X2, P2 = one(A, A + 0x100000), one(A + 0x1000000, A + 0x1800000)
    assert pk(X2, 2, 8192, 1024, 7, None, 0, P2, one(A + 0x2000000, A + 0x2000000 + 16), None) == L.FC_E_ARG
    assert pk(X2, 2, 8192, 1024, 7, None, 0, P2, one(A + 0x2000000, A + 0x1800000 + 32), None) == L.FC_E_ARG
    assert pk(X2, 2, 8192, 1024, 7, None, 0, P2, one(A + 0x2000000, None), None) == L.FC_E_NULL


def test_ll_gather_validation(L):
    f = L.lib.fc_ll_gather
    sl = (C.c_void_p * 2)(A + 0x1000000, A + 0x2000000)
    out = (C.c_void_p * 2)(A + 0x3000000, A + 0x3800000)
    d = dict(stale=A + 0x4000000, done=A + 0x5000000, cnt=A + 0x6000000)
    g = lambda R=2, n=4096, B=64, o=out, s=sl, **kw: f(s, R, n, B, 7, o, kw.get("stale", d["stale"]),
                                                       kw.get("done", d["done"]), kw.get("cnt", d["cnt"]), None)
    assert g(B=48) == L.FC_E_ARG
    assert g(R=0) == L.FC_E_ARG
    assert g(n=4096 + 32) == L.FC_E_SHAPE
    assert g(n=0) == L.FC_OK
    # counters may be NULL (nothing counted); every other check still applies (no call here launches)
    assert g(cnt=None, n=0) == L.FC_OK
    assert g(cnt=None, stale=None) == L.FC_E_NULL
    assert g(cnt=None, done=A + 0x4000000 + 8) == L.FC_E_ARG
    assert g(cnt=A + 0x6000004) == L.FC_E_ALIGN
    assert g(o=(C.c_void_p * 2)(A + 0x3000004, A + 0x3800000)) == L.FC_E_ALIGN
    assert g(s=(C.c_void_p * 2)(A + 0x1000008, A + 0x2000000)) == L.FC_E_ALIGN
    assert g(o=(C.c_void_p * 2)(A + 0x3000000, A + 0x3000000 + 64)) == L.FC_E_ARG   # two outputs overlap
    assert g(o=(C.c_void_p * 2)(A + 0x3000000, A + 0x2000000 + 64)) == L.FC_E_ARG   # an output over slots
    assert g(done=A + 0x4000000 + 8) == L.FC_E_ARG                                  # done over stale


def test_copy_validation(L):
    f = L.lib.fc_copy
    assert f(A, A + 0x100000, 100, None) == L.FC_E_SHAPE
    assert f(A, A + 64, 1024, None) == L.FC_E_ARG
    assert f(A, A + 0x100000, 0, None) == L.FC_OK
    assert f(None, A, 1024, None) == L.FC_E_NULL


def test_bandwidth_probe_validation(L):
    f = L.lib.fc_bandwidth_probe
    assert f(A, A + 0x100000, 1024, 3, None) == L.FC_E_ARG        # mode
    assert f(A, A + 0x100000, 100, 1, None) == L.FC_E_SHAPE
    assert f(A, A + 0x100000, 0, 2, None) == L.FC_OK
    assert f(None, A, 1024, 1, None) == L.FC_E_NULL                # read needs its source
    assert f(A, None, 1024, 1, None) == L.FC_E_NULL                # ... and its sink
    assert f(A, A + 0x100002, 1024, 1, None) == L.FC_E_ALIGN        # sink: 4-byte aligned
    assert f(A, A + 0x100004, 1024, 2, None) == L.FC_E_ALIGN        # written range: 16-byte aligned
    assert f(A, A + 512, 1024, 1, None) == L.FC_E_ARG               # sink inside the range read
    assert f(A, A + 64, 1024, 0, None) == L.FC_E_ARG                # copy: overlap
