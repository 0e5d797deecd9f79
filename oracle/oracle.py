"""ctypes wrapper around the C++ CPU oracle (``fc_oracle.cpp``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the package smoke check and the benchmark's
CPU-baseline leg, never by the product path.  It shares nothing with the HIP library; it takes and
returns numpy arrays and host memory only.

The library is compiled with g++ (``-O2 -ffp-contract=off``, no fast-math) on first use, or when the
source is newer than the built file.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# FC_ORACLE_SRC lets a mutation check build a deliberately altered copy of the oracle elsewhere.
SRC = os.environ.get("FC_ORACLE_SRC", os.path.join(HERE, "fc_oracle.cpp"))
# FC_SANITIZE=1 builds (and loads) a copy instrumented with AddressSanitizer and UndefinedBehaviorSanitizer
# that stops at the first report; Python then needs the ASan runtime preloaded:
#   FC_SANITIZE=1 LD_PRELOAD=$(g++ -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \
#       python -m pytest tests -m "not gpu"
SANITIZE = os.environ.get("FC_SANITIZE") == "1"
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
LIB = os.path.join(os.path.dirname(SRC), "liboracle_san.so" if SANITIZE else "liboracle.so")

_lock = threading.Lock()
_lib = None

u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
u32p = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")
u64p = np.ctypeslib.ndpointer(np.uint64, flags="C_CONTIGUOUS")
i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
vp = C.c_void_p
i64 = C.c_int64


def build(force: bool = False) -> str:
    """Compile the oracle into ``liboracle.so`` (single-threaded, no contraction, no fast-math)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = ["g++", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c++17", "-fPIC", "-shared",
               *(SAN_FLAGS if SANITIZE else []), SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            _lib = C.CDLL(build())
            L = _lib
            L.or_f32_to_f16.argtypes = [f32p, i64, C.c_int, u16p]
            L.or_f16_to_f32.argtypes = [u16p, i64, f32p]
            L.or_f32_to_bf16.argtypes = [f32p, i64, u16p]
            L.or_quantize_f32.argtypes = [f32p, i64, C.c_int, C.c_int, u8p, u32p]
            L.or_quantize_bf16.argtypes = [u16p, i64, C.c_int, C.c_int, u8p, u32p]
            L.or_dequant.argtypes = [u8p, u32p, i64, C.c_int, C.c_int, f32p]
            L.or_reduce_shard.argtypes = [vp, vp, C.c_int, i64, C.c_int, C.c_int, C.c_int, vp, vp, vp]
            L.or_rmsnorm.argtypes = [f32p, vp, u16p, C.c_float, i64, i64, u16p, vp]
            L.or_gather.argtypes = [vp, vp, C.c_int, i64, C.c_int, C.c_int, vp, vp, vp, C.c_float, i64, vp, vp]
            L.or_two_step.argtypes = [vp, C.c_int, i64, C.c_int, C.c_int, C.c_int, u8p, u32p, u8p, u32p, vp,
                                      vp, vp, C.c_float, i64, vp, vp]
            L.or_reduce_rmsnorm.argtypes = [vp, C.c_int, i64, i64, vp, u16p, C.c_float, u16p, vp, vp]
            L.or_ll_pack.argtypes = [u16p, i64, C.c_int, C.c_uint32, vp, u64p]
            L.or_ll_unpack_reduce.argtypes = [vp, C.c_int, i64, C.c_int, C.c_uint32, u16p, u8p, u8p, u32p]
            L.or_ll_gather.argtypes = [vp, C.c_int, i64, C.c_int, C.c_uint32, vp, u8p, u8p, u32p]
            L.or_flag_unpack_reduce.argtypes = [vp, vp, C.c_int, i64, C.c_int, C.c_uint32, u16p, u8p, u8p, u32p]
            L.or_sumsq_tree.argtypes = [f32p, i64]
            L.or_sumsq_tree.restype = C.c_float
            L.or_sumsq_seq.argtypes = [f32p, i64]
            L.or_sumsq_seq.restype = C.c_float
            L.or_norm_rows_f32.argtypes = [f32p, vp, u16p, C.c_float, i64, i64, C.c_int, f32p, vp]
            L.or_reduce_norm_quant.argtypes = [vp, vp, C.c_int, i64, C.c_int, C.c_int, C.c_int, vp, u16p, C.c_float,
                                               i64, C.c_int, vp, u8p, u32p, vp]
            L.or_two_step_normfirst.argtypes = [vp, C.c_int, i64, C.c_int, C.c_int, C.c_int, u8p, u32p, u8p, u32p,
                                                vp, u16p, C.c_float, i64, C.c_int, vp, u16p]
        return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _ptr_array(arrs):
    return (C.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ---- conversions --------------------------------------------------------------------------------------
def f32_to_f16(x, mode=0):
    """mode 0 nearest-even, 1 round down, 2 round up; returns fp16 bit patterns (uint16)."""
    x = _c(x, np.float32)
    out = np.empty(x.size, np.uint16)
    lib().or_f32_to_f16(x.ravel(), x.size, mode, out)
    return out.reshape(x.shape)


def f16_to_f32(h):
    h = _c(h, np.uint16)
    out = np.empty(h.size, np.float32)
    lib().or_f16_to_f32(h.ravel(), h.size, out)
    return out.reshape(h.shape)


def f32_to_bf16(x):
    x = _c(x, np.float32)
    out = np.empty(x.size, np.uint16)
    lib().or_f32_to_bf16(x.ravel(), x.size, out)
    return out.reshape(x.shape)


# ---- quantization ---------------------------------------------------------------------------------------
def quantize(x, bits, group):
    """x: bf16 bit patterns (uint16) or float32 values, flat length n.  Returns (codes uint8, meta uint32)."""
    n = x.size
    codes = np.zeros(n * bits // 8, np.uint8)
    meta = np.zeros(n // group, np.uint32)
    if x.dtype == np.uint16:
        lib().or_quantize_bf16(_c(x, np.uint16).ravel(), n, bits, group, codes, meta)
    else:
        lib().or_quantize_f32(_c(x, np.float32).ravel(), n, bits, group, codes, meta)
    return codes, meta


def dequant(codes, meta, n, bits, group):
    y = np.empty(n, np.float32)
    lib().or_dequant(_c(codes, np.uint8), _c(meta, np.uint32), n, bits, group, y)
    return y


def reduce_shard(codes_list, meta_list, L, bits_in, bits_out, group, want_sum=False):
    """codes_list/meta_list: per rank, that rank's quantized chunk of one shard (L elements)."""
    R = len(codes_list)
    cl = [_c(c, np.uint8) for c in codes_list]
    ml = [_c(m, np.uint32) for m in meta_list]
    S = np.empty(L, np.float32) if want_sum else None
    oc = np.zeros(L * bits_out // 8, np.uint8)
    om = np.zeros(L // group, np.uint32)
    lib().or_reduce_shard(_ptr_array(cl), _ptr_array(ml), R, L, bits_in, bits_out, group, _ptr(S), _ptr(oc), _ptr(om))
    return (oc, om, S) if want_sum else (oc, om)


def rmsnorm(y, residual, gamma, eps, hidden):
    y = _c(y, np.float32).ravel()
    rows = y.size // hidden
    out = np.empty(y.size, np.uint16)
    rout = np.empty(y.size, np.uint16) if residual is not None else None
    res = _c(residual, np.uint16).ravel() if residual is not None else None
    lib().or_rmsnorm(y, _ptr(res), _c(gamma, np.uint16), eps, rows, hidden, out, _ptr(rout))
    return out, rout


def gather(codes_list, meta_list, L, bits, group, plain=True, residual=None, gamma=None, eps=1e-5, hidden=0):
    R = len(codes_list)
    cl = [_c(c, np.uint8) for c in codes_list]
    ml = [_c(m, np.uint32) for m in meta_list]
    n = R * L
    y = np.empty(n, np.uint16) if plain else None
    out = rout = None
    res = _c(residual, np.uint16).ravel() if residual is not None else None
    g = _c(gamma, np.uint16) if gamma is not None else None
    if g is not None:
        out = np.empty(n, np.uint16)
        rout = np.empty(n, np.uint16) if residual is not None else None
    lib().or_gather(_ptr_array(cl), _ptr_array(ml), R, L, bits, group, _ptr(y), _ptr(res), _ptr(g), eps,
                    hidden if hidden else n, _ptr(out), _ptr(rout))
    return y, out, rout


def two_step(parts, bits1, bits2, group, residual=None, gamma=None, eps=1e-5, hidden=0, plain=True):
    """The whole quantized two-step all-reduce for R bf16 partials (list of uint16 arrays, length n each).

    Returns a dict with the per-rank messages, the requantized shards and the gathered outputs."""
    R = len(parts)
    ps = [_c(p, np.uint16).ravel() for p in parts]
    n = ps[0].size
    c1 = np.zeros(R * n * bits1 // 8, np.uint8)
    m1 = np.zeros(R * n // group, np.uint32)
    c2 = np.zeros(n * bits2 // 8, np.uint8)
    m2 = np.zeros(n // group, np.uint32)
    y = np.empty(n, np.uint16) if plain else None
    out = rout = None
    res = _c(residual, np.uint16).ravel() if residual is not None else None
    g = _c(gamma, np.uint16) if gamma is not None else None
    if g is not None:
        out = np.empty(n, np.uint16)
        rout = np.empty(n, np.uint16) if residual is not None else None
    lib().or_two_step(_ptr_array(ps), R, n, bits1, bits2, group, c1, m1, c2, m2, _ptr(y), _ptr(res), _ptr(g), eps,
                      hidden if hidden else n, _ptr(out), _ptr(rout))
    return dict(codes1=c1.reshape(R, -1), meta1=m1.reshape(R, -1), codes2=c2, meta2=m2, y=y, out=out,
                residual_out=rout)


def flag_unpack_reduce(payload_list, flags_list, n, block_elems, epoch, out=None, done=None, counters=None):
    """Receiver of per-block flag words: returns (out bf16 [n], stale [R*nblk], done [nblk], counters [2])."""
    R = len(payload_list)
    nblk = n // block_elems
    pl = [_c(p, np.uint16).ravel() for p in payload_list]
    fl = [_c(f, np.uint32).ravel() for f in flags_list]
    out = np.zeros(n, np.uint16) if out is None else _c(out, np.uint16).copy()
    done = np.zeros(nblk, np.uint8) if done is None else _c(done, np.uint8).copy()
    counters = np.zeros(2, np.uint32) if counters is None else _c(counters, np.uint32).copy()
    stale = np.zeros(R * nblk, np.uint8)
    lib().or_flag_unpack_reduce(_ptr_array(pl), _ptr_array(fl), R, n, block_elems, epoch & 0xFFFFFFFF, out, stale,
                                done, counters)
    return out, stale, done, counters


def ll_gather(slots_list, nwords, block_slots, epoch, out=None, done=None, counters=None):
    """Standalone all-gather on epoch-tagged blocks: returns (out [R][nwords] uint32, stale [R*nblk],
    done [R*nblk], counters [2]); out/done/counters may be passed in to continue a previous pass."""
    R = len(slots_list)
    nblk = nwords // block_slots
    sl = [_c(s, np.uint64) for s in slots_list]
    out = [np.zeros(nwords, np.uint32) for _ in range(R)] if out is None else [_c(o, np.uint32) for o in out]
    done = np.zeros(R * nblk, np.uint8) if done is None else _c(done, np.uint8).copy()
    counters = np.zeros(2, np.uint32) if counters is None else _c(counters, np.uint32).copy()
    stale = np.zeros(R * nblk, np.uint8)
    lib().or_ll_gather(_ptr_array(sl), R, nwords, block_slots, epoch & 0xFFFFFFFF, _ptr_array(out), stale, done,
                       counters)
    return out, stale, done, counters


# ---- norm before the all-gather ---------------------------------------------------------------------
# The order of a row's sum of squares: "seq" is the plain reading (the epilogue's left fold of the rounded
# squares); "tree" is the fixed tree order the GPU kernels commit to (8-element chunk folds, then a
# pairwise tree over the chunks), which lets tests check the kernels' other steps bit for bit.
ORDER = {"seq": 0, "tree": 1}


def sumsq_tree(h):
    """Fixed-order sum of squares of one row (8-element chunk folds, pairwise tree over chunks)."""
    h = _c(h, np.float32).ravel()
    return np.float32(lib().or_sumsq_tree(h, h.size))


def sumsq_seq(h):
    """Sum of squares of one row as a left fold of the rounded squares (the plain reading)."""
    h = _c(h, np.float32).ravel()
    return np.float32(lib().or_sumsq_seq(h, h.size))


def norm_rows_f32(y, residual, gamma, eps, hidden, order="seq"):
    """fp32 normalized rows o (not rounded) and bf16 residual_out (None without residual)."""
    y = _c(y, np.float32).ravel()
    o = np.empty(y.size, np.float32)
    rout = np.empty(y.size, np.uint16) if residual is not None else None
    res = _c(residual, np.uint16).ravel() if residual is not None else None
    lib().or_norm_rows_f32(y, _ptr(res), _c(gamma, np.uint16), eps, y.size // hidden, hidden, ORDER[order], o,
                           _ptr(rout))
    return o, rout


def reduce_norm_quant(codes_list, meta_list, L, bits_in, bits_out, group, residual, gamma, eps, hidden,
                      order="seq"):
    """One shard with the norm first: returns (codes, meta, residual_out, o) of the shard."""
    R = len(codes_list)
    cl = [_c(c, np.uint8) for c in codes_list]
    ml = [_c(m, np.uint32) for m in meta_list]
    res = _c(residual, np.uint16).ravel() if residual is not None else None
    rout = np.empty(L, np.uint16) if residual is not None else None
    oc = np.zeros(L * bits_out // 8, np.uint8)
    om = np.zeros(L // group, np.uint32)
    o = np.empty(L, np.float32)
    lib().or_reduce_norm_quant(_ptr_array(cl), _ptr_array(ml), R, L, bits_in, bits_out, group, _ptr(res),
                               _c(gamma, np.uint16), eps, hidden, ORDER[order], _ptr(rout), oc, om, _ptr(o))
    return oc, om, rout, o


def two_step_normfirst(parts, bits1, bits2, group, residual, gamma, eps, hidden, order="seq"):
    """The whole two-step all-reduce with the norm applied to each shard before the all-gather."""
    R = len(parts)
    ps = [_c(p, np.uint16).ravel() for p in parts]
    n = ps[0].size
    c1 = np.zeros(R * n * bits1 // 8, np.uint8)
    m1 = np.zeros(R * n // group, np.uint32)
    c2 = np.zeros(n * bits2 // 8, np.uint8)
    m2 = np.zeros(n // group, np.uint32)
    res = _c(residual, np.uint16).ravel() if residual is not None else None
    rout = np.empty(n, np.uint16) if residual is not None else None
    y = np.empty(n, np.uint16)
    lib().or_two_step_normfirst(_ptr_array(ps), R, n, bits1, bits2, group, c1, m1, c2, m2, _ptr(res),
                                _c(gamma, np.uint16), eps, hidden, ORDER[order], _ptr(rout), y)
    return dict(codes1=c1.reshape(R, -1), meta1=m1.reshape(R, -1), codes2=c2, meta2=m2, y=y, residual_out=rout)


def reduce_rmsnorm(parts, rows, hidden, residual, gamma, eps, want_y=False):
    R = len(parts)
    ps = [_c(p, np.uint16).ravel() for p in parts]
    n = rows * hidden
    out = np.empty(n, np.uint16)
    rout = np.empty(n, np.uint16) if residual is not None else None
    y = np.empty(n, np.uint16) if want_y else None
    res = _c(residual, np.uint16).ravel() if residual is not None else None
    lib().or_reduce_rmsnorm(_ptr_array(ps), R, rows, hidden, _ptr(res), _c(gamma, np.uint16), eps, out, _ptr(rout),
                            _ptr(y))
    return out, rout, y


def ll_pack(x, block_slots, epoch, order=None):
    x = _c(x, np.uint16).ravel()
    slots = np.zeros(x.size // 2, np.uint64)
    o = _c(order, np.int32) if order is not None else None
    lib().or_ll_pack(x, x.size, block_slots, epoch, _ptr(o), slots)
    return slots


def ll_unpack_reduce(slots_list, n, block_slots, epoch, out=None, done=None, counters=None):
    """Returns (out, stale [R, nblk], done, counters).  out/done/counters are updated in place if given."""
    R = len(slots_list)
    sl = [_c(s, np.uint64) for s in slots_list]
    nblk = n // 2 // block_slots
    out = np.zeros(n, np.uint16) if out is None else out
    done = np.zeros(nblk, np.uint8) if done is None else done
    counters = np.zeros(2, np.uint32) if counters is None else counters
    stale = np.zeros(R * nblk, np.uint8)
    lib().or_ll_unpack_reduce(_ptr_array(sl), R, n, block_slots, epoch, out, stale, done, counters)
    return out, stale.reshape(R, nblk), done, counters
