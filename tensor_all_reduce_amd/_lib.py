"""ctypes binding for libfc.so (see include/fc.h): argument marshalling only.

Every function takes torch tensors (device memory) and passes their addresses, sizes and the current
HIP stream to the C ABI of the same name; all arithmetic runs in the HIP kernels.  A non-OK status
raises :class:`FcError`.  If the library has not been built, importing this module raises: there is no
fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import torch  # loads PyTorch's HIP runtime first; libfc.so binds to that same runtime

HERE = os.path.dirname(os.path.abspath(__file__))
# FC_LIB_PATH loads another build of the same library (e.g. one compiled with a different cache policy,
# to compare the two); by default the in-tree build is used.
LIB_PATH = os.environ.get("FC_LIB_PATH", os.path.join(HERE, "libfc.so"))

FC_OK, FC_E_NULL, FC_E_ARG, FC_E_SHAPE, FC_E_ALIGN, FC_E_LAUNCH = range(6)


class FcError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.fc_status_string(status).decode()  # the library the failing call went through
        if status == FC_E_LAUNCH:
            msg += " (hipError %d)" % lib.fc_last_hip_error()
        super().__init__(f"{where}: {msg}")


class QMsg(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("meta", C.c_void_p)]


class Norm(C.Structure):
    _fields_ = [("residual", C.c_void_p), ("gamma", C.c_void_p), ("eps", C.c_float), ("hidden", C.c_int64),
                ("out", C.c_void_p), ("residual_out", C.c_void_p)]


def _hip_runtimes_mapped() -> set[str]:
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m tensor_all_reduce_amd.build` "
                          "(or __graft_entry__.build()); there is no CPU fallback")
    lib = C.CDLL(LIB_PATH)
    rts = _hip_runtimes_mapped()
    if len(rts) > 1:
        raise ImportError("two HIP runtimes are mapped in this process (%s); libfc.so must share "
                          "PyTorch's" % ", ".join(sorted(rts)))
    vp, i64, i32, u32 = C.c_void_p, C.c_int64, C.c_int, C.c_uint32
    lib.fc_status_string.restype = C.c_char_p
    lib.fc_status_string.argtypes = [i32]
    lib.fc_last_hip_error.restype = i32
    lib.fc_abi_version.restype = i32
    lib.fc_quantize.argtypes = [vp, i64, i32, i32, QMsg, vp]
    lib.fc_reduce_shard.argtypes = [C.POINTER(QMsg), i32, i64, i32, i32, i32, i32, C.POINTER(QMsg), vp]
    lib.fc_reduce_shard_norm.argtypes = [C.POINTER(QMsg), i32, i64, i32, i32, i32, i32, C.POINTER(Norm),
                                         C.POINTER(QMsg), vp]
    lib.fc_gather_dequant.argtypes = [C.POINTER(QMsg), i32, i64, i32, i32, vp, C.POINTER(Norm), vp]
    lib.fc_reduce_rmsnorm.argtypes = [C.POINTER(vp), i32, i64, C.POINTER(Norm), i32, vp]
    lib.fc_ll_unpack_reduce.argtypes = [C.POINTER(vp), i32, i64, i32, u32, vp, vp, vp, vp, vp]
    lib.fc_ll_pack.argtypes = [C.POINTER(vp), i32, i64, i32, u32, C.POINTER(vp), i32, C.POINTER(vp), vp]
    lib.fc_ll_poll_unpack_reduce.argtypes = [C.POINTER(vp), i32, i64, i32, u32, i32, i32, vp, vp, vp, vp, vp]
    lib.fc_flag_unpack_reduce.argtypes = [C.POINTER(vp), C.POINTER(vp), i32, i64, i32, u32, i32, i32, vp, vp, vp,
                                          vp, vp]
    lib.fc_flag_pack.argtypes = [C.POINTER(vp), i32, i64, i32, u32, C.POINTER(vp), i32, C.POINTER(vp), C.POINTER(vp),
                                 vp]
    lib.fc_ll_gather.argtypes = [C.POINTER(vp), i32, i64, i32, u32, C.POINTER(vp), vp, vp, vp, vp]
    lib.fc_copy.argtypes = [vp, vp, i64, vp]
    lib.fc_bandwidth_probe.argtypes = [vp, vp, i64, i32, vp]
    for f in ("fc_quantize", "fc_reduce_shard", "fc_reduce_shard_norm", "fc_gather_dequant", "fc_reduce_rmsnorm", "fc_ll_unpack_reduce",
              "fc_ll_pack", "fc_ll_gather", "fc_ll_poll_unpack_reduce", "fc_flag_unpack_reduce", "fc_flag_pack",
              "fc_copy", "fc_bandwidth_probe"):
        getattr(lib, f).restype = i32
    return lib


ABI_VERSION = 5  # the argument lists above follow include/fc.h at this FC_ABI_VERSION

_lib = _load()
lib = _lib
if _lib.fc_abi_version() != ABI_VERSION:
    raise ImportError(f"{LIB_PATH} has ABI version {_lib.fc_abi_version()}, this binding expects {ABI_VERSION}: "
                      "rebuild it with `python -m tensor_all_reduce_amd.build`")


def _dev(t, nbytes: int | None = None, what: str = "buffer") -> int | None:
    """Address of a device buffer.  None passes through (an optional argument) and an int is taken as a
    raw device address that the caller vouches for.  A tensor must be contiguous, in device memory and
    at least `nbytes` long, else ValueError: the kernels would otherwise read or write a host or too
    small buffer out of bounds, which is a device fault rather than an error."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: a torch tensor, an int device address or None is required, got {type(t).__name__}")
    if t.device.type != "cuda":
        raise ValueError(f"{what}: the tensor must be in device memory (it is on {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{what}: the tensor must be contiguous")
    have = t.numel() * t.element_size()
    if nbytes is not None and have < nbytes:
        raise ValueError(f"{what}: {have} bytes, the call reads or writes {nbytes}")
    return t.data_ptr()


_ptr = _dev


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(st: int, where: str):
    if st != FC_OK:
        raise FcError(st, where)


def _count(lst, want: int, what: str, per: str) -> None:
    """The C side reads exactly `want` entries of a host pointer array; a shorter list would make it read
    past the array and launch with garbage device addresses, so the lengths are checked here."""
    if len(lst) != want:
        raise ValueError(f"{what}: {len(lst)} entries, the call reads {want} ({per})")


def _qmsg(m, n: int = 0, bits: int = 8, group: int = 1, what: str = "message") -> QMsg:
    """A quantized message of n elements: n*bits/8 bytes of codes, a 4-byte word per group."""
    codes, meta = m
    return QMsg(_dev(codes, max(0, n) * bits // 8, what + " codes"),
                _dev(meta, 4 * (max(0, n) // max(1, group)), what + " meta"))


def _norm(norm, elems: int = 0) -> Norm | None:
    """The epilogue's arguments; residual, out and residual_out cover `elems` bf16 elements."""
    if norm is None:
        return None
    hidden = int(norm["hidden"])
    nb = 2 * max(0, elems)
    return Norm(_dev(norm.get("residual"), nb, "residual"), _dev(norm["gamma"], 2 * max(0, hidden), "gamma"),
                float(norm.get("eps", 1e-5)), hidden, _dev(norm.get("out"), nb, "out"),
                _dev(norm.get("residual_out"), nb, "residual_out"))


def fc_quantize(x, bits: int, group: int, codes, meta, n: int | None = None, stream=None) -> None:
    """Group-quantize bf16 `x` (n elements, default x.numel()) into `codes` and `meta`."""
    n = x.numel() if n is None else n
    _check(_lib.fc_quantize(_dev(x, 2 * max(0, n), "x"), n, bits, group, _qmsg((codes, meta), n, bits, group, "out"),
                            _stream(stream)), "fc_quantize")


def fc_reduce_shard(inputs, R: int, L: int, bits_in: int, bits_out: int, group: int, outputs, stream=None) -> None:
    """inputs: n_shards*R (codes, meta) pairs, [shard][rank]; outputs: n_shards (codes, meta) pairs."""
    n_shards = len(outputs)
    _count(inputs, n_shards * R, "inputs", f"{n_shards} shards x R={R}")
    ins = (QMsg * len(inputs))(*[_qmsg(m, L, bits_in, group, "input") for m in inputs])
    outs = (QMsg * n_shards)(*[_qmsg(m, L, bits_out, group, "output") for m in outputs])
    _check(_lib.fc_reduce_shard(ins, R, L, n_shards, bits_in, bits_out, group, outs, _stream(stream)),
           "fc_reduce_shard")


def fc_reduce_shard_norm(inputs, R: int, L: int, bits_in: int, bits_out: int, group: int, norm: dict, outputs,
                         stream=None) -> None:
    """As fc_reduce_shard, with the residual-add + RMSNorm applied to the shards' rows before the
    normalized rows are quantized into `outputs`.  norm: dict(residual, gamma, eps, hidden, residual_out)
    over the n_shards*L elements of the shards, without "out"."""
    n_shards = len(outputs)
    _count(inputs, n_shards * R, "inputs", f"{n_shards} shards x R={R}")
    ins = (QMsg * len(inputs))(*[_qmsg(m, L, bits_in, group, "input") for m in inputs])
    outs = (QMsg * n_shards)(*[_qmsg(m, L, bits_out, group, "output") for m in outputs])
    nm = _norm(norm, n_shards * L)
    _check(_lib.fc_reduce_shard_norm(ins, R, L, n_shards, bits_in, bits_out, group, C.byref(nm), outs,
                                     _stream(stream)), "fc_reduce_shard_norm")


def fc_gather_dequant(shards, L: int, bits: int, group: int, y=None, norm: dict | None = None, stream=None) -> None:
    """shards: R (codes, meta) pairs; y: bf16 [R*L] or None; norm: dict(residual, gamma, eps, hidden, out,
    residual_out) or None."""
    R = len(shards)
    arr = (QMsg * R)(*[_qmsg(m, L, bits, group, "shard") for m in shards])
    nm = _norm(norm, R * L)
    _check(_lib.fc_gather_dequant(arr, R, L, bits, group, _dev(y, 2 * R * max(0, L), "y"),
                                  C.byref(nm) if nm is not None else None,
                                  _stream(stream)), "fc_gather_dequant")


def fc_reduce_rmsnorm(parts, rows: int, norm: dict, max_workgroups: int = 0, stream=None) -> None:
    R = len(parts)
    elems = max(0, rows) * max(0, int(norm["hidden"]))
    arr = (C.c_void_p * R)(*[_dev(p, 2 * elems, "part") for p in parts])
    nm = _norm(norm, elems)
    _check(_lib.fc_reduce_rmsnorm(arr, R, rows, C.byref(nm), max_workgroups, _stream(stream)), "fc_reduce_rmsnorm")


# Receiver counters (include/fc.h): COUNTER_GROUPS groups of words COUNTER_STRIDE words apart, one group
# per workgroup index mod COUNTER_GROUPS; a count's total is the sum of its word over the groups.
COUNTER_GROUPS, COUNTER_STRIDE = 8, 128
COUNTER_WORDS = COUNTER_GROUPS * COUNTER_STRIDE
COUNTER_BYTES = 4 * COUNTER_WORDS


def counter_totals(counters, ncounts: int = 4):
    """The first `ncounts` counts of a receiver's counters buffer (a tensor of COUNTER_WORDS 32-bit words,
    read back to the host), summed over the groups: numpy uint64 [ncounts]."""
    import numpy as np
    w = counters.detach().cpu().numpy().view(np.uint32).reshape(COUNTER_GROUPS, COUNTER_STRIDE)
    return w[:, :ncounts].astype(np.uint64).sum(axis=0)


def fc_ll_unpack_reduce(slots, n: int, block_slots: int, epoch: int, out, stale, done, counters, stream=None) -> None:
    R = len(slots)
    n, nblk = max(0, n), max(0, n) // 2 // max(1, block_slots)
    arr = (C.c_void_p * R)(*[_dev(s, 4 * n, "slots") for s in slots])
    _check(_lib.fc_ll_unpack_reduce(arr, R, n, block_slots, epoch & 0xFFFFFFFF, _dev(out, 2 * n, "out"),
                                    _dev(stale, R * nblk, "stale"), _dev(done, nblk, "done"),
                                    _dev(counters, COUNTER_BYTES, "counters"), _stream(stream)), "fc_ll_unpack_reduce")


def fc_ll_gather(slots, nwords: int, block_slots: int, epoch: int, out, stale, done, counters, stream=None) -> None:
    """slots: R uint64 slot buffers; out: R uint32 (or any 4-byte) destination buffers."""
    R = len(slots)
    _count(out, R, "out", "one per rank's slots")
    nw = max(0, nwords)
    nblk = nw // max(1, block_slots)
    sa = (C.c_void_p * R)(*[_dev(s, 8 * nw, "slots") for s in slots])
    oa = (C.c_void_p * R)(*[_dev(o, 4 * nw, "out") for o in out])
    _check(_lib.fc_ll_gather(sa, R, nwords, block_slots, epoch & 0xFFFFFFFF, oa, _dev(stale, R * nblk, "stale"),
                             _dev(done, R * nblk, "done"), _dev(counters, COUNTER_BYTES, "counters"), _stream(stream)),
           "fc_ll_gather")


def _ranks(v):
    """A tensor (one rank) or a list of R tensors -> list."""
    return list(v) if isinstance(v, (list, tuple)) else [v]


def _ptrs(lst, nbytes: int | None = None, what: str = "buffer"):
    return (C.c_void_p * len(lst))(*[_dev(t, nbytes, what) for t in lst])


def fc_ll_pack(x, block_slots: int, epoch: int, slots, block_order=None, n: int | None = None, pace: int = 0,
               stream=None) -> None:
    """x, slots, block_order: one tensor each (one rank) or lists of R (R peers in one launch)."""
    xs, ss = _ranks(x), _ranks(slots)
    _count(ss, len(xs), "slots", "one per rank's x")
    if block_order is not None:
        _count(_ranks(block_order), len(xs), "block_order", "one per rank's x")
    n = xs[0].numel() if n is None else n
    nn = max(0, n)
    oa = None if block_order is None else _ptrs(_ranks(block_order), 4 * (nn // 2 // max(1, block_slots)),
                                                "block_order")
    _check(_lib.fc_ll_pack(_ptrs(xs, 2 * nn, "x"), len(xs), n, block_slots, epoch & 0xFFFFFFFF, oa, pace,
                           _ptrs(ss, 4 * nn, "slots"), _stream(stream)), "fc_ll_pack")


def fc_ll_poll_unpack_reduce(slots, n: int, block_slots: int, epoch: int, out, stale, done, counters,
                             max_polls: int = 0, max_workgroups: int = 0, stream=None) -> None:
    """counters: COUNTER_WORDS int32 or None; counts (counter_totals): stale pairs, pending blocks, re-reads."""
    R = len(slots)
    nn = max(0, n)
    nblk = nn // 2 // max(1, block_slots)
    arr = (C.c_void_p * R)(*[_dev(s, 4 * nn, "slots") for s in slots])
    _check(_lib.fc_ll_poll_unpack_reduce(arr, R, n, block_slots, epoch & 0xFFFFFFFF, max_polls, max_workgroups,
                                         _dev(out, 2 * nn, "out"), _dev(stale, R * nblk, "stale"),
                                         _dev(done, nblk, "done"), _dev(counters, COUNTER_BYTES, "counters"),
                                         _stream(stream)),
           "fc_ll_poll_unpack_reduce")


def fc_flag_unpack_reduce(payload, flags, n: int, block_elems: int, epoch: int, out, stale, done, counters,
                          max_polls: int = 0, max_workgroups: int = 0, stream=None) -> None:
    """payload: R bf16 (int16) buffers; flags: R int32 buffers of n / block_elems words; counters as for
    fc_ll_poll_unpack_reduce."""
    R = len(payload)
    _count(flags, R, "flags", "one per rank's payload")
    nn = max(0, n)
    nblk = nn // max(1, block_elems)
    pa = (C.c_void_p * R)(*[_dev(p, 2 * nn, "payload") for p in payload])
    fa = (C.c_void_p * R)(*[_dev(f, 4 * nblk, "flags") for f in flags])
    _check(_lib.fc_flag_unpack_reduce(pa, fa, R, n, block_elems, epoch & 0xFFFFFFFF, max_polls, max_workgroups,
                                      _dev(out, 2 * nn, "out"), _dev(stale, R * nblk, "stale"),
                                      _dev(done, nblk, "done"), _dev(counters, COUNTER_BYTES, "counters"), _stream(stream)),
           "fc_flag_unpack_reduce")


def fc_flag_pack(x, block_elems: int, epoch: int, payload, flags, block_order=None, n: int | None = None,
                 pace: int = 0, stream=None) -> None:
    """x, payload, flags, block_order: one tensor each (one rank) or lists of R (R peers in one launch)."""
    xs = _ranks(x)
    _count(_ranks(payload), len(xs), "payload", "one per rank's x")
    _count(_ranks(flags), len(xs), "flags", "one per rank's x")
    if block_order is not None:
        _count(_ranks(block_order), len(xs), "block_order", "one per rank's x")
    n = xs[0].numel() if n is None else n
    nn = max(0, n)
    nblk = nn // max(1, block_elems)
    oa = None if block_order is None else _ptrs(_ranks(block_order), 4 * nblk, "block_order")
    _check(_lib.fc_flag_pack(_ptrs(xs, 2 * nn, "x"), len(xs), n, block_elems, epoch & 0xFFFFFFFF, oa, pace,
                             _ptrs(_ranks(payload), 2 * nn, "payload"), _ptrs(_ranks(flags), 4 * nblk, "flags"),
                             _stream(stream)), "fc_flag_pack")


def fc_copy(src, dst, nbytes: int | None = None, stream=None) -> None:
    nbytes = src.numel() * src.element_size() if nbytes is None else nbytes
    _check(_lib.fc_copy(_dev(src, max(0, nbytes), "src"), _dev(dst, max(0, nbytes), "dst"), nbytes, _stream(stream)),
           "fc_copy")


def fc_bandwidth_probe(src, dst, nbytes: int, mode: int, stream=None) -> None:
    """mode 0 copy, 1 read (dst: a 4-byte sink), 2 write (src unused)."""
    nb = max(0, nbytes)
    _check(_lib.fc_bandwidth_probe(_dev(src, nb if mode in (0, 1) else None, "src"),
                                   _dev(dst, nb if mode in (0, 2) else 4, "dst"), nbytes, mode, _stream(stream)),
           "fc_bandwidth_probe")


def fc_abi_version() -> int:
    return _lib.fc_abi_version()
