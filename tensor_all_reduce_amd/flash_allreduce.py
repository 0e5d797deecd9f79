"""Host-side orchestration of one GPU's share of the flash all-reduce: buffers and call sequences.

PyTorch supplies device memory and the stream; every step runs in libfc.so's kernels.  The argument
tables (message pointers per shard and rank) are built once per buffer set, so enqueueing a step costs
a few ctypes calls and can be captured in a HIP graph.

Emulation on one GPU: the R ranks' partial sums are R buffers in local HBM, and the "transport" of each
step is the message buffer one call writes and the next call reads.  Ranks exchange data only through
those buffers.

Two-step layout (Flash Communication, summary "Core ideas of the solution"): rank r's message holds
the whole [T*H] partial, quantized; shard s is elements [s*L, (s+1)*L) with L = T*H/R, so rank r's chunk
of shard s sits at a fixed offset inside rank r's message.  After the reduce-scatter, shard s's
requantized message (the all-gather payload) sits at offset s inside one contiguous buffer.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _lib

u8, i16, i32, i64 = torch.uint8, torch.int16, torch.int32, torch.int64


def _device(device) -> torch.device:
    dev = torch.device(device)
    if dev.type != "cuda":
        raise ValueError(f"buffers must be in device memory, not on {dev}: every step runs in the HIP kernels")
    return dev


def _norm_args(gamma, out, residual, residual_out, eps: float, H: int, elems: int) -> _lib.Norm:
    """Checked epilogue arguments: residual, out and residual_out cover `elems` bf16 elements.  The returned
    structure holds raw device addresses, so it also keeps the tensors themselves (``_keep``): a temporary
    passed here stays allocated as long as the structure, and its memory cannot be handed to another
    tensor before the epilogue reads or writes it."""
    nm = _lib.Norm(_lib._dev(residual, 2 * elems, "residual"), _lib._dev(gamma, 2 * H, "gamma"), float(eps), H,
                   _lib._dev(out, 2 * elems, "out"), _lib._dev(residual_out, 2 * elems, "residual_out"))
    nm._keep = (gamma, out, residual, residual_out)
    return nm


# Rank buffers that a kernel reads side by side at equal offsets (the R ranks' chunks of a shard, the R
# partials of an unquantized reduce) are placed so that they do not start a large power of two apart:
# their R address streams would otherwise fall on the same HBM channels at the same time (measured on the
# 70B prefill reduce: 37.7 us with the messages 2^24 bytes apart, 32.4 us with a 4 KB stagger per rank).
STAGGER_BYTES = 4096
STAGGER_MIN_ROW = 1 << 20  # rows under 1 MB are left dense (a small buffer sits in the caches anyway)


def rank_rows(R: int, row: int, dtype, device, pad: int | None = None, zero: bool = False):
    """One allocation holding R rows of `row` elements, row r starting r * (row + pad) elements in.  pad
    defaults to STAGGER_BYTES worth of elements for rows of at least STAGGER_MIN_ROW bytes, else 0.
    Returns (buffer, rows): the flat buffer and a [R, row] view of it (each row contiguous)."""
    es = torch.empty(0, dtype=dtype).element_size()
    if pad is None:
        pad = STAGGER_BYTES // es if row * es >= STAGGER_MIN_ROW else 0
    buf = (torch.zeros if zero else torch.empty)(R * (row + pad), dtype=dtype, device=device)
    return buf, buf.view(R, row + pad)[:, :row]


def bf16_buffer(n: int, device) -> torch.Tensor:
    """bf16 bit patterns are held in int16 tensors (the kernels see raw 16-bit words)."""
    return torch.empty(n, dtype=i16, device=device)


def _check_shards(n: int, R: int, group: int) -> None:
    """The two-step layout needs R equal shards of whole groups."""
    if R < 1 or n % R or (n // R) % group:
        raise ValueError(f"T*H = {n} does not split into {R} shards of whole {group}-element groups")


class TwoStepAllReduce:
    """Buffers and enqueue functions for the quantized two-step all-reduce of R emulated ranks.

    parts: int16 [R, T*H] (bf16 bits) to copy in, or None (fill self.parts later).  Steps: quantize (all
    ranks, one launch), reduce_scatter (all shards, or one shard = one GPU's real share), all_gather
    (dequantize every shard, optionally with the residual-add + RMSNorm epilogue).

    Layout: the R partials are rows of one buffer, staggered by `pad` elements (zeros) between ranks for
    large messages, so that the one quantize launch (over all rows and pads) writes the R rank messages
    staggered too, and the reduce's R chunk streams of a shard do not start a power of two apart."""

    def __init__(self, R: int, T: int, H: int, bits_rs: int, bits_ag: int, group: int, device="cuda",
                 parts: torch.Tensor | None = None):
        self.R, self.T, self.H, self.b1, self.b2, self.G = R, T, H, bits_rs, bits_ag, group
        n = T * H
        _check_shards(n, R, group)
        self.n, self.L = n, n // R
        L = self.L
        dev = _device(device)
        # pad elements per rank: 8192 (a multiple of every group size) staggers the codes by 4 or 8 KB and
        # the meta by 256 B; the pads are zeros and are quantized with the rest (about 0.02% more bytes at
        # the 70B prefill shape)
        pad = 8192 if n * bits_rs // 8 >= STAGGER_MIN_ROW else 0
        self.pad = pad
        self._parts_buf, self.parts = rank_rows(R, n, i16, dev, pad=pad, zero=True)
        if parts is not None:
            self.parts.copy_(parts.reshape(R, n))
        self._codes1_buf, self.codes1 = rank_rows(R, n * bits_rs // 8, u8, dev, pad=pad * bits_rs // 8)
        self._meta1_buf, self.meta1 = rank_rows(R, n // group, i32, dev, pad=pad // group)
        self.codes2 = torch.empty(n * bits_ag // 8, dtype=u8, device=dev)
        self.meta2 = torch.empty(n // group, dtype=i32, device=dev)
        cb1, mb1 = L * bits_rs // 8, L // group
        cb2 = L * bits_ag // 8
        # (shard, rank) -> rank's chunk of the shard inside rank's message
        self._rs_in = (_lib.QMsg * (R * R))(*[
            _lib.QMsg(self.codes1[r].data_ptr() + s * cb1, self.meta1[r].data_ptr() + 4 * s * mb1)
            for s in range(R) for r in range(R)])
        self._rs_out = (_lib.QMsg * R)(*[
            _lib.QMsg(self.codes2.data_ptr() + s * cb2, self.meta2.data_ptr() + 4 * s * mb1) for s in range(R)])
        self._ag_in = self._rs_out
        self._q = _lib.QMsg(self._codes1_buf.data_ptr(), self._meta1_buf.data_ptr())

    # -- messages of one shard (views), e.g. to upload or inspect one GPU's share
    def rank_chunk(self, r: int, s: int):
        cb1, mb1 = self.L * self.b1 // 8, self.L // self.G
        return self.codes1[r, s * cb1:(s + 1) * cb1], self.meta1[r, s * mb1:(s + 1) * mb1]

    def shard_msg(self, s: int):
        cb2, mb = self.L * self.b2 // 8, self.L // self.G
        return self.codes2[s * cb2:(s + 1) * cb2], self.meta2[s * mb:(s + 1) * mb]

    # -- steps
    def quantize(self, stream=None):
        m = self.R * (self.n + self.pad)
        st = _lib.lib.fc_quantize(_lib._dev(self._parts_buf, 2 * m, "parts"), m, self.b1, self.G, self._q,
                                  _lib._stream(stream))
        _lib._check(st, "fc_quantize")

    def reduce_scatter(self, shard: int | None = None, stream=None):
        """All shards in one launch (shard=None), or only `shard` (one GPU's real share)."""
        R = self.R
        if shard is None:
            ins, outs, ns = self._rs_in, self._rs_out, R
        else:
            if not 0 <= int(shard) < R:
                raise ValueError(f"shard {shard}: the all-reduce has shards 0 .. {R - 1}")
            qs = C.sizeof(_lib.QMsg)
            ins = C.cast(C.addressof(self._rs_in) + qs * shard * R, C.POINTER(_lib.QMsg))
            outs = C.cast(C.addressof(self._rs_out) + qs * shard, C.POINTER(_lib.QMsg))
            ns = 1
        st = _lib.lib.fc_reduce_shard(ins, R, self.L, ns, self.b1, self.b2, self.G, outs, _lib._stream(stream))
        _lib._check(st, "fc_reduce_shard")

    def make_norm(self, gamma, out, residual=None, residual_out=None, eps: float = 1e-5) -> _lib.Norm:
        """The epilogue's arguments: every row of the T*H elements (as the gather's epilogue, or with out=None
        for the norm first)."""
        return _norm_args(gamma, out, residual, residual_out, eps, self.H, self.n)

    def reduce_scatter_norm(self, norm: _lib.Norm, stream=None):
        """Every shard's reduce with the norm first (make_norm with out=None; residual and residual_out
        over all T*H elements): the all-gather payload is the quantized normalized rows."""
        st = _lib.lib.fc_reduce_shard_norm(self._rs_in, self.R, self.L, self.R, self.b1, self.b2, self.G,
                                           C.byref(norm), self._rs_out, _lib._stream(stream))
        _lib._check(st, "fc_reduce_shard_norm")

    def run_norm_first(self, y, norm: _lib.Norm, stream=None):
        """Quantize, reduce + norm per shard, gather the normalized rows into y (bf16 [T*H])."""
        self.quantize(stream)
        self.reduce_scatter_norm(norm, stream)
        self.all_gather(y=y, stream=stream)

    def all_gather(self, y=None, norm: _lib.Norm | None = None, stream=None):
        st = _lib.lib.fc_gather_dequant(self._ag_in, self.R, self.L, self.b2, self.G, _lib._dev(y, 2 * self.n, "y"),
                                        C.byref(norm) if norm is not None else None, _lib._stream(stream))
        _lib._check(st, "fc_gather_dequant")

    def run(self, y=None, norm=None, stream=None):
        self.quantize(stream)
        self.reduce_scatter(None, stream)
        self.all_gather(y, norm, stream)


class TwoStepShare:
    """One GPU's real share of the quantized two-step all-reduce (rank `rank` owns shard `rank`).

    Buffers of this rank only: its partial x (bf16 [T*H]), its quantized message, the inbox of its shard
    (R chunk messages of L elements: rank r's chunk of shard `rank`; this rank's own chunk is read in
    place from its message), and the R all-gather messages (shard `rank` is written by reduce(); the
    others arrive from the peers).  On one GPU the caller fills the peers' inbox chunks and gather
    messages (upload or copy); on a real node the transport would.  Steps: quantize (own partial),
    reduce (own shard: fixed-order dequant-sum-requant of the R chunks), gather (all R shards, optionally
    with the residual-add + RMSNorm epilogue)."""

    def __init__(self, R: int, T: int, H: int, bits_rs: int, bits_ag: int, group: int, rank: int = 0,
                 device="cuda", x: torch.Tensor | None = None):
        self.R, self.T, self.H, self.b1, self.b2, self.G, self.rank = R, T, H, bits_rs, bits_ag, group, rank
        n = T * H
        _check_shards(n, R, group)
        if not 0 <= rank < R:
            raise ValueError(f"rank {rank} outside [0, {R})")
        self.n, self.L = n, n // R
        L, dev = self.L, _device(device)
        cb1, cb2, mb = L * bits_rs // 8, L * bits_ag // 8, L // group
        self.x = x if x is not None else torch.empty(n, dtype=i16, device=dev)
        _lib._dev(self.x, 2 * n, "x")
        self.codes1 = torch.empty(n * bits_rs // 8, dtype=u8, device=dev)   # own message, all R chunks
        self.meta1 = torch.empty(n // group, dtype=i32, device=dev)
        # peers' chunks of own shard, staggered between ranks (rank_rows) as the reduce reads them side by side
        self._inbox_codes_buf, self.inbox_codes = rank_rows(R, cb1, u8, dev)
        self._inbox_meta_buf, self.inbox_meta = rank_rows(R, mb, i32, dev, pad=64 if cb1 >= STAGGER_MIN_ROW else 0)
        self.codes2 = torch.empty(R, cb2, dtype=u8, device=dev)             # all-gather messages
        self.meta2 = torch.empty(R, mb, dtype=i32, device=dev)
        own = _lib.QMsg(self.codes1.data_ptr() + rank * cb1, self.meta1.data_ptr() + 4 * rank * mb)
        self._q = _lib.QMsg(self.codes1.data_ptr(), self.meta1.data_ptr())
        self._rs_in = (_lib.QMsg * R)(*[own if r == rank else
                                        _lib.QMsg(self.inbox_codes[r].data_ptr(), self.inbox_meta[r].data_ptr())
                                        for r in range(R)])
        self._ag = (_lib.QMsg * R)(*[_lib.QMsg(self.codes2[s].data_ptr(), self.meta2[s].data_ptr())
                                     for s in range(R)])
        self._rs_out = C.cast(C.addressof(self._ag) + C.sizeof(_lib.QMsg) * rank, C.POINTER(_lib.QMsg))

    def quantize(self, stream=None):
        st = _lib.lib.fc_quantize(_lib._dev(self.x, 2 * self.n, "x"), self.n, self.b1, self.G, self._q,
                                  _lib._stream(stream))
        _lib._check(st, "fc_quantize")

    def reduce(self, stream=None):
        st = _lib.lib.fc_reduce_shard(self._rs_in, self.R, self.L, 1, self.b1, self.b2, self.G, self._rs_out,
                                      _lib._stream(stream))
        _lib._check(st, "fc_reduce_shard")

    def make_norm(self, gamma, out, residual=None, residual_out=None, eps: float = 1e-5) -> _lib.Norm:
        """The epilogue's arguments: the gather's (out given: all T*H elements) or the own shard's norm first
        (out=None: its L elements)."""
        return _norm_args(gamma, out, residual, residual_out, eps, self.H, self.n if out is not None else self.L)

    def reduce_norm(self, norm: _lib.Norm, stream=None):
        """Own shard's reduce with the norm first (make_norm with out=None; residual and residual_out are
        the own shard's L elements): the own all-gather message holds the quantized normalized rows."""
        st = _lib.lib.fc_reduce_shard_norm(self._rs_in, self.R, self.L, 1, self.b1, self.b2, self.G, C.byref(norm),
                                           self._rs_out, _lib._stream(stream))
        _lib._check(st, "fc_reduce_shard_norm")

    def run_norm_first(self, y, norm: _lib.Norm, stream=None):
        self.quantize(stream)
        self.reduce_norm(norm, stream)
        self.gather(y=y, stream=stream)

    def gather(self, y=None, norm: _lib.Norm | None = None, stream=None):
        st = _lib.lib.fc_gather_dequant(self._ag, self.R, self.L, self.b2, self.G, _lib._dev(y, 2 * self.n, "y"),
                                        C.byref(norm) if norm is not None else None, _lib._stream(stream))
        _lib._check(st, "fc_gather_dequant")

    def run(self, y=None, norm=None, stream=None):
        self.quantize(stream)
        self.reduce(stream)
        self.gather(y, norm, stream)


class ReduceRMSNorm:
    """Unquantized fused reduce + residual-add + RMSNorm over R bf16 partials [rows, H] (TokenWeave)."""

    def __init__(self, parts: list, rows: int, H: int, gamma, out, residual=None, residual_out=None, eps=1e-5):
        self.R, self.rows, self.H = len(parts), rows, H
        self._parts = (C.c_void_p * self.R)(*[_lib._dev(p, 2 * rows * H, "part") for p in parts])
        self._keep = list(parts)  # the table holds raw addresses: keep the tensors allocated with it
        self.norm = _norm_args(gamma, out, residual, residual_out, eps, H, rows * H)

    def run(self, max_workgroups: int = 0, stream=None):
        st = _lib.lib.fc_reduce_rmsnorm(self._parts, self.R, self.rows, C.byref(self.norm), max_workgroups,
                                        _lib._stream(stream))
        _lib._check(st, "fc_reduce_rmsnorm")


class LLUnpackReduce:
    """Receiver of R ranks' epoch-tagged slot buffers (flash-comm self-synchronizing blocks)."""

    def __init__(self, slots: list, n: int, block_slots: int, out, stale, done, counters):
        self.R, self.n, self.B = len(slots), n, block_slots
        nblk = n // 2 // block_slots
        self._slots = (C.c_void_p * self.R)(*[_lib._dev(s, 4 * n, "slots") for s in slots])
        self._ptrs = (_lib._dev(out, 2 * n, "out"), _lib._dev(stale, self.R * nblk, "stale"),
                      _lib._dev(done, nblk, "done"), _lib._dev(counters, _lib.COUNTER_BYTES, "counters"))
        self._keep = (list(slots), out, stale, done, counters)  # raw addresses above: keep the tensors

    def run(self, epoch: int, stream=None):
        st = _lib.lib.fc_ll_unpack_reduce(self._slots, self.R, self.n, self.B, epoch & 0xFFFFFFFF, *self._ptrs,
                                          _lib._stream(stream))
        _lib._check(st, "fc_ll_unpack_reduce")


class SelfSyncReduce:
    """Receive side of a one-shot all-reduce whose R inbound messages carry their own readiness evidence
    (flash-comm, abstract), in the encoding the protocol selector picks for the message size and rank
    count ("auto"), or a given one ("ll", "flag512", "flag2048", "flag8192").

    inbox(): the buffers the R senders write (rank r's slots, or payload + flag words);
    send(): emulates the R senders in one launch (the peers' writes, on one GPU);
    begin(): clears done flags and counters for a new epoch; receive(): folds every block whose R copies
    carry the epoch, in ascending rank order, into out (bf16 [n]); with max_polls > 0 the receiver waits
    (bounded) for late blocks, so it may run while the senders still write.  The inbox starts zero-filled,
    so epochs start at 1 and each message takes a new one (epoch 0 is refused)."""

    def __init__(self, R: int, n: int, encoding: str = "auto", costs=None, device="cuda"):
        from . import selector as sel
        ok = {e for e in sel.ENCODINGS
              if (n % (2 * sel.LL_BLOCK_SLOTS) == 0 if e == "ll" else n % sel.flag_block(e) == 0)}
        if encoding == "auto":
            if not ok:
                raise ValueError(f"n={n} fits no encoding's block size")
            encoding = sel.select(costs if costs is not None else sel.load(), 2 * n, R, allowed=ok)
        elif encoding not in ok:
            raise ValueError(f"encoding {encoding!r} does not divide n={n}")
        self.R, self.n, self.encoding = R, n, encoding
        if encoding == "ll":
            self.B = sel.LL_BLOCK_SLOTS
            self.nblk = n // 2 // self.B
            self.slots = [torch.zeros(n // 2, dtype=torch.int64, device=device) for _ in range(R)]
        else:
            self.B = sel.flag_block(encoding)
            self.nblk = n // self.B
            self.payload = [torch.zeros(n, dtype=torch.int16, device=device) for _ in range(R)]
            self.flags = [torch.zeros(self.nblk, dtype=torch.int32, device=device) for _ in range(R)]
        self.out = torch.zeros(n, dtype=torch.int16, device=device)
        self.stale = torch.zeros(R * self.nblk, dtype=torch.uint8, device=device)
        self.done = torch.zeros(self.nblk, dtype=torch.uint8, device=device)
        self.counters = torch.zeros(_lib.COUNTER_WORDS, dtype=torch.int32, device=device)

    def inbox(self):
        return self.slots if self.encoding == "ll" else (self.payload, self.flags)

    def begin(self, stream=None):
        """stream: a torch stream (or None for the current one); the clears are fill kernels."""
        import contextlib
        with torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext():
            self.done.zero_()
            self.counters.zero_()

    @staticmethod
    def _check_epoch(epoch: int) -> None:
        if not 0 < epoch < (1 << 32):
            raise ValueError(f"epoch {epoch}: the zero-filled inbox already carries 0; use 1 .. 2^32-1")

    def send(self, xs, epoch: int, block_order=None, pace: int = 0, stream=None):
        self._check_epoch(epoch)
        if self.encoding == "ll":
            _lib.fc_ll_pack(list(xs), self.B, epoch, self.slots, block_order=block_order, pace=pace, stream=stream)
        else:
            _lib.fc_flag_pack(list(xs), self.B, epoch, self.payload, self.flags, block_order=block_order, pace=pace,
                              stream=stream)

    def receive(self, epoch: int, max_polls: int = 0, max_workgroups: int = 0, stream=None):
        self._check_epoch(epoch)
        if self.encoding == "ll":
            _lib.fc_ll_poll_unpack_reduce(self.slots, self.n, self.B, epoch, self.out, self.stale, self.done,
                                          self.counters, max_polls=max_polls, max_workgroups=max_workgroups,
                                          stream=stream)
        else:
            _lib.fc_flag_unpack_reduce(self.payload, self.flags, self.n, self.B, epoch, self.out, self.stale,
                                       self.done, self.counters, max_polls=max_polls,
                                       max_workgroups=max_workgroups, stream=stream)
