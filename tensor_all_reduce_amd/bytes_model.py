"""Algorithmic HBM bytes of each call: every input read once and every output written once, at its
stored width (bf16 2 B, codes bits/8 B, one 4-byte meta word per group, 8-byte slots).  The RMSNorm
weight gamma counts once per call.  These are the bytes a kernel cannot avoid moving; achieved GB/s =
these bytes / measured time."""
from __future__ import annotations


def quantize(n: int, bits: int, group: int) -> dict:
    return dict(read=2 * n, write=n * bits // 8 + 4 * (n // group))


def reduce_shard(R: int, L: int, bits_in: int, bits_out: int, group: int, n_shards: int) -> dict:
    return dict(read=n_shards * R * (L * bits_in // 8 + 4 * (L // group)),
                write=n_shards * (L * bits_out // 8 + 4 * (L // group)))


def gather(R: int, L: int, bits: int, group: int, hidden: int, plain: bool, norm: bool, residual: bool,
           residual_out: bool) -> dict:
    n = R * L
    rd = R * (L * bits // 8 + 4 * (L // group))
    wr = 0
    if plain:
        wr += 2 * n
    if norm:
        rd += 2 * hidden + (2 * n if residual else 0)
        wr += 2 * n + (2 * n if residual_out else 0)
    return dict(read=rd, write=wr)


def reduce_rmsnorm(R: int, rows: int, hidden: int, residual: bool, residual_out: bool) -> dict:
    n = rows * hidden
    return dict(read=2 * R * n + 2 * hidden + (2 * n if residual else 0),
                write=2 * n + (2 * n if residual_out else 0))


def ll_unpack(R: int, n: int, block_slots: int, completed_blocks: int | None = None) -> dict:
    """Slots read once per rank (4 B per element: half payload, half epoch word), done flags read, stale
    flags and done flags written, output written for the blocks completed (all of them by default)."""
    nblk = n // 2 // block_slots
    done_b = nblk if completed_blocks is None else completed_blocks
    return dict(read=R * 4 * n + nblk, write=2 * 2 * block_slots * done_b + R * nblk + done_b)


def total(d: dict) -> int:
    return d["read"] + d["write"]


def two_step_whole(R, T, H, bits_rs, bits_ag, group, residual=True, residual_out=True) -> dict:
    """The whole emulated all-reduce on one GPU: every rank's quantize, every shard's reduce, one gather +
    epilogue of the result."""
    n = T * H
    L = n // R
    q = quantize(R * n, bits_rs, group)
    r = reduce_shard(R, L, bits_rs, bits_ag, group, R)
    g = gather(R, L, bits_ag, group, H, plain=False, norm=True, residual=residual, residual_out=residual_out)
    return dict(quantize=q, reduce_shard=r, gather_norm=g)


def two_step_share(R, T, H, bits_rs, bits_ag, group, residual=True, residual_out=True) -> dict:
    """One GPU's real share: its own quantize, its own shard's reduce (R chunks in, one shard out), the
    gather + epilogue of all R shards."""
    n = T * H
    L = n // R
    q = quantize(n, bits_rs, group)
    r = reduce_shard(R, L, bits_rs, bits_ag, group, 1)
    g = gather(R, L, bits_ag, group, H, plain=False, norm=True, residual=residual, residual_out=residual_out)
    return dict(quantize=q, reduce_shard=r, gather_norm=g)


def reduce_norm(R: int, L: int, bits_in: int, bits_out: int, group: int, n_shards: int, hidden: int,
                residual: bool = True, residual_out: bool = True) -> dict:
    """The reduce with the norm first: R quantized chunks per shard in, the shard's residual rows and
    gamma in; the quantized normalized rows and residual_out out."""
    n = n_shards * L
    return dict(read=n_shards * R * (L * bits_in // 8 + 4 * (L // group)) + 2 * hidden + (2 * n if residual else 0),
                write=n_shards * (L * bits_out // 8 + 4 * (L // group)) + (2 * n if residual_out else 0))


def two_step_normfirst_whole(R, T, H, bits_rs, bits_ag, group) -> dict:
    """Norm before the all-gather, the whole emulated all-reduce: every rank's quantize, every shard's
    reduce + norm + quantization, the gather of the normalized rows to bf16."""
    n = T * H
    L = n // R
    return dict(quantize=quantize(R * n, bits_rs, group),
                reduce_shard=reduce_norm(R, L, bits_rs, bits_ag, group, R, H),
                gather=gather(R, L, bits_ag, group, H, plain=True, norm=False, residual=False, residual_out=False))


def two_step_normfirst_share(R, T, H, bits_rs, bits_ag, group) -> dict:
    """Norm before the all-gather, one GPU's real share: its quantize, its shard's reduce + norm, the
    gather of all R normalized shards."""
    n = T * H
    L = n // R
    return dict(quantize=quantize(n, bits_rs, group),
                reduce_shard=reduce_norm(R, L, bits_rs, bits_ag, group, 1, H),
                gather=gather(R, L, bits_ag, group, H, plain=True, norm=False, residual=False, residual_out=False))


def ll_gather(R: int, nwords: int, block_slots: int, completed_blocks: int | None = None) -> dict:
    """Standalone all-gather on epoch-tagged blocks: every rank's slots read once (8 B per payload word:
    4 payload, 4 epoch), done flags read, payload words written for the (rank, block) pairs completed (all
    by default), stale and done flags written."""
    nblk = R * (nwords // block_slots)
    done_b = nblk if completed_blocks is None else completed_blocks
    return dict(read=R * 8 * nwords + nblk, write=4 * block_slots * done_b + nblk + done_b)


def flag_unpack(R: int, n: int, block_elems: int) -> dict:
    """Receiver of the flag encoding with every block valid: each rank's payload (2 B per element) and flag
    words read, done flags read, the output and the stale and done flags written."""
    nblk = n // block_elems
    return dict(read=R * 2 * n + R * 4 * nblk + nblk, write=2 * n + R * nblk + nblk)
