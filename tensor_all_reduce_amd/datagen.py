"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and by the CPU oracle.

This module holds none of the method's arithmetic: it only draws random numbers and rounds them to
bf16 bit patterns.  Both sides of every parity check receive the identical arrays it returns.

The pages measure on real LLM inference (LLaMA-3-70B prefill and decoding; "multiple models and
workloads"); no weights or activations are available here, so seeded stand-ins of the same shapes and
value structure are used: Gaussian partial sums with rare large outliers (activation outliers are what
make per-group low-bit quantization non-trivial), a Gaussian residual stream and a near-one RMSNorm
weight.

Generator: numpy PCG64 with ``SeedSequence([0xFC, idx, purpose, rank])``, idx being the workload's number
(``Config.idx``); purposes are listed in
``PURPOSE``.  A partial is sigma*N(0,1) in fp32, multiplied by ``outlier_factor`` where an i.i.d.
Bernoulli(``outlier_p``) mask is set, then rounded to bf16 with ties to even.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PURPOSE = dict(values=0, outliers=1, residual=2, gamma=3, stale_mask=4, stale_values=5, permutation=6, gemm=7,
               flag_mask=8, flag_values=9)


@dataclass(frozen=True)
class Config:
    """One workload.  ``kind`` is 'two_step' (quantized RS/AG + RMSNorm), 'll' (epoch-tagged slots) or
    'rmsnorm' (unquantized fused reduce + residual-add + RMSNorm)."""
    idx: int
    name: str
    kind: str
    R: int
    T: int
    H: int
    sigma: float = 1.0
    outlier_p: float = 0.0
    outlier_factor: float = 1.0
    bits_rs: int = 8
    bits_ag: int = 8
    group: int = 128
    eps: float = 1e-5
    block_slots: int = 64
    stale_p: float = 0.0
    epoch: int = 0x2A
    splits: tuple = field(default_factory=tuple)
    slug: str = ""

    @property
    def n(self) -> int:
        return self.T * self.H

    @property
    def L(self) -> int:
        return self.n // self.R


# The five workloads (shapes of Llama-3-8B / Llama-3-70B hidden sizes; see module docstring).  ``idx`` is
# part of every generator's seed.
TINY = Config(1, "tiny R=2 T=4 H=256 int8 G=32", "two_step", R=2, T=4, H=256, sigma=1.0, outlier_p=0.01,
              outlier_factor=20.0, bits_rs=8, bits_ag=8, group=32, slug="tiny-r2-t4-h256")
DECODE_8B = Config(2, "llama3-8b decode R=8 T=64 H=4096 int8 G=128", "two_step", R=8, T=64, H=4096, sigma=0.5,
                   outlier_p=0.005, outlier_factor=30.0, bits_rs=8, bits_ag=8, group=128, slug="llama3-8b-decode")
PREFILL_70B = Config(3, "llama3-70b tp8 prefill R=8 T=4096 H=8192 int4-RS/int8-AG G=128", "two_step", R=8,
                     T=4096, H=8192, sigma=1.0, outlier_p=0.001, outlier_factor=50.0, bits_rs=4, bits_ag=8,
                     group=128, slug="llama3-70b-prefill")
SLOTS = Config(4, "self-synchronizing slots R=8 T=128 H=8192 B=64 2% stale", "ll", R=8, T=128, H=8192, sigma=1.0,
               block_slots=64, stale_p=0.02, slug="self-sync-slots")
TOKENWEAVE = Config(5, "tokenweave split R=8 T=8192(4096+4096) H=8192 bf16", "rmsnorm", R=8, T=8192, H=8192,
                    sigma=1.0, splits=(4096, 4096), slug="tokenweave-split")
# by name (slug), in this order
WORKLOADS = {c.slug: c for c in (TINY, DECODE_8B, PREFILL_70B, SLOTS, TOKENWEAVE)}


def rng_for(cfg: int, purpose: str, rank: int = 0, salt: int = 0) -> np.random.Generator:
    words = [0xFC, int(cfg), PURPOSE[purpose], int(rank)] + ([int(salt)] if salt else [])
    return np.random.default_rng(np.random.SeedSequence(words))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 bit patterns, ties to even (input preparation only; finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    return ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def partial(cfg: Config, rank: int, n: int | None = None) -> np.ndarray:
    """Rank `rank`'s bf16 partial sum, flat [T*H] (or the first n elements of the same stream)."""
    n = cfg.n if n is None else n
    v = rng_for(cfg.idx, "values", rank).standard_normal(n, dtype=np.float32)
    if cfg.sigma != 1.0:
        v *= np.float32(cfg.sigma)
    if cfg.outlier_p > 0:
        m = rng_for(cfg.idx, "outliers", rank).random(n, dtype=np.float32) < cfg.outlier_p
        v[m] *= np.float32(cfg.outlier_factor)
    return f32_to_bf16_bits(v)


def partials(cfg: Config) -> list[np.ndarray]:
    return [partial(cfg, r) for r in range(cfg.R)]


def residual(cfg: Config, n: int | None = None) -> np.ndarray:
    n = cfg.n if n is None else n
    return f32_to_bf16_bits(rng_for(cfg.idx, "residual").standard_normal(n, dtype=np.float32))


def gamma(cfg: Config) -> np.ndarray:
    g = rng_for(cfg.idx, "gamma").standard_normal(cfg.H, dtype=np.float32) * np.float32(0.1) + np.float32(1.0)
    return f32_to_bf16_bits(g)


# ---- epoch-tagged slot workloads --------------------------------------------------------------------------
# How a stale (rank, block) copy looks to the receiver.  Most are the previous round's epoch; the rest
# cover the other ways a word can differ from the expected epoch.
STALE_KINDS = ("prev", "zero", "next", "not", "msb", "random", "torn")
STALE_WEIGHTS = (0.70, 0.05, 0.05, 0.05, 0.05, 0.05, 0.05)


def write_order(cfg: Config, rank: int, nblk: int) -> np.ndarray:
    """The seeded order in which rank `rank` writes its blocks (arrival order emulation)."""
    return rng_for(cfg.idx, "permutation", rank).permutation(nblk).astype(np.int32)


def stale_epochs(cfg: Config, rank: int, nslots: int, epoch: int | None = None,
                 p: float | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Per-slot epoch words as rank `rank`'s blocks are seen by the receiver, and the per-block stale mask.

    Returns (epochs uint32 [nslots], stale uint8 [nblk]).  Slots of valid blocks carry `epoch`."""
    e = int(cfg.epoch if epoch is None else epoch) & 0xFFFFFFFF
    M = 0xFFFFFFFF
    p = cfg.stale_p if p is None else p
    B = cfg.block_slots
    nblk = nslots // B
    stale = (rng_for(cfg.idx, "stale_mask", rank).random(nblk) < p).astype(np.uint8)
    ep = np.full(nslots, e, np.uint32)
    rv = rng_for(cfg.idx, "stale_values", rank)
    idx = np.nonzero(stale)[0]
    kinds = rv.choice(len(STALE_KINDS), size=idx.size, p=STALE_WEIGHTS)
    for b, k in zip(idx, kinds):
        sl = slice(b * B, (b + 1) * B)
        kind = STALE_KINDS[k]
        if kind == "prev":
            ep[sl] = (e - 1) & M
        elif kind == "zero":
            ep[sl] = 0 if e != 0 else 1
        elif kind == "next":
            ep[sl] = (e + 1) & M
        elif kind == "not":
            ep[sl] = (~e) & M
        elif kind == "msb":
            ep[sl] = e ^ 0x80000000
        elif kind == "random":
            r = rv.integers(0, 2**32, size=B, dtype=np.uint64).astype(np.uint32)
            r[r == e] = e ^ 1
            ep[sl] = r
        else:  # torn: one slot of the block not yet written
            ep[b * B + int(rv.integers(0, B))] = (e - 1) & M
    return ep, stale


FLAG_KINDS = ("prev", "zero", "next", "not", "msb", "random")
FLAG_WEIGHTS = (0.75, 0.05, 0.05, 0.05, 0.05, 0.05)


def stale_flags(cfg: Config, rank: int, nblk: int, epoch: int | None = None, p: float | None = None,
                salt: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Per-block flag words of rank `rank` as the receiver sees them, and the stale mask.

    Returns (flags uint32 [nblk], stale uint8 [nblk]).  A valid block's flag carries `epoch`; a stale one
    carries one of the wrong words of FLAG_KINDS (a flag word is one store, so it cannot be torn)."""
    e = int(cfg.epoch if epoch is None else epoch) & 0xFFFFFFFF
    M = 0xFFFFFFFF
    p = cfg.stale_p if p is None else p
    stale = (rng_for(cfg.idx, "flag_mask", rank, salt).random(nblk) < p).astype(np.uint8)
    fl = np.full(nblk, e, np.uint32)
    rv = rng_for(cfg.idx, "flag_values", rank, salt)
    idx = np.nonzero(stale)[0]
    kinds = rv.choice(len(FLAG_KINDS), size=idx.size, p=FLAG_WEIGHTS)
    wrong = {"prev": (e - 1) & M, "zero": 0 if e != 0 else 1, "next": (e + 1) & M, "not": (~e) & M,
             "msb": e ^ 0x80000000}
    for b, k in zip(idx, kinds):
        kind = FLAG_KINDS[k]
        if kind == "random":
            r = int(rv.integers(0, 2**32, dtype=np.uint64))
            fl[b] = r if r != e else e ^ 1
        else:
            fl[b] = wrong[kind]
    return fl, stale


def _seed_words(seed) -> list[int]:
    """Flatten an int or a nested tuple of ints into seed words."""
    if isinstance(seed, (tuple, list)):
        out = []
        for s in seed:
            out += _seed_words(s)
        return out
    return [int(seed)]


def synth_bf16(seed, n: int, sigma: float = 1.0, outlier_p: float = 0.0, outlier_factor: float = 1.0) -> np.ndarray:
    """Seeded bf16 bits of an arbitrary test shape, same recipe as `partial` (seed: int or tuple of ints)."""
    rng = np.random.default_rng(np.random.SeedSequence([0xFC, 0xEE] + _seed_words(seed)))
    v = rng.standard_normal(n, dtype=np.float32) * np.float32(sigma)
    if outlier_p > 0:
        m = rng.random(n, dtype=np.float32) < outlier_p
        v[m] *= np.float32(outlier_factor)
    return f32_to_bf16_bits(v)


def synth_f32(seed, n: int, sigma: float = 1.0) -> np.ndarray:
    """Seeded fp32 values (stand-ins for fp32 partial sums, e.g. requantization inputs)."""
    rng = np.random.default_rng(np.random.SeedSequence([0xFC, 0xEF] + _seed_words(seed)))
    return rng.standard_normal(n, dtype=np.float32) * np.float32(sigma)


def adversarial_groups(group: int, seed: int = 0) -> np.ndarray:
    """bf16 bits of groups built to hit the quantizer's edge cases: constant groups, signed zeros, fp16
    subnormal-range values (zero-point not an fp16 value), values at the top of the fp16 range, exact
    half-step ties on a power-of-two grid, one huge outlier among tiny values, all-negative groups, and
    values below the fp16 subnormals with a negative minimum."""
    rng = np.random.default_rng(np.random.SeedSequence([0xFC, 0xAD, seed]))
    G = group
    gs = []
    gs.append(np.full(G, 1.5, np.float32))
    gs.append(np.full(G, -0.0, np.float32))
    z = np.zeros(G, np.float32)
    z[::2] = -0.0
    gs.append(z)
    gs.append((rng.standard_normal(G) * 3e-6).astype(np.float32))
    gs.append(np.full(G, 9.6112489700317383e-07, np.float32))
    top = rng.choice([-65280.0, 65280.0, 32768.0, -1.0], size=G).astype(np.float32)
    gs.append(top)
    k = rng.integers(0, 16, size=G).astype(np.float32)
    tie = k + 0.5
    tie[0], tie[1] = 0.0, 15.0
    gs.append(tie.astype(np.float32))
    o = (rng.standard_normal(G) * 1e-3).astype(np.float32)
    o[G // 3] = 6.0e4
    gs.append(o)
    gs.append(-np.abs(rng.standard_normal(G)).astype(np.float32) - 2.0)
    gs.append(np.linspace(-1, 1, G).astype(np.float32))
    # below half the smallest fp16 subnormal, with a negative minimum: its nearest fp16 is -0, and the
    # zero-point steps down from there to the negative subnormal
    tiny = np.full(G, -1e-9, np.float32)
    tiny[1::2] = 3e-9
    gs.append(tiny)
    return f32_to_bf16_bits(np.concatenate(gs))
