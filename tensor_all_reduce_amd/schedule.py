"""Token splitting and the two-half pipelined layer schedule (TokenWeave, abstract: the batch is split
into two wave-aware token subsets, and one subset's all-reduce + RMSNorm overlaps the other's compute).

Host-side scheduling only: the GEMMs are torch.matmul calls (a library contraction), the all-reduce +
RMSNorm of a half is fc_reduce_rmsnorm; nothing here computes on the host.

Wave-aware split.  The pages give no rule; the reading implemented here: a half of T_h rows runs a GEMM
[T_h, K] x [K, N] whose output is cut into tiles of tile_m x tile_n, ceil(T_h / tile_m) * ceil(N / tile_n)
of them, executed in waves of `cus` tiles (one tile per compute unit).  The split T1 is a multiple of
tile_m with both halves non-empty that minimises the total number of waves of the two halves; among
equal totals the one nearest T/2, then the lower one.  At T = 8192, N = 8192, 256 x 256 tiles and 256
compute units this gives 4096 / 4096.  Fewer than 2 * tile_m rows are not split (T1 = T).
"""
from __future__ import annotations

import math


def gemm_waves(rows: int, n: int, tile_m: int = 256, tile_n: int = 256, cus: int = 256) -> int:
    """Waves of a GEMM with `rows` output rows and `n` output columns (0 rows: 0 waves)."""
    if rows <= 0:
        return 0
    tiles = math.ceil(rows / tile_m) * math.ceil(n / tile_n)
    return math.ceil(tiles / cus)


def wave_aware_split(T: int, n: int, tile_m: int = 256, tile_n: int = 256, cus: int = 256) -> int:
    """Rows of the first half (see the module docstring); T when T < 2 * tile_m."""
    if T < 2 * tile_m:
        return T
    best = None
    for t1 in range(tile_m, T, tile_m):
        key = (gemm_waves(t1, n, tile_m, tile_n, cus) + gemm_waves(T - t1, n, tile_m, tile_n, cus),
               abs(2 * t1 - T), t1)
        if best is None or key < best:
            best = key
    return best[2]


class TwoHalfLayer:
    """One tensor-parallel layer step of one rank, split into two token halves and pipelined on two streams:

        stream c:  GEMM(A) -> GEMM(B)
        stream r:            all-reduce + RMSNorm(A) -> all-reduce + RMSNorm(B)

    A's all-reduce waits for GEMM(A) only, so it overlaps GEMM(B); B's waits for GEMM(B).  The GEMM of a half
    writes this rank's bf16 partial for its rows; the other R - 1 ranks' partials (on one GPU: buffers
    filled by the caller) complete the all-reduce.  Rows are independent, so the output equals the same two
    halves run one after the other on one stream, bit for bit.

    x: bf16 [T, K] activations; w: bf16 [K, H]; peers: R - 1 int16 (bf16 bits) [T, H] partials of the other
    ranks; residual, gamma, out, residual_out as for fc_reduce_rmsnorm (whole [T, H] tensors)."""

    def __init__(self, x, w, peers, residual, gamma, out, residual_out=None, eps: float = 1e-5, t1: int | None = None,
                 max_workgroups: int = 0, tile_m: int = 256, tile_n: int = 256, cus: int = 256):
        import torch
        from .flash_allreduce import ReduceRMSNorm
        T, K = x.shape
        H = w.shape[1]
        self.T, self.H = T, H
        self.t1 = wave_aware_split(T, H, tile_m, tile_n, cus) if t1 is None else t1
        self.x, self.w = x, w
        self.partial = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)  # this rank's GEMM output
        self.mw = max_workgroups
        self.halves = []
        for lo, hi in ((0, self.t1), (self.t1, T)):
            if hi <= lo:
                continue
            mine = self.partial[lo:hi].view(torch.int16).reshape(-1)
            parts = [mine] + [p.reshape(T, H)[lo:hi].reshape(-1) for p in peers]
            sl = slice(lo * H, hi * H)
            ar = ReduceRMSNorm(parts, hi - lo, H, gamma, out.reshape(-1)[sl],
                               residual=residual.reshape(-1)[sl] if residual is not None else None,
                               residual_out=residual_out.reshape(-1)[sl] if residual_out is not None else None, eps=eps)
            self.halves.append((lo, hi, ar))

    def _gemm(self, lo, hi):
        import torch
        torch.matmul(self.x[lo:hi], self.w, out=self.partial[lo:hi])

    def run(self, stream_c, stream_r):
        """Enqueue the pipelined step on two streams; returns the event that ends it (on stream_r)."""
        import torch
        done = []
        for lo, hi, _ in self.halves:
            with torch.cuda.stream(stream_c):
                self._gemm(lo, hi)
                ev = torch.cuda.Event()
                ev.record(stream_c)
            done.append(ev)
        for (lo, hi, ar), ev in zip(self.halves, done):
            stream_r.wait_event(ev)
            ar.run(max_workgroups=self.mw, stream=stream_r)
        end = torch.cuda.Event()
        end.record(stream_r)
        return end

    def run_serial(self, stream):
        """The same halves one after the other on one stream (the reference order)."""
        import torch
        with torch.cuda.stream(stream):
            for lo, hi, ar in self.halves:
                self._gemm(lo, hi)
                ar.run(max_workgroups=self.mw, stream=stream)
