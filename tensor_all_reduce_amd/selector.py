"""Cost-guided choice of the readiness encoding (flash-comm, abstract: a protocol selector adapts the
readiness encoding to the message size and the number of participating GPUs, balancing the cost of
synchronization against the extra bytes an encoding sends).

Encodings built here:

  "ll"        8-byte slots, 4 payload bytes + 4 epoch bytes: twice the payload bytes on the wire, and no
              fence anywhere: a slot is valid when its epoch word is.
  "flag<B>"   the payload unchanged plus one 4-byte flag word per block of B bf16 elements; the sender
              fences (release) before each flag store, the receiver reads the flag, fences (acquire),
              then reads the block: fewer bytes, one synchronization per block and a dependent read.

Model (the plainest reading of the trade the selector makes): the latency of one transfer of S payload
bytes from each of R ranks is the larger of a synchronization floor and a transfer time,

    t(enc, S, R) = max(a + b * R,  d + (c * R + e) * wire(enc, S))

where wire() is the bytes one rank sends.  a + b R is what the encoding costs however small the message
(launch, readiness checks, for a flag the dependent flag-then-payload read).  The transfer time has a
term for the bytes all R ranks move through the shared memory system (c R wire) and one for the bytes of
a single rank (e wire): each rank's message is written and checked in order of its own blocks and spans
whatever R is, which is why a flag encoding's latency grows with the message far more than with R.  c
and e also carry a flag encoding's per-block fence (a block is a fixed number of bytes, so blocks and
bytes cannot be told apart within one encoding).  The five non-negative coefficients are fitted per
encoding to latencies measured with a sender and a receiver running at the same time, minimising the
relative error.  ``select`` returns the encoding with the lowest predicted latency (ties: the listed
order).  Host logic only; ``python -m tensor_all_reduce_amd.selector --refit FILE`` refits a table's
coefficients from the latencies it stores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
from dataclasses import dataclass

DEFAULT_TABLE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "encoding_costs.json")
ENCODINGS = ("ll", "flag512", "flag2048", "flag8192")
LL_BLOCK_SLOTS = 64  # slot block of the "ll" encoding


def flag_block(enc: str) -> int:
    """Block elements of a "flag<B>" encoding."""
    if not enc.startswith("flag"):
        raise ValueError(f"not a flag encoding: {enc}")
    return int(enc[4:])


def wire_bytes(enc: str, S: int) -> int:
    """Bytes one rank sends to carry S payload bytes (bf16 elements, S even)."""
    if enc == "ll":
        return 2 * S
    return S + 4 * math.ceil(S / 2 / flag_block(enc))


def blocks(enc: str, S: int) -> int:
    """Blocks one rank publishes (each one a readiness decision of the receiver)."""
    if enc == "ll":
        return math.ceil(S / 4 / LL_BLOCK_SLOTS)
    return math.ceil(S / 2 / flag_block(enc))


@dataclass(frozen=True)
class EncodingCost:
    enc: str
    coef: tuple  # (a us, b us per rank, c us per wire byte and rank, d us, e us per wire byte)

    def predict(self, S: int, R: int) -> float:
        a, b, c, d, e = self.coef
        return max(a + b * R, d + (c * R + e) * wire_bytes(self.enc, S))


def fit(rows) -> dict[str, EncodingCost]:
    """rows: iterable of (enc, S, R, t_us), t_us > 0.  Per encoding, non-negative coefficients minimising
    the relative error (the choice compares latencies at one size, so a microsecond matters as much at
    10 us as a hundred at 1 ms), from several starting points (the max makes the problem non-convex)."""
    import numpy as np
    from scipy.optimize import least_squares
    by = {}
    for enc, S, R, t in rows:
        by.setdefault(enc, []).append((float(R), float(wire_bytes(enc, S)), float(t)))
    out = {}
    for enc, pts in by.items():
        R = np.array([p[0] for p in pts])
        w = np.array([p[1] for p in pts])
        t = np.array([p[2] for p in pts])
        # unit steps of comparable size for the five coefficients
        scale = np.array([t.min(), t.min(), t.max() / (R * w).max(), t.min(), t.max() / w.max()])

        def resid(q):
            a, b, c, d, e = q * scale
            return np.maximum(a + b * R, d + (c * R + e) * w) / t - 1.0
        best = None
        for x0 in ((1.0, 0.1, 1.0, 0.1, 0.1), (0.5, 0.05, 0.5, 0.5, 0.5), (1.0, 0.0, 2.0, 0.0, 0.0),
                   (0.8, 0.2, 1.0, 1.0, 1.0), (1.0, 0.1, 0.1, 0.1, 2.0)):
            r = least_squares(resid, x0=np.array(x0), bounds=(0.0, np.inf))
            if best is None or r.cost < best.cost:
                best = r
        out[enc] = EncodingCost(enc, tuple(float(v) for v in best.x * scale))
    return out


def select(costs: dict[str, EncodingCost], S: int, R: int, allowed=None) -> str:
    """The encoding with the lowest predicted latency for S payload bytes per rank and R ranks."""
    names = [e for e in ENCODINGS if e in costs and (allowed is None or e in allowed)]
    if not names:
        raise ValueError("no encoding to choose from")
    return min(names, key=lambda e: (costs[e].predict(S, R), names.index(e)))


def crossover(costs: dict[str, EncodingCost], R: int, lo: int = 1 << 10, hi: int = 1 << 30) -> list:
    """[(S, encoding)] at each payload size (powers of two from lo to hi) where the choice changes."""
    out, prev = [], None
    S = lo
    while S <= hi:
        e = select(costs, S, R)
        if e != prev:
            out.append((S, e))
            prev = e
        S *= 2
    return out


def regret(costs: dict[str, EncodingCost], rows) -> dict:
    """How much the choice of `costs` loses against the fastest encoding measured, over the (S, R) points of
    `rows` ((enc, S, R, t_us) tuples) where every encoding was measured: the number of points, how many
    chose the fastest, and the mean and largest loss in % of the fastest latency.  Scoring a stored table
    on latencies it was not fitted to tells how well it carries to another run or machine."""
    pts = {}
    for enc, S, R, t in rows:
        pts.setdefault((int(S), int(R)), {})[enc] = float(t)
    losses, hits = [], 0
    for (S, R), meas in sorted(pts.items()):
        if any(e not in meas for e in ENCODINGS if e in costs):
            continue
        best = min(meas.values())
        t = meas[select(costs, S, R, allowed=set(meas))]
        hits += t == best
        losses.append(100.0 * (t / best - 1.0))
    if not losses:
        return {"points": 0, "fastest": 0, "mean_pct": None, "max_pct": None}
    return {"points": len(losses), "fastest": hits, "mean_pct": round(sum(losses) / len(losses), 2),
            "max_pct": round(max(losses), 2)}


MODEL = "t_us = max(a + b*R, d + (c*R + e)*wire_bytes); coefficients [a, b, c, d, e]"


def save(path: str, costs: dict[str, EncodingCost], measured, command: str, machine: str) -> None:
    doc = {"model": MODEL, "command": command, "machine": machine,
           "coefficients": {e: list(c.coef) for e, c in costs.items()},
           "measured": [list(r) for r in measured]}
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


def load(path: str = DEFAULT_TABLE) -> dict[str, EncodingCost]:
    """A table's coefficients.  A table of the earlier four-coefficient model (no per-rank term) reads
    with e = 0."""
    with open(path) as f:
        doc = json.load(f)
    out = {}
    for e, c in doc["coefficients"].items():
        c = tuple(float(v) for v in c)
        if len(c) == 4:
            c = c + (0.0,)
        if len(c) != 5:
            raise ValueError(f"{path}: {e} has {len(c)} coefficients")
        out[e] = EncodingCost(e, c)
    return out


def refit(path: str) -> dict[str, EncodingCost]:
    """Refit a table's coefficients from the latencies it stores and rewrite it (its measurement command
    and machine kept)."""
    with open(path) as f:
        doc = json.load(f)
    rows = [tuple(r) for r in doc["measured"]]
    costs = fit(rows)
    save(path, costs, rows, doc["command"], doc["machine"])
    return costs


if __name__ == "__main__":
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--refit", metavar="FILE", required=True, help="table to refit from its stored latencies")
    args = ap.parse_args()
    for enc, c in refit(args.refit).items():
        print(enc, ["%.6g" % v for v in c.coef])
