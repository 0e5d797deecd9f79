"""Mutation check of the CPU oracle's pins.

Each entry of MUTANTS is a plausible mistake in ``oracle/fc_oracle.cpp`` (a wrong rounding direction, a
reversed fold, a dropped term, an off-by-one, a wrong comparison, ...), given as a piece of the source and
its altered text.  For each one this script writes an altered copy of the oracle to a scratch directory,
points the oracle loader at it (``FC_ORACLE_SRC``) and runs the oracle's pin tests; the pins are good
enough when every altered oracle fails at least one of them.

    python tests/mutation_check.py            # every mutant, in parallel; exit status 1 if one survives
    python tests/mutation_check.py -k fold    # the mutants whose name contains "fold"

It builds the oracle once per mutant (g++, a few seconds each) and is not part of the pytest suite;
``tests/test_mutation_list.py`` keeps the list in step with the source and runs one mutant end to end.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fc_oracle.cpp")
PIN_TESTS = ["test_oracle_formats.py", "test_oracle_quant.py", "test_oracle_allreduce.py", "test_oracle_ll.py",
             "test_oracle_ll_gather.py", "test_oracle_flag.py", "test_oracle_normfirst.py"]

# (name, original text, altered text): the original must occur exactly once in the oracle's source.
MUTANTS: list[tuple[str, str, str]] = [
    # number formats
    ("rne: ties away from zero",
     "double r = std::nearbyint(q); // default rounding mode: to nearest, ties to even",
     "double r = std::floor(q + 0.5);"),
    ("rne: no subnormal quantum",
     "if (binade < f.emin) binade = f.emin;  // subnormal range has the quantum of the smallest binade",
     ""),
    ("round-down: zero steps up",
     "if ((h & 0x7fffu) == 0) h = 0x8001u;            // +-0 -> -2^-24",
     "if ((h & 0x7fffu) == 0) h = 0x0001u;"),
    ("round-down: positive grows",
     "else h = (uint16_t)(h - 1u);                    // positive: shrink the magnitude",
     "else h = (uint16_t)(h + 1u);"),
    ("round-up: negative grows",
     "else if (h & 0x8000u) h = (uint16_t)(h - 1u);   // negative: shrink the magnitude",
     "else if (h & 0x8000u) h = (uint16_t)(h + 1u);"),
    ("bf16: truncation",
     "inline uint16_t bf16_rne(float x) { return (uint16_t)to_fmt_rne(x, kBF16); }",
     "inline uint16_t bf16_rne(float x) { return (uint16_t)(f32_to_bits(x) >> 16); }"),
    # quantizer
    ("quantize: no -0 canonicalisation",
     "lo = lo + 0.0f;  // -0 becomes +0",
     "lo = lo;  //"),
    ("quantize: zero-point to nearest",
     "m.zero = f16_rd(lo);",
     "m.zero = f16_rne(lo);"),
    ("quantize: scale to nearest",
     "m.scale = f16_ru(t);",
     "m.scale = f16_rne(t);"),
    ("quantize: qmax off by one",
     "const int qmax = (1 << bits) - 1;",
     "const int qmax = (1 << bits);"),
    ("quantize: codes round half up",
     "float r = std::nearbyint(v);  // ties to even",
     "float r = std::floor(v + 0.5f);"),
    ("quantize: constant group gets scale 1",
     "m.scale = 0;\n        inv = 0.0f;",
     "m.scale = 0x3c00;\n        inv = 1.0f;"),
    ("quantize: reciprocal of the unrounded scale",
     "const float s = f16_val(m.scale);\n        inv = 1.0f / s;",
     "inv = 1.0f / t;"),
    # codes and dequantization
    ("dequant: sign of the zero-point",
     "const float p = (float)q * s;\n    return p + z;",
     "const float p = (float)q * s;\n    return p - z;"),
    ("codes: nibbles swapped on read",
     "return (i & 1) ? (uint32_t)(b >> 4) : (uint32_t)(b & 0x0fu);",
     "return (i & 1) ? (uint32_t)(b & 0x0fu) : (uint32_t)(b >> 4);"),
    ("dequant: wrong group's meta",
     "y[i] = dequant_one(get_code(codes, i, bits), unpack_meta(meta[i / group]));",
     "y[i] = dequant_one(get_code(codes, i, bits), unpack_meta(meta[i / (2 * group)]));"),
    # reduce-scatter
    ("reduce: descending fold",
     "float acc = dequant_one(get_code(codes[0], i, bits_in), unpack_meta(meta[0][i / group]));\n"
     "        for (int r = 1; r < R; ++r) {",
     "float acc = dequant_one(get_code(codes[R - 1], i, bits_in), unpack_meta(meta[R - 1][i / group]));\n"
     "        for (int r = R - 2; r >= 0; --r) {"),
    ("reduce: last rank dropped",
     "for (int r = 1; r < R; ++r) {\n            const float d = dequant_one(",
     "for (int r = 1; r < R - 1; ++r) {\n            const float d = dequant_one("),
    ("reduce: requantizes the bf16-rounded sums",
     "if (out_codes && out_meta) quantize_f32(S.data(), L, bits_out, group, out_codes, out_meta);",
     "for (auto& v : S) v = bf16_val(bf16_rne(v));\n"
     "    if (out_codes && out_meta) quantize_f32(S.data(), L, bits_out, group, out_codes, out_meta);"),
    ("two-step: wrong rank's chunk",
     "cin[r] = codes1 + r * c1 + s * (L * bits1 / 8);\n            min_[r] = meta1 + r * g1 + s * (L / group);\n"
     "        }\n        or_reduce_shard(",
     "cin[r] = codes1 + ((r + s) % R) * c1 + s * (L * bits1 / 8);\n"
     "            min_[r] = meta1 + ((r + s) % R) * g1 + s * (L / group);\n        }\n        or_reduce_shard("),
    # RMSNorm epilogue
    ("rmsnorm: eps outside the root",
     "const float ms = ss / (float)hidden;\n    const float rinv = 1.0f / std::sqrt(ms + eps);\n"
     "    for (int64_t j = 0; j < hidden; ++j) {\n        const float a = hbuf[j] * rinv;\n        const float b",
     "const float ms = ss / (float)hidden;\n    const float rinv = 1.0f / (std::sqrt(ms) + eps);\n"
     "    for (int64_t j = 0; j < hidden; ++j) {\n        const float a = hbuf[j] * rinv;\n        const float b"),
    ("rmsnorm: mean over H - 1",
     "const float ss = sumsq_seq(hbuf, hidden);\n    const float ms = ss / (float)hidden;",
     "const float ss = sumsq_seq(hbuf, hidden);\n    const float ms = ss / (float)(hidden - 1);"),
    ("rmsnorm: gamma before the inverse root",
     "const float a = hbuf[j] * rinv;\n        const float b = a * bf16_val(gamma[j]);",
     "const float a = hbuf[j] * bf16_val(gamma[j]);\n        const float b = a * rinv;"),
    ("rmsnorm: residual subtracted",
     "uint16_t* out, uint16_t* residual_out, float* hbuf) {\n    for (int64_t j = 0; j < hidden; ++j) {\n"
     "        float h = y[j];\n        if (residual) h = h + bf16_val(residual[j]);",
     "uint16_t* out, uint16_t* residual_out, float* hbuf) {\n    for (int64_t j = 0; j < hidden; ++j) {\n"
     "        float h = y[j];\n        if (residual) h = h - bf16_val(residual[j]);"),
    ("rmsnorm: residual_out before the add",
     "for (int64_t j = 0; j < hidden; ++j) residual_out[j] = bf16_rne(hbuf[j]);\n    const float ss = sumsq_seq(",
     "for (int64_t j = 0; j < hidden; ++j) residual_out[j] = bf16_rne(y[j]);\n    const float ss = sumsq_seq("),
    ("rmsnorm: fused squares",
     "const float sq = h[j] * h[j];\n        ss = ss + sq;",
     "ss = std::fma(h[j], h[j], ss);"),
    # norm before the all-gather
    ("norm first: orders swapped",
     "const float ss = order == 1 ? sumsq_tree(hbuf, hidden) : sumsq_seq(hbuf, hidden);",
     "const float ss = order == 1 ? sumsq_seq(hbuf, hidden) : sumsq_tree(hbuf, hidden);"),
    ("norm first: tree without padding",
     "while (m < nch) m *= 2;",
     "m = nch;"),
    ("norm first: fused chunk fold",
     "const float sq = h[8 * c + e] * h[8 * c + e];\n            p = p + sq;",
     "p = std::fma(h[8 * c + e], h[8 * c + e], p);"),
    ("norm first: normalized values rounded to bf16",
     "o[j] = a * bf16_val(gamma[j]);",
     "o[j] = bf16_val(bf16_rne(a * bf16_val(gamma[j])));"),
    ("norm first: wrong shard's residual",
     "residual ? residual + s * L : nullptr,",
     "residual ? residual + ((s + 1) % R) * L : nullptr,"),
    # unquantized reduce + RMSNorm
    ("reduce + rmsnorm: last rank dropped",
     "for (int r = 1; r < R; ++r) acc = acc + bf16_val(parts[r][i]);\n        y[i] = acc;",
     "for (int r = 1; r < R - 1; ++r) acc = acc + bf16_val(parts[r][i]);\n        y[i] = acc;"),
    # slots
    ("slots: pack swaps a pair",
     "slots[k] = (uint64_t)x[2 * k] | ((uint64_t)x[2 * k + 1] << 16)",
     "slots[k] = (uint64_t)x[2 * k + 1] | ((uint64_t)x[2 * k] << 16)"),
    ("slots: epoch compared with <",
     "if ((uint32_t)(slots[r][k] >> 32) != epoch) st = true;\n            stale[(int64_t)r * nblk + b]",
     "if ((uint32_t)(slots[r][k] >> 32) < epoch) st = true;\n            stale[(int64_t)r * nblk + b]"),
    ("slots: last slot not checked",
     "for (int64_t k = b * block_slots; k < (b + 1) * block_slots; ++k)\n"
     "                if ((uint32_t)(slots[r][k] >> 32) != epoch) st = true;\n            stale[(int64_t)r * nblk + b]",
     "for (int64_t k = b * block_slots; k < (b + 1) * block_slots - 1; ++k)\n"
     "                if ((uint32_t)(slots[r][k] >> 32) != epoch) st = true;\n            stale[(int64_t)r * nblk + b]"),
    ("slots: done blocks not skipped",
     "if (done[b]) continue;\n        bool all_valid = true;\n        for (int r = 0; r < R; ++r) {\n            bool st",
     "bool all_valid = true;\n        for (int r = 0; r < R; ++r) {\n            bool st"),
    ("slots: pending not counted",
     "if (!all_valid) { counters[1] += 1; continue; }\n        for (int64_t k = b * block_slots;",
     "if (!all_valid) { continue; }\n        for (int64_t k = b * block_slots;"),
    ("slots: elements of a slot swapped",
     "out[2 * k + e] = bf16_rne(acc);",
     "out[2 * k + (1 - e)] = bf16_rne(acc);"),
    ("slots: valid ranks of a stale block reduced",
     "if (!all_valid) { counters[1] += 1; continue; }\n        for (int64_t k = b * block_slots;",
     "if (!all_valid) { counters[1] += 1; }\n        for (int64_t k = b * block_slots;"),
    # flag words
    ("flags: epoch compared with <",
     "const bool st = flags[r][b] != epoch;",
     "const bool st = flags[r][b] < epoch;"),
    ("flags: stale copies folded",
     "if (!all_valid) { counters[1] += 1; continue; }\n        for (int64_t i = b * block_elems;",
     "if (!all_valid) { counters[1] += 1; }\n        for (int64_t i = b * block_elems;"),
    ("flags: descending fold",
     "float acc = bf16_val(payload[0][i]);\n            for (int r = 1; r < R; ++r) acc = acc + bf16_val(payload[r][i]);",
     "float acc = bf16_val(payload[R - 1][i]);\n            for (int r = R - 2; r >= 0; --r) acc = acc + bf16_val(payload[r][i]);"),
    # standalone all-gather
    ("all-gather: epoch compared with <",
     "if ((uint32_t)(slots[r][k] >> 32) != epoch) st = true;\n            stale[f]",
     "if ((uint32_t)(slots[r][k] >> 32) < epoch) st = true;\n            stale[f]"),
    ("all-gather: stale blocks copied",
     "counters[1] += 1;\n                continue;\n            }",
     "counters[1] += 1;\n            }"),
    ("all-gather: done blocks not skipped",
     "if (done[f]) continue;",
     ""),
    ("all-gather: pending not counted",
     "counters[0] += 1;\n                counters[1] += 1;\n                continue;",
     "counters[0] += 1;\n                continue;"),
    ("all-gather: last slot not checked",
     "for (int64_t k = b * block_slots; k < (b + 1) * block_slots; ++k)\n"
     "                if ((uint32_t)(slots[r][k] >> 32) != epoch) st = true;\n            stale[f]",
     "for (int64_t k = b * block_slots; k < (b + 1) * block_slots - 1; ++k)\n"
     "                if ((uint32_t)(slots[r][k] >> 32) != epoch) st = true;\n            stale[f]"),
]

# Mutants that no pin can tell from the oracle, with the reason; they are run and reported, and do not
# count as failures of the pins.
EQUIVALENT = {
    "rmsnorm: gamma before the inverse root":
        "only the order of two fp32 products changes: the result moves by at most one fp32 ulp before the "
        "bf16 rounding, within the one bf16 ulp the epilogue's pins allow against double precision (and "
        "the two-ulp bar of the GPU parity tests); no closed form or invariant separates the two orders",
}


def mutate(source: str, old: str, new: str) -> str:
    if source.count(old) != 1:
        raise ValueError(f"the text to alter occurs {source.count(old)} times, not once: {old[:60]!r}")
    return source.replace(old, new)


def run_one(name: str, old: str, new: str, timeout: float = 600.0) -> tuple[str, bool, str]:
    """Build the altered oracle and run the pins; returns (name, killed, the first failing test or why)."""
    with open(SRC) as fh:
        text = mutate(fh.read(), old, new)
    tmp = tempfile.mkdtemp(prefix="fc_mutant_")
    try:
        path = os.path.join(tmp, "fc_oracle.cpp")
        with open(path, "w") as fh:
            fh.write(text)
        env = dict(os.environ, FC_ORACLE_SRC=path)
        env.pop("FC_SANITIZE", None)
        cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
               *[os.path.join(ROOT, "tests", t) for t in PIN_TESTS]]
        r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
        if r.returncode == 0:
            return name, False, "every pin passed"
        failed = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED") or ln.startswith("ERROR")]
        return name, True, failed[0] if failed else f"pytest exit status {r.returncode}"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("-k", default="", help="only the mutants whose name contains this text")
    ap.add_argument("-j", type=int, default=min(6, os.cpu_count() or 1), help="parallel builds and test runs")
    args = ap.parse_args()
    todo = [m for m in MUTANTS if args.k in m[0]]
    with open(SRC) as fh:
        text = fh.read()
    for name, old, new in todo:
        mutate(text, old, new)  # every mutant applies before any is run
    survivors, equivalent = [], []
    with cf.ThreadPoolExecutor(max_workers=args.j) as ex:
        for name, killed, why in ex.map(lambda m: run_one(*m), todo):
            if killed:
                print(f"killed    {name}: {why}", flush=True)
            elif name in EQUIVALENT:
                equivalent.append(name)
                print(f"survived  {name} (equivalent: {EQUIVALENT[name]})", flush=True)
            else:
                survivors.append(name)
                print(f"SURVIVED  {name}: {why}", flush=True)
    killed = len(todo) - len(survivors) - len(equivalent)
    print(f"{killed} of {len(todo)} mutants killed, {len(equivalent)} equivalent, {len(survivors)} survived",
          flush=True)
    return 1 if survivors else 0


if __name__ == "__main__":
    sys.exit(main())
