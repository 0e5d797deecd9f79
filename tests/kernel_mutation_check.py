"""Mutation check of the GPU parity tests.

Each entry of MUTANTS is a plausible arithmetic mistake in one of the HIP kernels (a rounding direction,
a dropped correction step, a swapped operand, an intermediate rounding, a sign, a weaker readiness
test), given as a piece of a source file under ``tensor_all_reduce_amd/csrc`` and its altered text, with
the GPU test files that should catch it.  No mutant changes an address, an index, a bound or a wait: each
computes wrong values in the same memory footprint, so running it is as safe as running the library.

    python tests/kernel_mutation_check.py build DIR   # on any machine with hipcc: one library per mutant
    python tests/kernel_mutation_check.py run DIR     # on the GPU: each mutant's tests must fail

``build`` writes DIR/<mutant>/libfc.so; ``run`` loads each through FC_LIB_PATH and runs its tests with
pytest (-x: the first failure ends a mutant's run); it exits with status 1 if a mutant passes its tests.
``tests/test_kernel_mutation_list.py`` keeps the list in step with the sources.
"""
from __future__ import annotations

import argparse
import os
import re
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tensor_all_reduce_amd", "csrc")

# (name, source file, original text, altered text, GPU test files): the original occurs exactly once.
MUTANTS: list[tuple[str, str, str, str, list[str]]] = [
    ("zero-point rounded to nearest", "fc_device.h",
     "    return f16_to_f32(h) > v ? ((h & 0x8000u) ? h + 1u : h - 1u) : h;",
     "    return h;",
     ["test_gpu_quant.py"]),
    ("scale rounded to nearest", "fc_device.h",
     "    return f16_to_f32(h) < v ? h + 1u : h;",
     "    return h;",
     ["test_gpu_quant.py"]),
    ("reciprocal of the scale without its correction step", "fc_device.h",
     "    return __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);",
     "    return r0;",
     ["test_gpu_quant.py", "test_gpu_two_step.py"]),
    ("range / qmax without its correction step", "fc_device.h",
     "    return __builtin_fmaf(__builtin_fmaf(-q0, (float)QMAX, x), r, q0);",
     "    return q0;",
     ["test_gpu_quant.py", "test_gpu_two_step.py"]),
    ("-0 minimum kept", "fc_device.h",
     "    lo = lo + 0.0f;  // -0 -> +0",
     "",
     ["test_gpu_quant.py", "test_gpu_two_step.py"]),
    ("4-bit dequantization scales swapped", "fc_device.h",
     "            const float sk = (k & 1) ? s20 : s24;",
     "            const float sk = (k & 1) ? s24 : s20;",
     ["test_gpu_two_step.py"]),
    ("reduce-scatter sums rounded to bf16 before the requantization", "fc_twostep.hip",
     "    quantize_lane<B2, E, LPG>(acc, w, m);",
     "    for (int e = 0; e < E; ++e) acc[e] = bf16_lo(pack_bf16x2(acc[e], 0.0f));\n"
     "    quantize_lane<B2, E, LPG>(acc, w, m);",
     ["test_gpu_two_step.py"]),
    ("epilogue: eps outside the root", "fc_twostep.hip",
     "        const float rinv = 1.0f / sqrtf(ms + na.eps);",
     "        const float rinv = 1.0f / (sqrtf(ms) + na.eps);",
     ["test_gpu_two_step.py", "test_gpu_rmsnorm.py", "test_gpu_eps_rows.py"]),
    ("epilogue: residual subtracted", "fc_twostep.hip",
     "                for (int e = 0; e < 8; ++e) h[k][e] = h[k][e] + rv[e];",
     "                for (int e = 0; e < 8; ++e) h[k][e] = h[k][e] - rv[e];",
     ["test_gpu_two_step.py", "test_gpu_rmsnorm.py"]),
    ("unquantized reduce rounds each partial sum to bf16", "fc_twostep.hip",
     "                        for (int e = 0; e < 8; ++e) y[e] = y[e] + v[e];",
     "                        for (int e = 0; e < 8; ++e) y[e] = bf16_lo(pack_bf16x2(y[e] + v[e], 0.0f));",
     ["test_gpu_rmsnorm.py"]),
    ("norm first: fused squares in the chunk fold", "fc_twostep.hip",
     "                const float sq = h[8 * c + e] * h[8 * c + e];\n                q = q + sq;",
     "                q = __builtin_fmaf(h[8 * c + e], h[8 * c + e], q);",
     ["test_gpu_normfirst.py"]),
    ("slot receiver checks only the first slot of each lane's pair", "fc_slots.hip",
     "        const uint64_t bal = (__ballot(q[k].y != epoch) | __ballot(q[k].w != epoch)) & amask[k];",
     "        const uint64_t bal = __ballot(q[k].y != epoch) & amask[k];",
     ["test_gpu_ll.py"]),
    ("all-gather checks only the first slot of each lane's pair", "fc_slots.hip",
     "        const uint64_t bal = (__ballot(v[k].y != epoch) | __ballot(v[k].w != epoch)) & amask[k];",
     "        const uint64_t bal = __ballot(v[k].y != epoch) & amask[k];",
     ["test_gpu_ll_gather.py"]),
    ("flag receiver takes a later epoch for the expected one", "fc_live.hip",
     "            uint64_t bad = __ballot(watch && f != epoch);",
     "            uint64_t bad = __ballot(watch && f < epoch);",
     ["test_gpu_live.py"]),
]


def slug(name: str) -> str:
    return re.sub(r"[^a-z0-9]+", "_", name.lower()).strip("_")


def mutate(text: str, old: str, new: str) -> str:
    if text.count(old) != 1:
        raise ValueError(f"the text to alter occurs {text.count(old)} times, not once: {old[:60]!r}")
    return text.replace(old, new)


def build(out: str, only: str = "") -> None:
    sys.path.insert(0, ROOT)
    from tensor_all_reduce_amd import build as b
    for name, src, old, new, _ in MUTANTS:
        if only not in name:
            continue
        d = os.path.join(out, slug(name))
        shutil.rmtree(d, ignore_errors=True)
        shutil.copytree(CSRC, os.path.join(d, "csrc"))
        path = os.path.join(d, "csrc", src)
        with open(path) as fh:
            text = mutate(fh.read(), old, new)
        with open(path, "w") as fh:
            fh.write(text)
        b.build(csrc=os.path.join(d, "csrc"), lib=os.path.join(d, "libfc.so"), build_dir=os.path.join(d, "obj"))
        print(f"built  {name}", flush=True)


def run(out: str, only: str = "", timeout: float = 300.0) -> int:
    survivors = []
    for name, _, _, _, tests in MUTANTS:
        if only not in name:
            continue
        lib = os.path.join(out, slug(name), "libfc.so")
        env = dict(os.environ, FC_LIB_PATH=lib)
        cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "gpu", "-p", "no:cacheprovider", "--timeout",
               str(int(timeout)), "--timeout-method", "thread", *[os.path.join(ROOT, "tests", t) for t in tests]]
        print(f"mutant {name}: {' '.join(tests)}", flush=True)
        r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout + 60)
        failed = [ln for ln in r.stdout.splitlines() if ln.startswith(("FAILED", "ERROR"))]
        if r.returncode == 0:
            survivors.append(name)
            print("  SURVIVED: every test passed", flush=True)
        elif r.returncode == 1 and failed:
            print(f"  caught: {failed[0][:160]}", flush=True)
        else:  # anything else (a crash, a collection error) is reported and ends the run
            print(f"  pytest exit status {r.returncode}; output tail:\n{r.stdout[-1500:]}\n{r.stderr[-1500:]}",
                  flush=True)
            return 2
    print(f"{len(survivors)} mutant(s) survived" + (": " + "; ".join(survivors) if survivors else ""), flush=True)
    return 1 if survivors else 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("what", choices=["build", "run"])
    ap.add_argument("dir")
    ap.add_argument("-k", default="", help="only the mutants whose name contains this text")
    args = ap.parse_args()
    if args.what == "build":
        build(args.dir, args.k)
        return 0
    return run(args.dir, args.k)


if __name__ == "__main__":
    sys.exit(main())
