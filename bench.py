#!/usr/bin/env python
"""Benchmark of one MI355X's share of the flash all-reduce, on synthetic inputs already resident in HBM.

Headline step (`value`): the whole emulated quantized all-reduce of the Llama-3-8B decode workload (8
ranks x [64, 4096] bf16, int8 groups of 128) on one GPU: every rank's group quantization (one launch),
every shard's fixed-order dequant-reduce-requant (one launch) and the all-gather dequantize with the
fused residual-add + RMSNorm epilogue (one launch).  Steps are replayed from a HIP graph, each on its own
buffer set; the sets together exceed twice the 256 MB last-level cache, so inputs come from HBM.
value = algorithmic bytes per step / time per step (GB/s).

The other hot-path rows are measured at their own workloads and reported under "rows": the 70B prefill
two-step path (int4 reduce-scatter / int8 all-gather), one GPU's real share of both two-step workloads
(its own quantize, one shard's reduce, the gather), the variant with the norm applied to each shard before
the all-gather (whole path and one GPU's share), the standalone all-gather on epoch-tagged blocks, the
self-synchronizing slot receiver (first pass
with late blocks, then the retry), and the unquantized reduce-RMSNorm on two wave-aware half batches,
alone and overlapped with a bf16 GEMM on a second stream, with a workgroup-cap sweep, and the two-half pipelined layer step (wave-aware split, each half's
all-reduce overlapping the other half's GEMM).

Prints one JSON line.  --gpus N > 1 is refused: everything runs on one GPU.
`python bench.py --pmc-summary FETCH_CSV WRITE_CSV OUT` turns two rocprofv3 --pmc runs into the traffic
summary that later runs report, and `--profile-report` writes a workload's whole profile summary (see
profiles/).
"""
import argparse
import csv
import hashlib
import re
import json
import math
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused quant-reduce-RMSNorm effective GB/s (% HBM peak) + µs per call"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
KERNEL_SOURCES = ["tensor_all_reduce_amd/csrc/fc_twostep.hip", "tensor_all_reduce_amd/csrc/fc_device.h"]
PROFILES = os.path.join(ROOT, "profiles")


def traffic_file(slug):
    return os.path.join(PROFILES, f"pmc_traffic_{slug}.txt")


def kernel_of_call(call, cfg):
    """Substring naming the kernel instantiation a call launches for this workload."""
    return {"quantize": f"k_quantize<{cfg.bits_rs}, {cfg.group},",
            "reduce_shard": f"k_reduce<{cfg.bits_rs}, {cfg.bits_ag}, {cfg.group},",
            "gather_norm": f"k_rows<fc::GatherProducer<{cfg.bits_ag},"}[call]


DEFAULT_ROWS = "decode,share,normfirst,ll,llgather,rmsnorm,layer,encodings"
ALL_ROWS = DEFAULT_ROWS + ",warm"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 200 on the prefill, 600 else)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps before them (default: as many)")
    ap.add_argument("--config", default="llama3-70b-prefill",
                    choices=["tiny-r2-t4-h256", "llama3-8b-decode", "llama3-70b-prefill"],
                    help="headline two-step workload (default: the 70B prefill shard, the largest of the metric)")
    ap.add_argument("--warm", action="store_true", help="reuse one buffer set (cache-resident)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--oracle-by-config", action="store_true",
                    help="also time the oracle on every workload (a detail line; about a minute of CPU)")
    ap.add_argument("--rows", default="default",
                    help=f"other hot-path rows: default ({DEFAULT_ROWS}) | all (adds warm) | none | comma list")
    ap.add_argument("--detail-out", metavar="JSON", help="also write every row's full record to this file")
    ap.add_argument("--kernel-reps", type=int, default=0, help="graph replays per call timing (0 = auto)")
    ap.add_argument("--fit-encodings", metavar="JSON", help="write the selector's fitted cost table here")
    ap.add_argument("--pmc-rows", metavar="BYTES_JSON", help="only launch the row kernels for counter runs")
    ap.add_argument("--rows-pmc-report", nargs=5, metavar=("STATS_CSV", "FETCH_CSV", "WRITE_CSV", "BYTES_JSON", "OUT_MD"))
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT"))
    ap.add_argument("--stats-table", nargs=4, metavar=("STATS_CSV", "OUT_MD", "TITLE", "COMMAND"))
    ap.add_argument("--profile-report", nargs=6, metavar=("WORKLOAD", "STATS_CSV", "FETCH_CSV", "WRITE_CSV", "VALU_CSV",
                                                          "OUT_MD"))
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 200 if args.config == "llama3-70b-prefill" else 600
    if args.warmup is None:
        # the prefill step runs up to 10% slower over its first ~80 replayed steps on fresh buffers: as
        # many warm-up steps as timed ones keep that transient out of the timed region
        args.warmup = args.steps
    return args


def _code_text(text: str) -> str:
    """Source text without comments, blank lines and trailing blanks: what a compiler sees of it."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    lines = []
    for line in text.splitlines():
        # the first // outside a string literal starts a comment
        cut = line.find("//")
        while cut >= 0 and line.count('"', 0, cut) % 2 == 1:
            cut = line.find("//", cut + 2)
        if cut >= 0:
            line = line[:cut]
        line = line.rstrip()
        if line.strip():
            lines.append(line)
    return "\n".join(lines)


def sources_sha(files=None) -> str:
    """Hash of kernel sources (default: those of the two-step kernels) with their comments stripped,
    recorded with counter summaries: counters taken before a change to the code stop being reported, a
    change to a comment keeps them."""
    h = hashlib.sha256()
    for f in files or KERNEL_SOURCES:
        path = f if "/" in f else os.path.join(ROOT, "tensor_all_reduce_amd", "csrc", f)
        with open(path if os.path.isabs(path) else os.path.join(ROOT, path), encoding="utf-8") as fh:
            h.update(_code_text(fh.read()).encode())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------------------------------------
# HBM traffic from hardware counters
# ---------------------------------------------------------------------------------------------------------
def pmc_summary(fetch_csv, write_csv, out_path):
    """Median FETCH_SIZE and WRITE_SIZE per kernel (KiB per dispatch), scaled by what the same counters
    read for the 1 GiB copy kernel (whose true traffic is 1 GiB each way)."""
    def load(path, counter):
        d = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                d.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: statistics.median(v) for k, v in d.items()}
    f, w = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    copy = next(k for k in f if "k_copy" in k)
    fs, ws = (1 << 20) / f[copy], (1 << 20) / w[copy]
    lines = [f"# HBM traffic per launch from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE (separate runs)",
             f"# scale factors from the 1 GiB copy kernel: fetch x{fs:.4f}, write x{ws:.4f}",
             f"sources_sha {sources_sha()}"]
    for k in sorted(f):
        if not k.startswith(("fc::", "void fc::")):
            continue
        lines.append(f"kernel {round(f[k] * fs * 1024)} {round(w.get(k, 0.0) * ws * 1024)} {k}")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _rp_out(csv_path):
    """The rocprofv3 output options (-d DIR -o NAME) that wrote `csv_path` (DIR/NAME_<table>.csv)."""
    d, f = os.path.split(csv_path)
    for table in ("_kernel_stats.csv", "_counter_collection.csv"):
        if f.endswith(table):
            return f"-d {d} -o {f[:-len(table)]}"
    raise ValueError(f"{csv_path}: not a rocprofv3 kernel-stats or counter-collection table")


def profile_report(config, stats_csv, fetch_csv, write_csv, valu_csv, out_md):
    """The profile summary of one two-step workload (profiles/two_step_<slug>.md) from four rocprofv3 runs of
    the benchmark: --kernel-trace --stats, then --pmc FETCH_SIZE, --pmc WRITE_SIZE and
    --pmc SQ_INSTS_VALU SQ_WAVES, each in a run of its own.  Also writes the traffic summary that later
    benchmark runs report (profiles/pmc_traffic_<slug>.txt)."""
    from tensor_all_reduce_amd import bytes_model as bm, datagen as dg
    cfg = dg.WORKLOADS[config]
    pmc_summary(fetch_csv, write_csv, traffic_file(cfg.slug))
    calls = bm.two_step_whole(cfg.R, cfg.T, cfg.H, cfg.bits_rs, cfg.bits_ag, cfg.group)
    keys = {call: kernel_of_call(call, cfg) for call in calls}

    def call_of(name):
        return next((c for c, k in keys.items() if k in name), None)

    def short(name):
        return name.replace("void ", "").split("(")[0]
    stats = list(csv.DictReader(open(stats_csv)))
    pmc = {}
    for path in (fetch_csv, write_csv, valu_csv):
        for r in csv.DictReader(open(path)):
            pmc.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    med = {k: statistics.median(v) for k, v in pmc.items()}
    traffic = load_traffic(cfg)
    headline = cfg is dg.PREFILL_70B  # the default workload
    runs = "" if headline else f" --config {config}"  # the default steps and warm-up of the benchmark
    x = " --steps 4 --warmup 1 --kernel-reps 1" if headline else f" --config {config} --steps 290 --warmup 0 --kernel-reps 1"
    base = "python3 bench.py --no-cpu-baseline --rows none"
    lines = [f"# Two-step all-reduce kernels on the {cfg.name} workload", "",
             "Kernel durations from a rocprofv3 kernel trace of the benchmark (run from the repository root on one "
             "MI355X; the benchmark replays each call from HIP graphs over cold buffer sets):", "", "```",
             f"rocprofv3 --kernel-trace --stats --output-format csv {_rp_out(stats_csv)} -- {base}{runs}",
             "```", "", "| kernel | calls | avg us | min us | max us | algorithmic bytes | GB/s at avg |",
             "|---|---|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"]
        c = call_of(name)
        by = bm.total(calls[c]) if c else (2 << 30 if "k_copy" in name else None)
        if by is None:
            continue
        avg = float(r["AverageNs"]) / 1e3
        lines.append(f"| `{short(name)}` | {r['Calls']} | {avg:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {by} | {by / (avg * 1e-6) / 1e9:.0f} |")
    lines += ["", "(`k_copy` is the 1 GiB copy-ceiling kernel of the benchmark: 2 GiB moved per call.  Durations "
              "under the tracer run longer than the graph-timed figures the benchmark reports.)", "",
              "HBM traffic per launch from two counter runs (FETCH_SIZE, then WRITE_SIZE), scaled by what the same "
              "counters read for the 1 GiB copy kernel, and vector-ALU instructions per wavefront and per byte "
              f"from a third run (kernel sources {sources_sha()}):", "", "```"]
    for ctr, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv), ("SQ_INSTS_VALU SQ_WAVES", valu_csv)):
        lines.append(f"timeout -s KILL 240 rocprofv3 --pmc {ctr} --output-format csv {_rp_out(path)} -- {base}{x}")
    lines += ["```", "", f"Summarised with `python bench.py --profile-report {config} STATS FETCH WRITE VALU {out_md}`.",
              "", "| kernel | fetch bytes | algorithmic read | write bytes | algorithmic write | VALU instr / wavefront "
              "| VALU instr / algorithmic byte (per wavefront lane-op: x64) |", "|---|---|---|---|---|---|---|"]
    for name in sorted({k for k, _ in med}):
        c = call_of(name)
        if not c:
            continue
        tr = traffic_for(c, cfg, traffic) or {}
        a = calls[c]
        v, w = med.get((name, "SQ_INSTS_VALU")), med.get((name, "SQ_WAVES"))
        vpw = f"{v / w:.0f}" if v and w else "-"
        vpb = f"{v / bm.total(a):.4f} ({64 * v / bm.total(a):.2f})" if v else "-"
        fb, wb = tr.get("fetch"), tr.get("write")
        lines.append(f"| `{short(name)}` | {fb} ({fb / a['read']:.3f}x) | {a['read']} | {wb} ({wb / a['write']:.3f}x) | "
                     f"{a['write']} | {vpw} | {vpb} |" if fb is not None else f"| `{short(name)}` | - | {a['read']} | - | "
                     f"{a['write']} | {vpw} | {vpb} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def pmc_rows(out_json):
    """Single-workload launches of the row kernels, for counter runs (one counter per run): the 1 GiB copy
    (the counters' scale reference), then per kernel a few launches over 3 rotating buffer sets (together
    larger than the L2s): the slot receiver's first pass on the slot workload, half A of the TokenWeave
    reduce + RMSNorm, the all-gather of the int8 prefill messages (first pass), the two f2 receivers
    (flag words per 2048 elements, polling slot receiver) on 8 x 2 MiB with every block there, and the
    reduce with the norm first on every shard of the 70B prefill.  Writes the
    algorithmic bytes of one launch of each kernel to `out_json`."""
    import numpy as np
    import torch
    from tensor_all_reduce_amd import _lib, bytes_model as bm, datagen as dg
    from tensor_all_reduce_amd.flash_allreduce import ReduceRMSNorm, rank_rows
    dev = torch.device("cuda:0")
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view({2: np.int16, 4: np.int32, 8: np.int64}[a.dtype.itemsize])).to(dev)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    _lib.fc_copy(src, dst)
    del src, dst
    algo = {}
    # slot receiver, first pass
    c4 = dg.SLOTS
    R, n, B, e = c4.R, c4.n, c4.block_slots, c4.epoch
    nslots, nblk = n // 2, n // 2 // B
    sets = []
    for k in range(3):
        slots = []
        for r, s_ in enumerate(rank_rows(R, nslots, torch.int64, dev)[1]):
            _lib.fc_ll_pack(up(dg.partial(c4, r)), B, e, s_, block_order=up(dg.write_order(c4, r, nblk)))
            s_.view(torch.int32).view(-1, 2)[:, 1] = up(dg.stale_epochs(c4, r, nslots)[0])
            slots.append(s_)
        sets.append(slots)
    out = torch.empty(n, dtype=torch.int16, device=dev)
    stale = torch.empty(R * nblk, dtype=torch.uint8, device=dev)
    done = torch.zeros(nblk, dtype=torch.uint8, device=dev)
    cnt = torch.zeros(_lib.COUNTER_WORDS, dtype=torch.int32, device=dev)
    for k in range(6):
        done.zero_()
        cnt.zero_()
        _lib.fc_ll_unpack_reduce(sets[k % 3], n, B, e, out, stale, done, cnt)
    torch.cuda.synchronize()
    pend = int(_lib.counter_totals(cnt)[1])
    algo["k_ll_unpack"] = bm.ll_unpack(R, n, B, completed_blocks=nblk - pend)
    del sets, out, stale, done, cnt
    # TokenWeave half A
    c5 = dg.TOKENWEAVE
    a = c5.splits[0]
    na = a * c5.H
    pbuf, parts = rank_rows(c5.R, na, torch.int16, dev)
    for r in range(c5.R):
        parts[r].copy_(up(dg.partial(c5, r, na)))
    res, gam = up(dg.residual(c5, na)), up(dg.gamma(c5))
    o5, ro5 = torch.empty(na, dtype=torch.int16, device=dev), torch.empty(na, dtype=torch.int16, device=dev)
    rr = ReduceRMSNorm(parts, a, c5.H, gam, o5, residual=res, residual_out=ro5, eps=c5.eps)
    for _ in range(3):
        rr.run()
    torch.cuda.synchronize()
    algo["BF16ReduceProducer"] = bm.reduce_rmsnorm(c5.R, a, c5.H, True, True)
    del parts, pbuf, res, o5, ro5, rr
    # all-gather of the int8 prefill messages, first pass
    c3 = dg.PREFILL_70B
    msg3 = c3.L * c3.bits_ag // 8 + 4 * (c3.L // c3.group)
    nwords = -(-msg3 // 4 // B) * B
    gblk = nwords // B
    gen = torch.Generator(device=dev)
    gen.manual_seed(0xFC0B)
    gsets = []
    for k in range(3):
        sl = []
        for r in range(c3.R):
            w = torch.randint(0, 1 << 32, (nwords,), dtype=torch.int64, device=dev, generator=gen)
            ep = torch.from_numpy(dg.stale_epochs(c4, r, nwords)[0].astype(np.int64)).to(dev)
            sl.append(w | (ep << 32))
        gsets.append(sl)
    gout = [torch.empty(nwords, dtype=torch.int32, device=dev) for _ in range(c3.R)]
    gst = torch.empty(c3.R * gblk, dtype=torch.uint8, device=dev)
    gdn = torch.zeros(c3.R * gblk, dtype=torch.uint8, device=dev)
    gcnt = torch.zeros(_lib.COUNTER_WORDS, dtype=torch.int32, device=dev)
    for k in range(6):
        gdn.zero_()
        gcnt.zero_()
        _lib.fc_ll_gather(gsets[k % 3], nwords, B, e, gout, gst, gdn, gcnt)
    torch.cuda.synchronize()
    gpend = int(_lib.counter_totals(gcnt)[1])
    algo["k_ll_gather"] = bm.ll_gather(c3.R, nwords, B, completed_blocks=c3.R * gblk - gpend)
    del gsets, gout
    # f2 receivers, every block there
    n2, be = 1 << 20, 2048
    xs = [up(dg.synth_bf16((0xF2, r), n2)) for r in range(8)]
    fsets, lsets = [], []
    for k in range(3):
        pays = [torch.empty(n2, dtype=torch.int16, device=dev) for _ in range(8)]
        fls = [torch.empty(n2 // be, dtype=torch.int32, device=dev) for _ in range(8)]
        _lib.fc_flag_pack(xs, be, 7, pays, fls)
        fsets.append((pays, fls))
        sl = [torch.empty(n2 // 2, dtype=torch.int64, device=dev) for _ in range(8)]
        _lib.fc_ll_pack(xs, 64, 7, sl)
        lsets.append(sl)
    out2 = torch.empty(n2, dtype=torch.int16, device=dev)
    st2 = torch.empty(8 * (n2 // 64), dtype=torch.uint8, device=dev)
    dn2 = torch.zeros(n2 // 64, dtype=torch.uint8, device=dev)
    c2 = torch.zeros(_lib.COUNTER_WORDS, dtype=torch.int32, device=dev)
    for k in range(6):
        dn2.zero_()
        _lib.fc_flag_unpack_reduce(*fsets[k % 3], n2, be, 7, out2, st2, dn2, c2)
    for k in range(6):
        dn2.zero_()
        _lib.fc_ll_poll_unpack_reduce(lsets[k % 3], n2, 64, 7, out2, st2, dn2, c2)
    torch.cuda.synchronize()
    algo["k_flag_unpack"] = bm.flag_unpack(8, n2, be)
    algo["k_ll_poll"] = bm.ll_unpack(8, n2, 64)
    del fsets, lsets, out2, st2, dn2, c2
    # the reduce with the norm first, every shard of the 70B prefill (int4 messages in, int8 rows out); the
    # counters do not depend on the values: random codes, scale 1/16 and zero 0 in every group
    R3, L3, G3, b13, b23 = c3.R, c3.L, c3.group, c3.bits_rs, c3.bits_ag
    qsets = []
    for k in range(3):
        ins = [(torch.randint(0, 256, (L3 * b13 // 8,), dtype=torch.uint8, device=dev, generator=gen),
                torch.full((L3 // G3,), 0x2C00, dtype=torch.int32, device=dev)) for _ in range(R3 * R3)]
        outs = [(torch.empty(L3 * b23 // 8, dtype=torch.uint8, device=dev),
                 torch.empty(L3 // G3, dtype=torch.int32, device=dev)) for _ in range(R3)]
        res3 = torch.randn(R3 * L3, device=dev, generator=gen).to(torch.bfloat16).view(torch.int16)
        qsets.append((ins, outs, res3, torch.empty_like(res3)))
    gam3 = up(dg.gamma(c3))
    for k in range(6):
        ins, outs, res3, rout3 = qsets[k % 3]
        _lib.fc_reduce_shard_norm(ins, R3, L3, b13, b23, G3,
                                  dict(residual=res3, gamma=gam3, eps=c3.eps, hidden=c3.H, residual_out=rout3), outs)
    torch.cuda.synchronize()
    algo["k_reduce_norm"] = bm.reduce_norm(R3, L3, b13, b23, G3, R3, c3.H)
    with open(out_json, "w") as f:
        json.dump(algo, f, indent=1)
    print(json.dumps(algo))


def rows_pmc_report(stats_csv, fetch_csv, write_csv, bytes_json, out_md):
    """Profile summary of the row kernels: durations and per-launch HBM traffic against algorithmic bytes."""
    algo = json.load(open(bytes_json))

    def load(path, counter):
        d = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                d.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: statistics.median(v) for k, v in d.items()}
    f, w = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    copy = next(k for k in f if "k_copy" in k)
    fs, ws = (1 << 30) / (f[copy] * 1024), (1 << 30) / (w[copy] * 1024)
    stats = {r["Name"]: r for r in csv.DictReader(open(stats_csv))}
    cmd = f"python3 bench.py --pmc-rows {bytes_json}"
    lines = ["# Row kernels: durations and HBM traffic per launch", "",
             "One workload per kernel, launched over 3 rotating buffer sets (together larger than the L2s), in "
             "four runs of the same command on one MI355X (run from the repository root, under /tmp as TMPDIR):", "",
             "```", f"rocprofv3 --kernel-trace --stats --output-format csv {_rp_out(stats_csv)} -- {cmd}",
             f"timeout -s KILL 240 rocprofv3 --pmc FETCH_SIZE --output-format csv {_rp_out(fetch_csv)} -- {cmd}",
             f"timeout -s KILL 240 rocprofv3 --pmc WRITE_SIZE --output-format csv {_rp_out(write_csv)} -- {cmd}",
             "```", "",
             f"Counters are scaled by what they read for the 1 GiB copy kernel (fetch x{fs:.4f}, write x{ws:.4f}); "
             f"summarised with `python bench.py --rows-pmc-report STATS FETCH WRITE BYTES_JSON {out_md}` "
             f"(kernel sources {sources_sha(('fc_slots.hip', 'fc_live.hip', 'fc_twostep.hip', 'fc_device.h', 'fc_sync.h'))}).", "",
             "| kernel | workload | avg us (traced) | fetch bytes | algorithmic read | write bytes | algorithmic write "
             "| GB/s at avg (algorithmic) |", "|---|---|---|---|---|---|---|---|"]
    what = {"k_ll_unpack": "slot workload, first pass (2% late)", "BF16ReduceProducer": "TokenWeave half A, 4096 rows",
            "k_ll_gather": "int8 prefill messages, first pass", "k_flag_unpack": "8 x 2 MiB, flag per 2048, all there",
            "k_ll_poll": "8 x 2 MiB slots, all there, no re-read",
            "k_reduce_norm": "norm first, 70B prefill, all 8 shards (int4 in, int8 out)"}
    for key, a in algo.items():
        name = next((k for k in f if key in k), None)
        if name is None:
            continue
        st = next((r for k, r in stats.items() if key in k), None)
        avg = float(st["AverageNs"]) / 1e3 if st else float("nan")
        fb, wb = round(f[name] * 1024 * fs), round(w.get(name, 0.0) * 1024 * ws)
        gbps = (a["read"] + a["write"]) / (avg * 1e-6) / 1e9
        lines.append(f"| `{name.replace('void ', '').split('(')[0]}` | {what[key]} | {avg:.2f} | {fb} ({fb / a['read']:.3f}x) "
                     f"| {a['read']} | {wb} ({wb / a['write']:.3f}x) | {a['write']} | {gbps:.0f} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def stats_table(stats_csv, out_md, title, command):
    """A kernel-duration table (rocprofv3 --kernel-trace --stats) of every library kernel in a run."""
    rows = sorted(csv.DictReader(open(stats_csv)), key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# {title}", "", "Kernel durations from a rocprofv3 kernel trace (run from the repository root on one "
             "MI355X; durations under the tracer run longer than the benchmark's graph-timed figures):", "",
             "```", command, "```", "", "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in rows:
        if "fc::" not in r["Name"]:
            continue
        lines.append(f"| `{r['Name'].replace('void ', '').split('(')[0]}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def load_traffic(cfg):
    """{kernel name: (fetch bytes, write bytes)} of this workload, if the summary was taken on the current
    kernel sources (else None: the counters no longer describe the kernels)."""
    path = traffic_file(cfg.slug)
    if not os.path.exists(path):
        return None
    sha, kern = None, {}
    for line in open(path):
        p = line.split()
        if not p or p[0].startswith("#"):
            continue
        if p[0] == "sources_sha":
            sha = p[1]
        elif p[0] == "kernel":
            kern[" ".join(p[3:])] = (int(p[1]), int(p[2]))
    return kern if sha == sources_sha() else None


def traffic_for(call, cfg, traffic):
    if not traffic:
        return None
    key = kernel_of_call(call, cfg)
    for name, (fb, wb) in traffic.items():
        if key in name:
            return {"fetch": fb, "write": wb, "total": fb + wb, "kernel": name}
    return None


# ---------------------------------------------------------------------------------------------------------
class one_core:
    """Pins this process to one host core (the third, if there are three) while the oracle is timed, so
    every oracle time is single-core whatever the host's scheduler does."""

    def __enter__(self):
        self.old = os.sched_getaffinity(0)
        cpus = sorted(self.old)
        self.core = cpus[min(2, len(cpus) - 1)]
        os.sched_setaffinity(0, {self.core})
        return self

    def __exit__(self, *exc):
        os.sched_setaffinity(0, self.old)
        return False


def cpu_baseline(cfg, seconds):
    """The oracle (single-threaded C++) on the same workload, pinned to one host core, whole steps
    repeated for about `seconds`."""
    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    import oracle
    from tensor_all_reduce_amd import bytes_model as bm, datagen as dg
    if cfg.n > (1 << 22):  # the 70B prefill step takes seconds on one core: time a block of rows
        T = max(cfg.R, (1 << 22) // cfg.H // cfg.R * cfg.R)
        sample = f"{T} of {cfg.T} tokens x all {cfg.R} ranks, whole steps repeated"
    else:
        T = cfg.T
        sample = f"the whole step ({cfg.R} ranks x {cfg.T} x {cfg.H}), repeated"
    n = T * cfg.H
    parts = [dg.partial(cfg, r, n) for r in range(cfg.R)]
    res, gam = dg.residual(cfg, n), dg.gamma(cfg)
    step_bytes = sum(bm.total(v) for v in bm.two_step_whole(cfg.R, T, cfg.H, cfg.bits_rs, cfg.bits_ag,
                                                             cfg.group).values())
    oracle.lib()
    with one_core() as pin:
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.two_step(parts, cfg.bits_rs, cfg.bits_ag, cfg.group, residual=res, gamma=gam, eps=cfg.eps,
                            hidden=cfg.H, plain=False)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": round(step_bytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": sample + f" {reps}x in {el:.1f} s; single-threaded C++ (g++ -O2 -ffp-contract=off) on host "
                               f"core {pin.core}",
            "us_per_step": round(el / reps * 1e6, 1), "host_cpu": host_cpu_model(),
            "host_cores": os.cpu_count()}


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def oracle_by_config(max_elems=1 << 22):
    """The oracle on each of the five workloads: single-threaded, pinned to one host core, median of 5 runs
    (3 for the two largest).  Workloads over `max_elems` elements per rank run on a block of their rows
    and are scaled to the whole workload (rows are independent, so the cost is linear in them).  Then the
    norm-first path on the decode workload, the all-gather of the int8 prefill messages and the flag
    receiver on 8 x 2 MiB, as their benchmark rows run them."""
    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    import numpy as np
    import oracle
    from tensor_all_reduce_amd import bytes_model as bm, datagen as dg
    oracle.lib()
    out = {}
    with one_core():
        for cfg in dg.WORKLOADS.values():
            T = cfg.T if cfg.n <= max_elems else max(cfg.R, max_elems // cfg.H // cfg.R * cfg.R)
            n = T * cfg.H
            reps = 3 if cfg.n > max_elems else 5
            parts = [dg.partial(cfg, r, n) for r in range(cfg.R)]
            if cfg.kind == "two_step":
                res, gam = dg.residual(cfg, n), dg.gamma(cfg)
                run = lambda: oracle.two_step(parts, cfg.bits_rs, cfg.bits_ag, cfg.group, residual=res, gamma=gam,
                                              eps=cfg.eps, hidden=cfg.H, plain=False)
                full_bytes = sum(bm.total(v) for v in bm.two_step_whole(cfg.R, cfg.T, cfg.H, cfg.bits_rs,
                                                                        cfg.bits_ag, cfg.group).values())
            elif cfg.kind == "ll":
                nslots, nblk = n // 2, n // 2 // cfg.block_slots
                slots = []
                for r in range(cfg.R):
                    sl = oracle.ll_pack(parts[r], cfg.block_slots, cfg.epoch, order=dg.write_order(cfg, r, nblk))
                    ep = dg.stale_epochs(cfg, r, nslots)[0]
                    slots.append((sl & np.uint64(0xFFFFFFFF)) | (ep.astype(np.uint64) << np.uint64(32)))
                run = lambda: oracle.ll_unpack_reduce(slots, n, cfg.block_slots, cfg.epoch)
                full_bytes = cfg.R * 4 * cfg.n + 2 * cfg.n
            else:
                res, gam = dg.residual(cfg, n), dg.gamma(cfg)
                run = lambda: oracle.reduce_rmsnorm(parts, T, cfg.H, res, gam, cfg.eps)
                full_bytes = (2 * cfg.R + 6) * cfg.n
            times = []
            for _ in range(reps):
                t0 = time.perf_counter()
                run()
                times.append(time.perf_counter() - t0)
            us = statistics.median(times) * 1e6 * (cfg.T / T)
            out[cfg.slug] = {"us_per_step": round(us, 1), "GB/s": round(full_bytes / (us * 1e-6) / 1e9, 4),
                             "runs": reps, "sample_rows": T, "rows": cfg.T}
        # the rows beyond the five workloads, on the workloads their benchmark rows use
        c2, c3, c4 = dg.DECODE_8B, dg.PREFILL_70B, dg.SLOTS
        parts = [dg.partial(c2, r) for r in range(c2.R)]
        res, gam = dg.residual(c2), dg.gamma(c2)
        extra = {
            "norm_first_decode": (lambda: oracle.two_step_normfirst(parts, c2.bits_rs, c2.bits_ag, c2.group, res, gam,
                                                                    c2.eps, c2.H),
                                  sum(bm.total(v) for v in bm.two_step_normfirst_whole(
                                      c2.R, c2.T, c2.H, c2.bits_rs, c2.bits_ag, c2.group).values())),
        }
        msg3 = c3.L * c3.bits_ag // 8 + 4 * (c3.L // c3.group)
        nwords = -(-msg3 // 4 // c4.block_slots) * c4.block_slots
        rng = np.random.default_rng(0xFC0C)
        gsl = [(rng.integers(0, 1 << 32, nwords, dtype=np.uint64)
                | (dg.stale_epochs(c4, r, nwords)[0].astype(np.uint64) << np.uint64(32))) for r in range(c3.R)]
        extra["allgather_int8_prefill_messages"] = (lambda: oracle.ll_gather(gsl, nwords, c4.block_slots, c4.epoch),
                                                    bm.total(bm.ll_gather(c3.R, nwords, c4.block_slots)))
        n2, be = 1 << 20, 2048
        xs = [dg.synth_bf16((0xF2, r), n2) for r in range(8)]
        fl = [np.full(n2 // be, 7, np.uint32) for _ in range(8)]
        extra["flag_receiver_8x2MiB"] = (lambda: oracle.flag_unpack_reduce(xs, fl, n2, be, 7),
                                         bm.total(bm.flag_unpack(8, n2, be)))
        for name, (run, by) in extra.items():
            times = []
            for _ in range(5):
                t0 = time.perf_counter()
                run()
                times.append(time.perf_counter() - t0)
            us = statistics.median(times) * 1e6
            out[name] = {"us_per_step": round(us, 1), "GB/s": round(by / (us * 1e-6) / 1e9, 4), "runs": 5}
    return out


# ---------------------------------------------------------------------------------------------------------
LEAD_CYCLES = 300_000  # the spin kernel's length (about 125 us at the engine clock)


class Ctx:
    def __init__(self):
        import numpy as np
        import torch
        self.np, self.torch = np, torch
        self.dev = torch.device("cuda:0")

    def up(self, a):
        return self.torch.from_numpy(self.np.ascontiguousarray(a).view(self.np.int16)).to(self.dev)

    def ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def warm(self, g, ms: float = 30.0):
        """Replay g until `ms` of wall time has passed (rows other than the headline: their buffers are
        fresh, and the first milliseconds of replays on fresh buffers run slower)."""
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < ms:
            g.replay()
            self.torch.cuda.synchronize()

    def graph(self, fn, count):
        g = self.torch.cuda.CUDAGraph()
        with self.torch.cuda.graph(g):
            for k in range(count):
                fn(k)
        return g

    def lead(self, stream=None):
        """A spin kernel of ~125 us ahead of a start event: the GPU stays busy while the host submits the
        work that follows, so the timed span never holds an idle GPU waiting for the first launch (a graph
        launch takes the host 15-80 us)."""
        if stream is None:
            self.torch.cuda._sleep(LEAD_CYCLES)
        else:
            with self.torch.cuda.stream(stream):
                self.torch.cuda._sleep(LEAD_CYCLES)

    def time_graph(self, g, reps, per):
        """Replay `g` reps times; microseconds per item (per = items per replay)."""
        torch = self.torch
        g.replay()
        torch.cuda.synchronize()
        a, b = self.ev(), self.ev()
        self.lead()
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * per)


def copy_ceiling(cx):
    """Copy, read-only and write-only bandwidth on 1 GiB (GB/s): the ceilings a kernel's access mix is
    compared with."""
    from tensor_all_reduce_amd import _lib
    torch = cx.torch
    nb = 1 << 30
    src = torch.empty(nb, dtype=torch.uint8, device=cx.dev)
    dst = torch.empty(nb, dtype=torch.uint8, device=cx.dev)
    out = {}
    for mode, name, moved in ((0, "copy", 2 * nb), (1, "read", nb), (2, "write", nb)):
        _lib.fc_bandwidth_probe(src, dst, nb, mode)
        torch.cuda.synchronize()
        a, b = cx.ev(), cx.ev()
        cx.lead()
        a.record()
        for _ in range(10):
            _lib.fc_bandwidth_probe(src, dst, nb, mode)
        b.record()
        torch.cuda.synchronize()
        out[name] = moved * 10 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return out


def mixed_ceiling_us(read_bytes, write_bytes, ceil):
    """Shortest time for this access mix at the measured read and write ceilings (microseconds)."""
    return (read_bytes / (ceil["read"] * 1e9) + write_bytes / (ceil["write"] * 1e9)) * 1e6


def add_mixed(per_call, calls, ceil):
    for name, c in per_call.items():
        if name in calls:
            t = mixed_ceiling_us(calls[name]["read"], calls[name]["write"], ceil)
            c["pct_mixed_ceiling"] = round(100 * t / c["us"], 1)


def bench_two_step(cx, cfg, steps, warmup, warm, kernel_reps, traffic, norm_first=False, warm_ms=0.0):
    """The quantized two-step path: timed whole steps, then each call alone.  norm_first: the variant with
    the norm applied to each shard before the all-gather (gather of the normalized rows)."""
    torch = cx.torch
    from tensor_all_reduce_amd import bytes_model as bm, datagen as dg
    from tensor_all_reduce_amd.flash_allreduce import TwoStepAllReduce
    R, T, H, G, b1, b2 = cfg.R, cfg.T, cfg.H, cfg.group, cfg.bits_rs, cfg.bits_ag
    calls = (bm.two_step_normfirst_whole if norm_first else bm.two_step_whole)(R, T, H, b1, b2, G)
    step_bytes = sum(bm.total(v) for v in calls.values())
    # every call's own working set over all buffer sets exceeds twice the last-level cache
    nsets = 1 if warm else max(1, math.ceil(2 * MALL_BYTES / min(bm.total(v) for v in calls.values())))
    parts0 = cx.up(cx.np.stack(dg.partials(cfg)))
    res0, gam = cx.up(dg.residual(cfg)), cx.up(dg.gamma(cfg))
    sets = []
    for k in range(nsets):
        p = TwoStepAllReduce(R, T, H, b1, b2, G, device=cx.dev, parts=parts0.clone() if k else parts0)
        res = res0.clone() if k else res0
        out = torch.empty(cfg.n, dtype=torch.int16, device=cx.dev)
        rout = torch.empty(cfg.n, dtype=torch.int16, device=cx.dev)
        norm = p.make_norm(gam, None if norm_first else out, residual=res, residual_out=rout, eps=cfg.eps)
        sets.append((p, norm, (res, out, rout)))
    if warm:  # graphs of 64 steps on the one buffer set (a graph of one step would time its launch)
        sets, nsets = sets * 64, 64
    torch.cuda.synchronize()

    def step(k):
        p, norm, bufs = sets[k]
        if norm_first:
            p.run_norm_first(bufs[1], norm)
        else:
            p.run(norm=norm)

    for k in range(min(warmup, nsets)):
        step(k)
    torch.cuda.synchronize()
    g_all = cx.graph(step, nsets)
    g_tail = cx.graph(step, steps % nsets) if steps % nsets else None
    for _ in range(max(1, warmup // nsets)):
        g_all.replay()
    torch.cuda.synchronize()
    if warm_ms:
        cx.warm(g_all, warm_ms)
    # timed region: exactly `steps` steps
    e0, e1 = cx.ev(), cx.ev()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    cx.lead()
    e0.record()
    for _ in range(steps // nsets):
        g_all.replay()
    if g_tail is not None:
        g_tail.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / steps

    # spread: the same steps replayed in chunks of c consecutive buffer sets, one event pair per chunk.  An
    # event recorded between two replays costs about 5 us on the prefill step (its completion signal waits
    # for the work before it), so a chunk holds several steps: every set when there are few of them
    c = nsets if nsets < 10 else max(1, min(20, nsets // 10))
    nchunk = min(30, nsets // c)
    chunks = [cx.graph(lambda k, i=i: step(i * c + k), c) for i in range(nchunk)]
    rounds = -(-16 // nchunk)  # at least 16 samples: few buffer sets are walked several times
    evs = [cx.ev() for _ in range(rounds * nchunk + 1)]
    torch.cuda.synchronize()
    cx.lead()
    evs[0].record()
    for r in range(rounds):
        for i, gc in enumerate(chunks):
            gc.replay()
            evs[r * nchunk + i + 1].record()
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 / c for i in range(rounds * nchunk))
    pct = lambda q: round(per[min(len(per) - 1, int(q * (len(per) - 1) + 0.5))], 3)
    spread = {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9), "chunks": rounds * nchunk, "steps_per_chunk": c}
    del chunks

    reps = kernel_reps or max(2, steps // nsets)
    if norm_first:
        fns = {"quantize": lambda k: sets[k][0].quantize(),
               "reduce_shard": lambda k: sets[k][0].reduce_scatter_norm(sets[k][1]),
               "gather": lambda k: sets[k][0].all_gather(y=sets[k][2][1])}
    else:
        fns = {"quantize": lambda k: sets[k][0].quantize(), "reduce_shard": lambda k: sets[k][0].reduce_scatter(),
               "gather_norm": lambda k: sets[k][0].all_gather(norm=sets[k][1])}
    per_call = {}
    # each call alone over the buffer sets, the calls taken in turn, `reps` rounds: every call samples the
    # same stretch of the run (the engine clock drifts under sustained load)
    graphs = {name: cx.graph(fn, nsets) for name, fn in fns.items()}
    samples = {name: [] for name in fns}
    for name, g in graphs.items():
        g.replay()
    torch.cuda.synchronize()
    for _ in range(reps):
        for name, g in graphs.items():
            samples[name].append(_once(cx, g, nsets))
    del graphs
    # each call inside the step: the steps launched one call at a time in step order, an event pair around
    # every call (so each kernel runs after the same predecessor as in the timed steps, with the messages
    # of its own step in the caches); the kernels' average duration there is the roofline's
    in_step = {name: [] for name in fns}
    names = list(fns)
    for _ in range(reps):
        evs = [[cx.ev() for _ in range(len(names) + 1)] for _ in range(nsets)]
        g_all.replay()  # keeps the GPU busy while the host enqueues the calls, so no pair spans an idle GPU
        for k in range(nsets):
            evs[k][0].record()
            for j, name in enumerate(names):
                fns[name](k)
                evs[k][j + 1].record()
        torch.cuda.synchronize()
        for k in range(nsets):
            for j, name in enumerate(names):
                in_step[name].append(evs[k][j].elapsed_time(evs[k][j + 1]) * 1e3)
    for name in fns:
        us = statistics.median(samples[name])
        by = bm.total(calls[name])
        gbps = by / (us * 1e-6) / 1e9
        us_in = statistics.fmean(in_step[name])
        per_call[name] = {"us": round(us, 3), "bytes": by, "GB/s": round(gbps, 1),
                          "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4), "us_in_step": round(us_in, 3),
                          "GB/s_in_step": round(by / (us_in * 1e-6) / 1e9, 1),
                          "traffic": None if norm_first else traffic_for(name, cfg, traffic)}
    del sets, g_all, g_tail
    torch.cuda.empty_cache()
    return dict(ms_step=ms_step, wall=wall, step_bytes=step_bytes, nsets=nsets, per_call=per_call, spread=spread)


def bench_share(cx, cfg, steps, warmup, kernel_reps, norm_first=False):
    """One GPU's real share (P mode) of the quantized two-step path, rank 0: its own quantize, its own
    shard's reduce, the gather + epilogue of all shards.  The peers' chunks of shard 0 and the other
    shards' all-gather messages are produced once by the whole emulated path and copied into every buffer
    set outside the timed region (the transport's work).  Timed like the whole path: cold buffer sets,
    whole steps from a HIP graph, then each call alone."""
    torch = cx.torch
    from tensor_all_reduce_amd import bytes_model as bm, datagen as dg
    from tensor_all_reduce_amd.flash_allreduce import TwoStepAllReduce, TwoStepShare
    R, T, H, G, b1, b2 = cfg.R, cfg.T, cfg.H, cfg.group, cfg.bits_rs, cfg.bits_ag
    calls = (bm.two_step_normfirst_share if norm_first else bm.two_step_share)(R, T, H, b1, b2, G)
    step_bytes = sum(bm.total(v) for v in calls.values())
    nsets = max(1, math.ceil(2 * MALL_BYTES / min(bm.total(v) for v in calls.values())))
    whole = TwoStepAllReduce(R, T, H, b1, b2, G, device=cx.dev, parts=cx.up(cx.np.stack(dg.partials(cfg))))
    res0, gam = cx.up(dg.residual(cfg)), cx.up(dg.gamma(cfg))
    whole.quantize()
    if norm_first:
        whole.reduce_scatter_norm(whole.make_norm(gam, None, residual=res0, eps=cfg.eps))
    else:
        whole.reduce_scatter()
    sets = []
    for k in range(nsets):
        sh = TwoStepShare(R, T, H, b1, b2, G, rank=0, device=cx.dev, x=whole.parts[0].clone())
        for r in range(1, R):
            c, m = whole.rank_chunk(r, 0)
            sh.inbox_codes[r].copy_(c)
            sh.inbox_meta[r].copy_(m)
        for s in range(1, R):
            c, m = whole.shard_msg(s)
            sh.codes2[s].copy_(c)
            sh.meta2[s].copy_(m)
        out = torch.empty(cfg.n, dtype=torch.int16, device=cx.dev)
        if norm_first:  # the own shard's rows only
            res = res0[:cfg.L].clone()
            rout = torch.empty(cfg.L, dtype=torch.int16, device=cx.dev)
            norm = sh.make_norm(gam, None, residual=res, residual_out=rout, eps=cfg.eps)
        else:
            res = res0.clone()
            rout = torch.empty(cfg.n, dtype=torch.int16, device=cx.dev)
            norm = sh.make_norm(gam, out, residual=res, residual_out=rout, eps=cfg.eps)
        sets.append((sh, norm, (res, out, rout)))
    del whole
    torch.cuda.synchronize()

    def step(k):
        sh, norm, bufs = sets[k]
        if norm_first:
            sh.run_norm_first(bufs[1], norm)
        else:
            sh.run(norm=norm)

    g_all = cx.graph(step, nsets)
    for _ in range(max(1, warmup // nsets)):
        g_all.replay()
    torch.cuda.synchronize()
    cx.warm(g_all)
    reps = max(1, steps // nsets)
    us_step = cx.time_graph(g_all, reps, nsets)
    if norm_first:
        fns = {"quantize": lambda k: sets[k][0].quantize(), "reduce_shard": lambda k: sets[k][0].reduce_norm(sets[k][1]),
               "gather": lambda k: sets[k][0].gather(y=sets[k][2][1])}
    else:
        fns = {"quantize": lambda k: sets[k][0].quantize(), "reduce_shard": lambda k: sets[k][0].reduce(),
               "gather_norm": lambda k: sets[k][0].gather(norm=sets[k][1])}
    per_call = {}
    for name, fn in fns.items():
        us = cx.time_graph(cx.graph(fn, nsets), kernel_reps or max(2, reps), nsets)
        by = bm.total(calls[name])
        per_call[name] = {"us": round(us, 3), "bytes": by, "GB/s": round(by / (us * 1e-6) / 1e9, 1)}
    v = step_bytes / (us_step * 1e-6) / 1e9
    res = {"workload": cfg.name, "mode": "one GPU's real share (rank 0)" + (", norm before the all-gather"
                                                                              if norm_first else ""),
           "us_per_step": round(us_step, 3),
           "bytes_per_step": step_bytes, "GB/s": round(v, 1), "pct_hbm_peak": round(100 * v / HBM_PEAK_GBPS, 2),
           "buffer_sets": nsets, "steps_timed": reps * nsets, "calls": per_call}
    del sets, g_all
    torch.cuda.empty_cache()
    return res


def bench_ll(cx):
    """Self-synchronizing slots, 8 ranks x [128, 8192], 64-slot blocks, 2% late (rank, block) copies with the
    seeded mix of wrong epoch words: time the first pass and the retry after the late blocks arrive."""
    torch, np = cx.torch, cx.np
    from tensor_all_reduce_amd import _lib, bytes_model as bm, datagen as dg
    from tensor_all_reduce_amd.flash_allreduce import LLUnpackReduce, rank_rows
    cfg = dg.SLOTS
    R, n, B, e = cfg.R, cfg.n, cfg.block_slots, cfg.epoch
    nslots, nblk = n // 2, n // 2 // B
    set_bytes = R * 4 * n
    nsets = max(1, math.ceil(2 * MALL_BYTES / set_bytes))
    xs = [cx.up(dg.partial(cfg, r)) for r in range(R)]
    orders = [torch.from_numpy(dg.write_order(cfg, r, nblk)).to(cx.dev) for r in range(R)]
    eps, masks = zip(*[dg.stale_epochs(cfg, r, nslots) for r in range(R)])
    late_ep = [torch.from_numpy(ep.view(np.int32)).to(cx.dev) for ep in eps]
    good_ep = torch.full((nslots,), e, dtype=torch.int64, device=cx.dev).to(torch.int32)
    sets = []
    for k in range(nsets):
        slots = list(rank_rows(R, nslots, torch.int64, cx.dev)[1])  # the R inboxes staggered in one allocation
        for r in range(R):
            _lib.fc_ll_pack(xs[r], B, e, slots[r], block_order=orders[r])
        out = torch.zeros(n, dtype=torch.int16, device=cx.dev)
        stale = torch.zeros(R * nblk, dtype=torch.uint8, device=cx.dev)
        done = torch.zeros(nblk, dtype=torch.uint8, device=cx.dev)
        cnt = torch.zeros(_lib.COUNTER_WORDS, dtype=torch.int32, device=cx.dev)
        sets.append((slots, LLUnpackReduce(slots, n, B, out, stale, done, cnt), done, cnt,
                     LLUnpackReduce(slots, n, B, out, stale, done, None)))

    def set_epochs(which):
        for slots, *_ in sets:
            for r in range(R):
                slots[r].view(torch.int32).view(-1, 2)[:, 1] = which[r] if which is not None else good_ep

    def reset():
        for _, _, done, cnt, _ in sets:
            done.zero_()
            cnt.zero_()
    g = cx.graph(lambda k: sets[k][1].run(e), nsets)
    g0 = cx.graph(lambda k: sets[k][4].run(e), nsets)  # the same receiver without counters
    cx.warm(g0)
    t1, t2, t0 = [], [], []
    for _ in range(5):
        set_epochs(late_ep)
        reset()
        torch.cuda.synchronize()
        t0.append(_once(cx, g0, nsets))
        reset()
        torch.cuda.synchronize()
        t1.append(_once(cx, g, nsets))
        cnt0 = _lib.counter_totals(sets[0][3])
        set_epochs(None)
        torch.cuda.synchronize()
        t2.append(_once(cx, g, nsets))
    pending = int(cnt0[1])
    by1 = bm.total(bm.ll_unpack(R, n, B, completed_blocks=nblk - pending))
    us1, us2, us0 = statistics.median(t1), statistics.median(t2), statistics.median(t0)
    res = {"workload": cfg.name, "pass1_us": round(us1, 2), "pass1_bytes": by1,
           "pass1_GB/s": round(by1 / (us1 * 1e-6) / 1e9, 1), "stale_pairs": int(cnt0[0]), "pending_blocks": pending,
           "blocks": nblk, "retry_us": round(us2, 2), "buffer_sets": nsets,
           "pass1_nocount_us": round(us0, 2), "pass1_nocount_GB/s": round(by1 / (us0 * 1e-6) / 1e9, 1)}
    del sets, g, g0
    torch.cuda.empty_cache()
    return res


def bench_ll_gather(cx):
    """Standalone all-gather on epoch-tagged blocks, 8 ranks, 64-slot blocks, 2% late (rank, block) copies:
    bf16 shards of the slot workload ([16, 8192] per rank) and the int8 all-gather messages of the 70B
    prefill shards (codes then meta, 1.08 M words per rank).  First pass, then the retry once the late
    blocks have arrived."""
    torch, np = cx.torch, cx.np
    from tensor_all_reduce_amd import _lib, bytes_model as bm, datagen as dg
    c4, c3 = dg.SLOTS, dg.PREFILL_70B
    B, e = c4.block_slots, c4.epoch
    res = {}
    msg3 = c3.L * c3.bits_ag // 8 + 4 * (c3.L // c3.group)
    for tag, R, nwords in (("bf16_shards", c4.R, c4.n // c4.R // 2), ("int8_prefill_messages", c3.R,
                                                                         -(-msg3 // 4 // B) * B)):
        nblk = nwords // B
        nsets = max(1, math.ceil(2 * MALL_BYTES / (R * nwords * 12)))
        gen = torch.Generator(device=cx.dev)
        gen.manual_seed(0xFC0A + nwords)
        eps = [torch.from_numpy(dg.stale_epochs(c4, r, nwords)[0].astype(np.int64)).to(cx.dev) for r in range(R)]
        good = torch.full((nwords,), e, dtype=torch.int64, device=cx.dev)
        sets = []
        for k in range(nsets):
            words = [torch.randint(0, 1 << 32, (nwords,), dtype=torch.int64, device=cx.dev, generator=gen)
                     for _ in range(R)]
            slots = [w.clone() for w in words]
            out = [torch.empty(nwords, dtype=torch.int32, device=cx.dev) for _ in range(R)]
            stale = torch.zeros(R * nblk, dtype=torch.uint8, device=cx.dev)
            done = torch.zeros(R * nblk, dtype=torch.uint8, device=cx.dev)
            cnt = torch.zeros(_lib.COUNTER_WORDS, dtype=torch.int32, device=cx.dev)
            sets.append((words, slots, out, stale, done, cnt))

        def set_epochs(late):
            for words, slots, *_ in sets:
                for r in range(R):
                    slots[r].copy_(words[r] | ((eps[r] if late else good) << 32))

        def run(k, counted=True):
            _, slots, out, stale, done, cnt = sets[k]
            _lib.fc_ll_gather(slots, nwords, B, e, out, stale, done, cnt if counted else None)
        g = cx.graph(run, nsets)
        g0 = cx.graph(lambda k: run(k, False), nsets)  # the same pass without counters
        cx.warm(g0)
        t1, t2, t0 = [], [], []
        for _ in range(5):
            set_epochs(True)
            for s in sets:
                s[4].zero_()
            torch.cuda.synchronize()
            t0.append(_once(cx, g0, nsets))
            for s in sets:
                s[4].zero_()
                s[5].zero_()
            torch.cuda.synchronize()
            t1.append(_once(cx, g, nsets))
            pend = int(_lib.counter_totals(sets[0][5])[1])
            set_epochs(False)
            torch.cuda.synchronize()
            t2.append(_once(cx, g, nsets))
        by1 = bm.total(bm.ll_gather(R, nwords, B, completed_blocks=R * nblk - pend))
        us1, us2, us0 = statistics.median(t1), statistics.median(t2), statistics.median(t0)
        res[tag] = {"R": R, "words_per_rank": nwords, "pass1_us": round(us1, 2), "pass1_bytes": by1,
                    "pass1_GB/s": round(by1 / (us1 * 1e-6) / 1e9, 1), "pending_pairs": pend, "pairs": R * nblk,
                    "retry_us": round(us2, 2), "buffer_sets": nsets, "pass1_nocount_us": round(us0, 2),
                    "pass1_nocount_GB/s": round(by1 / (us0 * 1e-6) / 1e9, 1)}
        del sets, g, g0
        torch.cuda.empty_cache()
    return {"workload": "standalone all-gather on epoch-tagged blocks, B=64, 2% late", "by_payload": res}


def bench_encodings(cx, fit_out=None):
    """Readiness encodings with a sender and a receiver running at the same time: per rank count R and
    payload size S, the receiver (fc_ll_poll_unpack_reduce or fc_flag_unpack_reduce) is launched first on
    a stream of its own compute units, where it spins within its poll budget; the R senders (one launch of
    fc_ll_pack or fc_flag_pack) follow on a stream of the other compute units.  Latency = from the senders'
    start to the receiver's end (a copy kernel holds the senders' stream while the host enqueues, so no
    host launch gap is timed).  Every live pass must complete every block.  The cost model of the
    protocol selector is fitted to these latencies."""
    torch, np = cx.torch, cx.np
    from tensor_all_reduce_amd import _lib, datagen as dg, selector as sel
    from tensor_all_reduce_amd.streams import sender_receiver_streams
    rcu = 128
    sa, sb = sender_receiver_streams(receiver_cus=rcu)
    xa, xb = torch.cuda.ExternalStream(sa.cuda_stream), torch.cuda.ExternalStream(sb.cuda_stream)
    hold = [torch.empty(256 << 20, dtype=torch.uint8, device=cx.dev) for _ in range(2)]
    polls, mwg, reps = 200_000, 2 * rcu, 7
    sizes = [16 << 10, 32 << 10, 64 << 10, 128 << 10, 256 << 10, 512 << 10, 1 << 20, 2 << 20, 4 << 20, 8 << 20, 16 << 20]
    rows, detail = [], []
    for R in (2, 4, 8):
        for S in sizes:
            n = S // 2
            xs = [cx.up(dg.synth_bf16((0xE1, R, S, r), n)) for r in range(R)]
            for enc in sel.ENCODINGS:
                if enc == "ll":
                    B = sel.LL_BLOCK_SLOTS
                    nblk = n // 2 // B
                    bufs = [torch.empty(n // 2, dtype=torch.int64, device=cx.dev) for _ in range(R)]
                    _lib.fc_ll_pack(xs, B, 1000, bufs)  # an earlier epoch: every copy starts stale
                else:
                    be = sel.flag_block(enc)
                    nblk = n // be
                    pays = [torch.zeros(n, dtype=torch.int16, device=cx.dev) for _ in range(R)]
                    fls = [torch.full((nblk,), 1000, dtype=torch.int32, device=cx.dev) for _ in range(R)]
                out = torch.empty(n, dtype=torch.int16, device=cx.dev)
                stale = torch.empty(R * nblk, dtype=torch.uint8, device=cx.dev)
                done = torch.zeros(nblk, dtype=torch.uint8, device=cx.dev)
                cnt = torch.zeros(_lib.COUNTER_WORDS, dtype=torch.int32, device=cx.dev)

                def receive(e, stream):
                    if enc == "ll":
                        _lib.fc_ll_poll_unpack_reduce(bufs, n, B, e, out, stale, done, cnt, max_polls=polls,
                                                      max_workgroups=mwg, stream=stream)
                    else:
                        _lib.fc_flag_unpack_reduce(pays, fls, n, be, e, out, stale, done, cnt, max_polls=polls,
                                                   max_workgroups=mwg, stream=stream)

                def send(e, stream):
                    if enc == "ll":
                        _lib.fc_ll_pack(xs, B, e, bufs, stream=stream)
                    else:
                        _lib.fc_flag_pack(xs, be, e, pays, fls, stream=stream)

                live, alone, ok = [], [], True
                for rep in range(reps):
                    e = 1001 + rep
                    done.zero_()
                    cnt.zero_()
                    torch.cuda.synchronize()
                    a, b = cx.ev(), cx.ev()
                    receive(e, sa)                      # spins on its own compute units
                    _lib.fc_copy(hold[0], hold[1], stream=sb)
                    a.record(xb)
                    send(e, sb)
                    b.record(xa)
                    torch.cuda.synchronize()
                    c = _lib.counter_totals(cnt)
                    ok = ok and int(c[1]) == 0
                    live.append(a.elapsed_time(b) * 1e3)
                    # the receiver alone, every block already there
                    done.zero_()
                    cnt.zero_()
                    torch.cuda.synchronize()
                    a, b = cx.ev(), cx.ev()
                    _lib.fc_copy(hold[0], hold[1], stream=sa)
                    a.record(xa)
                    receive(e, sa)
                    b.record(xa)
                    torch.cuda.synchronize()
                    alone.append(a.elapsed_time(b) * 1e3)
                t = statistics.median(live)
                if ok:
                    rows.append((enc, S, R, round(t, 2)))
                detail.append({"enc": enc, "S": S, "R": R, "live_us": round(t, 2),
                               "receiver_alone_us": round(statistics.median(alone), 2), "all_blocks_live": ok})
                del out, stale, done, cnt
                if enc == "ll":
                    del bufs
                else:
                    del pays, fls
    sa.close()
    sb.close()
    del hold
    torch.cuda.empty_cache()
    costs = sel.fit(rows)
    refit_score = sel.regret(costs, rows)              # in sample: fitted to these latencies
    committed = sel.regret(sel.load(), rows)          # out of sample: the table shipped in the package
    res = {"receiver_cus": rcu, "sender_cus": "the rest", "reps": reps, "points": detail,
           "model": {e: list(c.coef) for e, c in costs.items()},
           "choice_matches_fastest_measured": f"{refit_score['fastest']}/{refit_score['points']}",
           "refit_regret": refit_score, "committed_table": committed,
           "crossover_R8": sel.crossover(costs, 8), "crossover_R2": sel.crossover(costs, 2)}
    if fit_out:
        total = torch.cuda.get_device_properties(0).multi_processor_count
        sel.save(fit_out, costs, rows, "python bench.py --rows encodings --no-cpu-baseline --fit-encodings " + fit_out,
                 f"one {torch.cuda.get_device_name(0)}: receiver on {rcu} compute units, senders on {total - rcu}")
    return res


def _once(cx, g, per):
    torch = cx.torch
    a, b = cx.ev(), cx.ev()
    cx.lead()
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / per


def bench_rmsnorm_overlap(cx):
    """Unquantized fused reduce + residual-add + RMSNorm, 8 ranks x [8192, 8192] split into two wave-aware
    halves of 4096 rows: each half alone (per workgroup cap), the bf16 GEMM [4096,8192]x[8192,8192] alone,
    and half A's reduce on one stream overlapped with the GEMM on another."""
    torch, np = cx.torch, cx.np
    from tensor_all_reduce_amd import bytes_model as bm, datagen as dg
    from tensor_all_reduce_amd.flash_allreduce import ReduceRMSNorm, rank_rows
    cfg = dg.TOKENWEAVE
    R, T, H = cfg.R, cfg.T, cfg.H
    a = cfg.splits[0]
    pbuf, parts = rank_rows(R, T * H, torch.int16, cx.dev)  # the R partials staggered in one allocation
    for r in range(R):
        parts[r].copy_(cx.up(dg.partial(cfg, r)))
    res, gam = cx.up(dg.residual(cfg)), cx.up(dg.gamma(cfg))
    out = torch.empty(T * H, dtype=torch.int16, device=cx.dev)
    rout = torch.empty(T * H, dtype=torch.int16, device=cx.dev)
    halves = []
    for lo, hi in ((0, a), (a, T)):
        sl = slice(lo * H, hi * H)
        halves.append(ReduceRMSNorm([p[sl] for p in parts], hi - lo, H, gam, out[sl], residual=res[sl],
                                    residual_out=rout[sl], eps=cfg.eps))
    half_bytes = bm.total(bm.reduce_rmsnorm(R, a, H, True, True))
    gen = torch.Generator(device=cx.dev)
    gen.manual_seed(0xFC07)
    A = torch.randn(a, H, device=cx.dev, dtype=torch.bfloat16, generator=gen)
    Bm = torch.randn(H, H, device=cx.dev, dtype=torch.bfloat16, generator=gen)
    C = torch.empty(a, H, device=cx.dev, dtype=torch.bfloat16)
    s1, s2 = torch.cuda.Stream(device=cx.dev), torch.cuda.Stream(device=cx.dev)
    reps = 8

    def timed(stream, fn):
        ea, eb = cx.ev(), cx.ev()
        with torch.cuda.stream(stream):
            cx.lead(stream)
            ea.record()
            for _ in range(reps):
                fn()
            eb.record()
        return ea, eb

    def gemm():
        torch.matmul(A, Bm, out=C)
    # warm up (the first milliseconds on fresh buffers run slower)
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < 30.0:
        for h in halves:
            h.run(stream=s1)
        torch.cuda.synchronize()
    with torch.cuda.stream(s2):
        gemm()
    torch.cuda.synchronize()
    ga, gb = timed(s2, gemm)
    torch.cuda.synchronize()
    gemm_us = ga.elapsed_time(gb) * 1e3 / reps
    sweep = {}
    for mw in (8, 16, 32, 64, 128, 256, 0):
        ea, eb = timed(s1, lambda: halves[0].run(max_workgroups=mw, stream=s1))
        torch.cuda.synchronize()
        alone = ea.elapsed_time(eb) * 1e3 / reps
        # overlapped: both streams start after a common event
        start = cx.ev()
        cx.lead()
        start.record(torch.cuda.current_stream())
        s1.wait_event(start)
        s2.wait_event(start)
        ra, rb = timed(s1, lambda: halves[0].run(max_workgroups=mw, stream=s1))
        qa, qb = timed(s2, gemm)
        end1, end2 = cx.ev(), cx.ev()
        end1.record(s1)
        end2.record(s2)
        torch.cuda.synchronize()
        over_r = ra.elapsed_time(rb) * 1e3 / reps
        over_g = qa.elapsed_time(qb) * 1e3 / reps
        makespan = max(start.elapsed_time(end1), start.elapsed_time(end2)) * 1e3 / reps
        sweep[str(mw) if mw else "rows"] = {
            "alone_us": round(alone, 1), "alone_GB/s": round(half_bytes / (alone * 1e-6) / 1e9, 1),
            "overlap_reduce_us": round(over_r, 1), "overlap_gemm_us": round(over_g, 1),
            "overlap_makespan_us": round(makespan, 1), "serial_us": round(alone + gemm_us, 1)}
    # both halves back to back at the default grid
    ea, eb = timed(s1, lambda: (halves[0].run(stream=s1), halves[1].run(stream=s1)))
    torch.cuda.synchronize()
    both = ea.elapsed_time(eb) * 1e3 / reps
    res = {"workload": cfg.name, "half_bytes": half_bytes, "both_halves_us": round(both, 1),
           "both_halves_GB/s": round(2 * half_bytes / (both * 1e-6) / 1e9, 1),
           "gemm_alone_us": round(gemm_us, 1), "gemm_TFLOP/s": round(2 * a * H * H / (gemm_us * 1e-6) / 1e12, 1),
           "max_workgroups_sweep": sweep}
    del parts, pbuf, halves, A, Bm, C
    torch.cuda.empty_cache()
    return res


def bench_layer(cx):
    """The two-half pipelined layer step (GEMM [T_h, 8192] x [8192, 8192] of each half on one stream, the
    8-rank all-reduce + RMSNorm of each half on another) against the same halves run serially and against
    no split, at T = 8192 and at T = 6000 (a split that is not a halving)."""
    torch = cx.torch
    from tensor_all_reduce_amd import datagen as dg
    from tensor_all_reduce_amd.schedule import TwoHalfLayer, gemm_waves, wave_aware_split
    cfg = dg.TOKENWEAVE
    R, H = cfg.R, cfg.H
    res_rows = {}
    for T in (cfg.T, 6000):
        gen = torch.Generator(device=cx.dev)
        gen.manual_seed(0xFC07 + T)
        x = torch.randn(T, H, device=cx.dev, dtype=torch.bfloat16, generator=gen)
        w = (torch.randn(H, H, device=cx.dev, dtype=torch.bfloat16, generator=gen) * H ** -0.5).to(torch.bfloat16)
        peers = [torch.randn(T, H, device=cx.dev, dtype=torch.bfloat16, generator=gen).view(torch.int16)
                 for _ in range(R - 1)]
        res = torch.randn(T, H, device=cx.dev, dtype=torch.bfloat16, generator=gen).view(torch.int16)
        gam = cx.up(dg.gamma(cfg))
        out = torch.empty(T * H, dtype=torch.int16, device=cx.dev)
        rout = torch.empty(T * H, dtype=torch.int16, device=cx.dev)
        s1, s2 = torch.cuda.Stream(device=cx.dev), torch.cuda.Stream(device=cx.dev)
        split = TwoHalfLayer(x, w, peers, res, gam, out, residual_out=rout)
        whole = TwoHalfLayer(x, w, peers, res, gam, out, residual_out=rout, t1=T)

        def timed(fn, reps=5):
            fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                a = cx.ev()
                cx.lead()
                a.record(torch.cuda.current_stream())
                s1.wait_event(a)
                s2.wait_event(a)
                fn()
                b1, b2 = cx.ev(), cx.ev()
                b1.record(s1)
                b2.record(s2)
                torch.cuda.synchronize()
                ts.append(max(a.elapsed_time(b1), a.elapsed_time(b2)) * 1e3)
            return statistics.median(ts)
        t1 = split.t1
        res_rows[str(T)] = {
            "t1": t1, "waves": [gemm_waves(t1, H), gemm_waves(T - t1, H)], "unsplit_waves": gemm_waves(T, H),
            "unsplit_us": round(timed(lambda: whole.run_serial(s1)), 1),
            "serial_halves_us": round(timed(lambda: split.run_serial(s1)), 1),
            "pipelined_us": round(timed(lambda: split.run(s1, s2)), 1)}
        del x, w, peers, res, out, rout, split, whole
        torch.cuda.empty_cache()
    return {"workload": f"two-half layer step, GEMM [T, {H}] x [{H}, {H}] bf16 + {R}-rank bf16 all-reduce + RMSNorm",
            "by_T": res_rows}


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return 0
    if args.stats_table:
        stats_table(*args.stats_table)
        return 0
    if args.rows_pmc_report:
        rows_pmc_report(*args.rows_pmc_report)
        return 0
    if args.pmc_rows:
        pmc_rows(args.pmc_rows)
        return 0
    if args.profile_report:
        c, *paths = args.profile_report
        profile_report(c, *paths)
        return 0
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the R ranks are emulated on one GPU "
              "(inter-GPU transfers are local HBM buffers); run with --gpus 1", file=sys.stderr)
        return 2
    from tensor_all_reduce_amd import bytes_model as bm, datagen as dg
    cx = Ctx()
    cfg = dg.WORKLOADS[args.config]
    traffic = load_traffic(cfg)
    assert cfg.kind == "two_step", "the benchmark's metric is the quantized two-step path"
    main_r = bench_two_step(cx, cfg, args.steps, args.warmup, args.warm, args.kernel_reps, traffic)
    ms_step = main_r["ms_step"]
    value = main_r["step_bytes"] / (ms_step * 1e-3) / 1e9
    per_call = main_r["per_call"]
    dom = max(per_call, key=lambda k: per_call[k]["us"])
    ceil = copy_ceiling(cx)
    copy_gbps = ceil["copy"]
    add_mixed(per_call, bm.two_step_whole(cfg.R, cfg.T, cfg.H, cfg.bits_rs, cfg.bits_ag, cfg.group), ceil)
    tr = per_call[dom]["traffic"]
    sp = main_r["spread"]
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "R": cfg.R, "T": cfg.T, "H": cfg.H, "bits_rs": cfg.bits_rs,
                   "bits_ag": cfg.bits_ag, "group": cfg.group, "mode": "W: whole emulated all-reduce on one GPU",
                   "cache": "warm" if args.warm else "cold", "buffer_sets": main_r["nsets"],
                   "launch": "hip graph, 3 kernels per step"},
        "us_per_step": round(ms_step * 1e3, 3), "us_spread_p10_p50_p90": [sp["p10"], sp["p50"], sp["p90"]],
        "bytes_per_step": main_r["step_bytes"],
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2), "pct_copy_ceiling": round(100 * value / copy_gbps, 2),
        "ceilings_GBps": {k: round(v, 1) for k, v in ceil.items()},
        "calls": {k: {"us": v["us"], "GBps": v["GB/s"], "frac": v["frac_hbm"], "pct_mix": v.get("pct_mixed_ceiling"),
                      "us_in_step": v["us_in_step"]} for k, v in per_call.items()},
        # the dominant kernel's average duration inside the step (event pairs around each launch, in step
        # order), as a kernel trace of the same run averages it
        "roofline": {"bound": "hbm", "kernel": dom + (f" ({tr['kernel'].split('(')[0].replace('void ', '')})"
                                                      if tr else ""),
                     "achieved": per_call[dom]["GB/s_in_step"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(per_call[dom]["GB/s_in_step"] / HBM_PEAK_GBPS, 4),
                     "traffic": tr["total"] if tr else None, "algorithmic_bytes": per_call[dom]["bytes"],
                     "us": per_call[dom]["us_in_step"]},
        "wall_s": round(main_r["wall"], 3),
    }
    rows = set(DEFAULT_ROWS.split(",")) if args.rows == "default" else set(ALL_ROWS.split(",")) \
        if args.rows == "all" else set() if args.rows == "none" else set(args.rows.split(","))
    other = dg.DECODE_8B if cfg is dg.PREFILL_70B else dg.PREFILL_70B
    extra = {}
    if "decode" in rows or "prefill" in rows:
        so = 600 if other is dg.DECODE_8B else 30
        ro = bench_two_step(cx, other, so, so // 10, False, 0, load_traffic(other), warm_ms=30.0)
        add_mixed(ro["per_call"], bm.two_step_whole(other.R, other.T, other.H, other.bits_rs, other.bits_ag,
                                                    other.group), ceil)
        vo = ro["step_bytes"] / (ro["ms_step"] * 1e-3) / 1e9
        extra[f"two_step_{other.slug}"] = {"workload": other.name, "us_per_step": round(ro["ms_step"] * 1e3, 3),
                                           "us_per_step_spread": ro["spread"], "GB/s": round(vo, 1),
                                           "pct_hbm_peak": round(100 * vo / HBM_PEAK_GBPS, 2),
                                           "pct_copy_ceiling": round(100 * vo / copy_gbps, 2),
                                           "calls": ro["per_call"]}
    if "warm" in rows and not args.warm:
        # context, not the headline: inputs already in the caches, as right after the GEMM that produced them
        rw = bench_two_step(cx, cfg, args.steps, args.warmup, True, args.kernel_reps, None, warm_ms=30.0)
        vw = rw["step_bytes"] / (rw["ms_step"] * 1e-3) / 1e9
        extra["warm_caches"] = {"workload": cfg.name, "mode": "one buffer set, cache-resident",
                                "us_per_step": round(rw["ms_step"] * 1e3, 3), "GB/s": round(vw, 1),
                                "calls": {k: v["us"] for k, v in rw["per_call"].items()}}
    if "share" in rows:
        for c in (dg.PREFILL_70B, dg.DECODE_8B):
            st = 30 if c is dg.PREFILL_70B else 600
            extra[f"share_{c.slug}"] = bench_share(cx, c, st, st // 10, 0)
    if "normfirst" in rows:
        for c in (dg.PREFILL_70B, dg.DECODE_8B):
            st = 30 if c is dg.PREFILL_70B else 300
            rw = bench_two_step(cx, c, st, st // 10, False, 0, None, norm_first=True, warm_ms=30.0)
            vw = rw["step_bytes"] / (rw["ms_step"] * 1e-3) / 1e9
            extra[f"norm_first_{c.slug}"] = {
                "workload": c.name, "mode": "whole emulated all-reduce, norm before the all-gather",
                "us_per_step": round(rw["ms_step"] * 1e3, 3), "GB/s": round(vw, 1),
                "pct_hbm_peak": round(100 * vw / HBM_PEAK_GBPS, 2), "calls": rw["per_call"],
                "share": bench_share(cx, c, st, st // 10, 0, norm_first=True)}
    if "ll" in rows:
        extra["self_sync_slots"] = bench_ll(cx)
    if "llgather" in rows:
        extra["self_sync_allgather"] = bench_ll_gather(cx)
    if "rmsnorm" in rows:
        extra["tokenweave_reduce_rmsnorm"] = bench_rmsnorm_overlap(cx)
    if "layer" in rows:
        extra["two_half_layer"] = bench_layer(cx)
    if "encodings" in rows:
        extra["readiness_encodings"] = bench_encodings(cx, args.fit_encodings)
    # each row's time against the ceiling for its own read/write mix
    if "self_sync_slots" in extra:
        r, c4 = extra["self_sync_slots"], dg.SLOTS
        a = bm.ll_unpack(c4.R, c4.n, c4.block_slots, completed_blocks=r["blocks"] - r["pending_blocks"])
        r["pass1_pct_mixed_ceiling"] = round(100 * mixed_ceiling_us(a["read"], a["write"], ceil) / r["pass1_us"], 1)
    if "self_sync_allgather" in extra:
        for r in extra["self_sync_allgather"]["by_payload"].values():
            a = bm.ll_gather(r["R"], r["words_per_rank"], dg.SLOTS.block_slots,
                             completed_blocks=r["pairs"] - r["pending_pairs"])
            r["pass1_pct_mixed_ceiling"] = round(100 * mixed_ceiling_us(a["read"], a["write"], ceil) / r["pass1_us"], 1)
    if "tokenweave_reduce_rmsnorm" in extra:
        r, c5 = extra["tokenweave_reduce_rmsnorm"], dg.TOKENWEAVE
        a = bm.reduce_rmsnorm(c5.R, c5.splits[0], c5.H, True, True)
        r["both_halves_pct_mixed_ceiling"] = round(
            100 * 2 * mixed_ceiling_us(a["read"], a["write"], ceil) / r["both_halves_us"], 1)
    detail = {"headline_calls": per_call, "headline_spread": sp, "rows": extra}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
        if args.oracle_by_config:
            detail["oracle_by_config"] = oracle_by_config()
    line["rows"] = row_summary(extra)
    # the full records on stderr, one line each: stdout carries the one compact headline record
    for k, v in detail.items():
        print(json.dumps({"detail": k, "record": v}), file=sys.stderr, flush=True)
    if args.detail_out:
        with open(args.detail_out, "w") as fh:
            json.dump(detail, fh, indent=1)
    print(json.dumps(line), flush=True)
    return 0


def _pct(gbps):
    return round(100 * gbps / HBM_PEAK_GBPS, 1)


def row_summary(extra: dict) -> dict:
    """One short entry per measured row for the headline record: microseconds, effective GB/s (algorithmic
    bytes / time) and % of the 8 TB/s HBM peak."""
    out = {}
    for k, r in extra.items():
        if k.startswith("two_step_"):
            out[k] = {"us": round(r["us_per_step"], 2), "GBps": r["GB/s"], "pct": _pct(r["GB/s"]),
                      "calls_us": [round(c["us"], 2) for c in r["calls"].values()]}
        elif k.startswith("share_"):
            out[k] = {"mode": "P", "us": round(r["us_per_step"], 2), "GBps": r["GB/s"], "pct": _pct(r["GB/s"]),
                      "calls_us": [round(c["us"], 2) for c in r["calls"].values()]}
        elif k.startswith("norm_first_"):
            sh = r["share"]
            out[k] = {"us": round(r["us_per_step"], 2), "GBps": r["GB/s"], "pct": _pct(r["GB/s"]),
                      "P_us": round(sh["us_per_step"], 2), "P_GBps": sh["GB/s"], "P_pct": _pct(sh["GB/s"])}
        elif k == "self_sync_slots":
            out[k] = {"pass1_us": r["pass1_us"], "GBps": r["pass1_GB/s"], "pct": _pct(r["pass1_GB/s"]),
                      "retry_us": r["retry_us"], "pending": r["pending_blocks"]}
            if "pass1_nocount_us" in r:
                out[k].update(nocount_us=r["pass1_nocount_us"], nocount_pct=_pct(r["pass1_nocount_GB/s"]))
        elif k == "self_sync_allgather":
            for tag, g in r["by_payload"].items():
                out[f"allgather_{tag}"] = {"pass1_us": g["pass1_us"], "GBps": g["pass1_GB/s"],
                                           "pct": _pct(g["pass1_GB/s"]), "retry_us": g["retry_us"]}
                if "pass1_nocount_us" in g:
                    out[f"allgather_{tag}"].update(nocount_us=g["pass1_nocount_us"],
                                                   nocount_pct=_pct(g["pass1_nocount_GB/s"]))
        elif k == "tokenweave_reduce_rmsnorm":
            ov = r["max_workgroups_sweep"].get("rows", {})
            out[k] = {"both_halves_us": r["both_halves_us"], "GBps": r["both_halves_GB/s"],
                      "pct": _pct(r["both_halves_GB/s"]), "overlap_makespan_us": ov.get("overlap_makespan_us"),
                      "serial_us": ov.get("serial_us")}
        elif k == "two_half_layer":
            t = r["by_T"].get("8192", {})
            out[k] = {"T": 8192, "pipelined_us": t.get("pipelined_us"), "serial_us": t.get("serial_halves_us"),
                      "unsplit_us": t.get("unsplit_us")}
        elif k == "readiness_encodings":
            out[k] = {"agree": r["choice_matches_fastest_measured"], "committed_regret": r.get("committed_table")}
        elif k == "warm_caches":
            out[k] = {"us": r["us_per_step"], "GBps": r["GB/s"]}
    return out


if __name__ == "__main__":
    sys.exit(main())
