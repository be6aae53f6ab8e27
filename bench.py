#!/usr/bin/env python3
"""Benchmark one MoE layer step on one MI355X: expert mapping, dispatch
(histogram, scan, stable scatter, mxfp8 quantisation) and combine + shared
expert + residual + RMSNorm, on the DeepSeek-V3-shaped workload
(Bs=512 tokens, H=7168, 256 expert instances = 32 ranks x 8, top-8,
Zipf(1.2) routing, one shared expert).

A step is one pass of the whole path: expert mapping and pruning, dispatch,
combine.  It is timed as two launches, moe_update_dispatch (the mapping fused
into the dispatch) and moe_combine_add_rmsnorm, the faster of the two forms on
this workload.  The pages' three-call sequence (moe_update_expert,
moe_dispatch, moe_combine_add_rmsnorm) is timed as well and reported under
"step_three_calls".

    python bench.py [--steps 500] [--warmup 50] [--sets 0] [--cpu-seconds 10]
    python bench.py --headline-only                      # the c3 step alone (for traces)
    python bench.py --copy-mb 256                        # copy kernel for counter scaling
    python bench.py --summarize-trace STATS.csv --out profiles/X.md --command CMD
    python bench.py --summarize-counters FETCH.csv WRITE.csv --kernel NAME \
                    --sources a.hip,b.h --out profiles/X.txt --command CMD1 --command CMD2
    python bench.py --summarize-copy FETCH.csv WRITE.csv --copy-mb 256 --out profiles/X.txt ...
    python bench.py --gemm [--gemm-formats]              # the expert GEMM row (its own line)
    python bench.py --gemm --gemm-dense                  # the GEMM on one instance of 4096 rows

By default the same line also carries, after the headline has been timed:
the step replayed from a captured HIP graph (the host's share of the eager
step), every other workload (c1, c2, c4, c4b) kernel by kernel, the
16-layer c5 stack captured in one graph, and the ceilings measured on the
same device with the measurement kernels of libmoe_calib.so (a streaming
copy, streams with each kernel's read/write mix, and each kernel's access
shape with its arithmetic taken out).  --headline-only leaves them out.

Prints one JSON line.  `value` is whole-step throughput in GB/s of
algorithmic bytes (each input read once, each output written once) with all
inputs resident in HBM: every timed loop rotates over enough buffer sets
(about 4 GB of its own traffic; COLD_BYTES) that the 256 MB Infinity Cache
serves little of it.  Per-kernel durations are taken with HIP events on the
stream the kernels run on, bracketing a run of back-to-back launches over the
rotating sets (events between the kernels of a step would add their own
packets to the step).  The CPU oracle runs the same step on the host cores,
on one core and on all of them, as a reference point.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch+combine HBM GB/s (% of peak) and tokens/s, Bs=512 H=7168 K=8"
# Timed loops rotate over buffer sets covering at least this many bytes of each loop's own
# traffic.  The 256 MB Infinity Cache does not replace least-recently-used lines only:
# with 440 MB of rotating sets it still served part of each launch (the c3 combine ran
# 3 us faster than its cold time); past about 2-4 GB the times stop falling.
COLD_BYTES = 4 << 30


def cold_sets(set_bytes, lo=2, hi=96):
    """Buffer sets a timed loop rotates over: COLD_BYTES of traffic in all."""
    return max(lo, min(hi, -(-COLD_BYTES // max(1, set_bytes))))


HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--sets", type=int, default=0,
                   help="rotating buffer sets of the headline step (0: enough for about "
                        "4 GB of traffic per kernel loop, so the Infinity Cache serves little)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="time budget of the CPU oracle baseline (0 = skip)")
    p.add_argument("--no-check", action="store_true", help="skip the parity check of step 0")
    p.add_argument("--headline-only", action="store_true",
                   help="time the c3 step and its kernels only (no other configs, c5 stack, "
                        "graph replay or ceilings): the command kernel traces are taken on")
    p.add_argument("--hot", action="store_true",
                   help="also time each kernel on one reused buffer set (hot Infinity Cache)")
    p.add_argument("--only-config", metavar="NAME", choices=("c1", "c2", "c4", "c4b"),
                   help="time one other workload's kernels only (its own JSON line): the "
                        "command its counter passes are taken on")
    p.add_argument("--variants", action="store_true",
                   help="also time the dispatch variants (static and per-instance scales)")
    p.add_argument("--gemm", action="store_true",
                   help="time the expert computation (grouped mxfp8 GEMM) instead; one JSON line")
    p.add_argument("--gemm-dense", action="store_true",
                   help="with --gemm: one instance of all 4096 rows instead of the Zipf split "
                        "(context: a shape whose rounds of 256 x 256 tiles are whole)")
    p.add_argument("--gemm-exponents", choices=("group-major", "row-major"),
                   default="group-major",
                   help="with --gemm: the activation exponents' layout (group-major: the "
                        "dispatch's MOE_Q_MXFP8_GM output; row-major: its MOE_Q_MXFP8 output)")
    p.add_argument("--gemm-formats", action="store_true",
                   help="with --gemm: also time the int8 formats (off by default so that a "
                        "kernel trace of --gemm covers the mxfp8 kernel alone)")
    p.add_argument("--copy-mb", type=int, default=0,
                   help="instead of the step, time a plain device copy of this many MB "
                        "(the reference kernel for counter scaling and achievable bandwidth)")
    g = p.add_argument_group("profile summaries (rocprofv3 CSV output -> profiles/*.txt|md)")
    g.add_argument("--summarize-trace", metavar="STATS_CSV",
                   help="kernel_stats.csv of a --kernel-trace --stats run")
    g.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="counter_collection.csv of a FETCH_SIZE run and of a WRITE_SIZE run")
    g.add_argument("--summarize-stalls", nargs="+", metavar="PMC_CSV",
                   help="per-dispatch counter means of --kernel over the given counter CSVs")
    g.add_argument("--summarize-copy", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="the same for the --copy-mb kernel: derives the counter scales")
    g.add_argument("--headline-of", metavar="BENCH_JSON",
                   help="summarise only the headline part of the traced run (the first "
                        "headline_launches dispatches of each kernel in that bench line)")
    g.add_argument("--kernel", help="kernel name (prefix) to summarise")
    g.add_argument("--sources", default="", help="comma-separated csrc files of that kernel")
    g.add_argument("--out", help="summary file to write")
    g.add_argument("--command", action="append", default=[],
                   help="the command(s) that produced the CSV files")
    g.add_argument("--title", default="rocprofv3 kernel statistics")
    g.add_argument("--workload-tag", default=None, help="workload named in a counter summary")
    return p.parse_args()


def copy_calibration(mb, steps, warmup):
    """A plain streaming copy of known size (libmoe_calib.so's stream kernel,
    non-temporal loads and stores): read mb MB, write mb MB, buffers rotating
    through COLD_BYTES.  The counter runs of this command calibrate the
    FETCH_SIZE / WRITE_SIZE scales."""
    import torch
    from combine_expert_amd import calib
    n = mb << 20
    nset = cold_sets(2 * n)
    src = [torch.empty(n, dtype=torch.uint8, device="cuda").fill_(7) for _ in range(nset)]
    dst = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(nset)]
    for k in range(warmup):
        calib.stream(src[k % nset], n, dst[k % nset], n)
    torch.cuda.synchronize()
    us = _events_us(torch, lambda k: calib.stream(src[k % nset], n, dst[k % nset], n), steps, 0)
    print(json.dumps({"copy_mb": mb, "kernel": "k_stream (libmoe_calib.so, non-temporal)",
                      "bytes_per_launch": 2 * n, "read_bytes": n, "write_bytes": n,
                      "avg_us": round(us, 3), "GBps": round(2 * n / us / 1e3, 1),
                      "buffer_sets": nset}), flush=True)


# ----------------------------------------------------------------- bytes

def algorithmic_bytes(Bs, H, K, E, rows, n_logical, F, quant_mode, n_scale, shared=True):
    """Bytes each kernel must move: every input read once, every output written once."""
    N = Bs * K
    upd = N * 4 + n_logical * F * 4 + N * 4 + N  # ids, table, balanced ids, mask
    code_b = 2 if quant_mode == 0 else 1
    scale_b = {0: 0, 2: 4, 3: 4, 4: 1}[quant_mode] * n_scale
    dsp = (Bs * H * 2 + N * 4 + N                 # x, ids, mask
           + rows * H * code_b + rows * scale_b   # coded rows and their scales
           + E * 4 + (E + 1) * 4 + 2 * N * 4)     # counts, offsets, src, assist
    cmb = (rows * H * 2 + 2 * N * 4               # expert rows, assist, scales
           + (Bs * H * 2 if shared else 0) + Bs * H * 2 + H * 2   # shared, residual, gamma
           + 2 * Bs * H * 2 + Bs * 4)             # y, x_out, rstd
    # fused mapping + dispatch: logical ids and the table in, mapped ids and mask
    # out, then the dispatch traffic without re-reading the mapped ids and mask
    fused = upd + dsp - (N * 4 + N)
    return dict(update_expert=upd, dispatch=dsp, update_dispatch=fused, combine=cmb)


# the csrc files each kernel's counter summaries are keyed to
DISPATCH_SRC = ("dispatch_impl.h", "dispatch.hip", "device.h", "kernels.h")
COMBINE_SRC = ("combine.hip", "device.h", "kernels.h")


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "combine_expert_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(kernel_file, digest_names):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if they
    were taken on the current kernel source."""
    path = os.path.join(PROFILES, kernel_file)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_digest") != source_digest(*digest_names):
        return None
    return d.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------- profile summaries

WORKLOAD_TAG = "Bs=512 H=7168 K=8 E=256 mxfp8 (bench.py)"
COPY_CAL = "copy_calibration.txt"


def short_name(kernel_name):
    """A kernel's name without namespaces, template arguments or parameters."""
    n = kernel_name.replace("(anonymous namespace)::", "")
    n = n.split("(")[0].split("<")[0].strip()
    return n.split("::")[-1].split(" ")[-1]


def _median_counter(path, kernel, counter):
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
            if r["Counter_Name"] == counter and short_name(r["Kernel_Name"]) == kernel]
    if not vals:
        raise SystemExit(f"{path}: no {counter} rows for a kernel named {kernel}*")
    return statistics.median(vals), len(vals)


def summarize_trace(args):
    """Per-kernel statistics from kernel_stats.csv, with p10 / p50 / p90 of the
    per-dispatch durations from the kernel_trace.csv beside it."""
    rows = list(csv.DictReader(open(args.summarize_trace)))
    durs = {}
    trace = args.summarize_trace.replace("kernel_stats.csv", "kernel_trace.csv")
    recs = []
    if os.path.exists(trace):
        recs = sorted(csv.DictReader(open(trace)), key=lambda r: int(r["Start_Timestamp"]))
    if args.headline_of and recs:
        # the headline part of the run: every dispatch up to the last combine of the
        # headline (the bench line's headline_launches counts them); later dispatches
        # belong to the other workloads the same command times
        with open(args.headline_of) as f:
            line = json.loads(next(ln for ln in f if ln.startswith("{")))
        n_cmb = line["headline_launches"]["k_combine"]
        cmb = [r for r in recs if "k_combine" in r["Kernel_Name"]]
        cut = int(cmb[n_cmb - 1]["End_Timestamp"])
        recs = [r for r in recs if int(r["Start_Timestamp"]) <= cut]
    for r in recs:
        durs.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if args.headline_of and recs:
        tot = sum(sum(d) for d in durs.values())
        rows = sorted(({"Name": n, "Calls": len(d), "AverageNs": 1e3 * sum(d) / len(d),
                        "MinNs": 1e3 * min(d), "MaxNs": 1e3 * max(d),
                        "Percentage": 100.0 * sum(d) / tot} for n, d in durs.items()),
                      key=lambda r: -r["Percentage"])

    def pct(v, q):
        v = sorted(v)
        return v[min(len(v) - 1, int(round(q * (len(v) - 1))))]

    lines = [f"# {args.title}", "", "Command (from the repository root, on one MI355X):", "",
             "```", *args.command, "```", "",
             "| kernel | calls | avg us | p10 us | p50 us | p90 us | min us | max us | share |",
             "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        d = durs.get(r["Name"], [])
        p = [f"{pct(d, q):.3f}" if d else "-" for q in (0.1, 0.5, 0.9)]
        lines.append(f"| {r['Name']} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                     f"{p[0]} | {p[1]} | {p[2]} | {float(r['MinNs']) / 1e3:.3f} | "
                     f"{float(r['MaxNs']) / 1e3:.3f} | {float(r['Percentage']):.1f}% |")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_counters(args):
    """HBM bytes per launch = FETCH_SIZE KiB x 1024 x fetch_scale + WRITE_SIZE KiB x 1024 x
    write_scale, the scales being what the counters read for a copy of known size."""
    fetch, nf = _median_counter(args.summarize_counters[0], args.kernel, "FETCH_SIZE")
    write, nw = _median_counter(args.summarize_counters[1], args.kernel, "WRITE_SIZE")
    with open(os.path.join(PROFILES, COPY_CAL)) as f:
        cal = json.load(f)
    rd = round(fetch * 1024 * cal["fetch_scale"])
    wr = round(write * 1024 * cal["write_scale"])
    names = [n for n in args.sources.split(",") if n]
    d = {"kernel": args.kernel, "workload": args.workload_tag or WORKLOAD_TAG,
         "source_digest": source_digest(*names),
         "source_files": names, "FETCH_SIZE_KiB_per_dispatch": fetch,
         "WRITE_SIZE_KiB_per_dispatch": write, "dispatches": [nf, nw],
         "fetch_scale": cal["fetch_scale"], "write_scale": cal["write_scale"],
         "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
         "hbm_bytes_per_launch": rd + wr, "commands": args.command,
         "note": f"median over the profiled dispatches of the kernel; scales from {COPY_CAL}"}
    with open(args.out, "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")


STALL_RATIOS = [
    # (name, numerator, denominator, unit); GRBM_GUI_ACTIVE is not used as a cycle base:
    # for kernels of tens of microseconds it also counts time outside the dispatch
    ("waves waiting on a wait counter / wave cycles", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES", ""),
    ("waves waiting to issue an instruction / wave cycles", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES", ""),
    ("LDS waits / all waits", "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY", ""),
    ("vector cache stalled on pending L2 data / CU busy cycles", "TCP_PENDING_STALL_CYCLES_sum",
     "SQ_BUSY_CU_CYCLES", ""),
    ("address unit stalled by the vector cache / address-unit busy", "TA_ADDR_STALLED_BY_TC_CYCLES_sum",
     "TA_BUSY_sum_est", ""),
    ("L2 hit rate", "TCC_HIT_sum", "_tcc_req", ""),
    ("mean L2 read latency seen by the vector cache", "TCP_TCC_READ_REQ_LATENCY_sum",
     "TCP_TCC_READ_REQ_sum", "cycles"),
]


def summarize_stalls(args):
    """Per-dispatch averages of rocprofv3 --pmc counters for one kernel, over
    several CSV files (one pass each), with ratios drawn from them."""
    vals, durs = {}, []
    for path in args.summarize_stalls:
        for r in csv.DictReader(open(path)):
            if short_name(r["Kernel_Name"]) != args.kernel:
                continue
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            if "End_Timestamp" in r and "Start_Timestamp" in r:
                durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if not vals:
        raise SystemExit(f"no counter rows for a kernel named {args.kernel}")
    avg = {k: statistics.mean(v) for k, v in vals.items()}
    dur = statistics.median(durs) if durs else None
    if "TCC_HIT_sum" in avg and "TCC_MISS_sum" in avg:
        avg["_tcc_req"] = avg["TCC_HIT_sum"] + avg["TCC_MISS_sum"]
    if "TA_BUSY_avr" in avg:
        avg["TA_BUSY_sum_est"] = avg["TA_BUSY_avr"] * 256  # one address unit per CU
    lines = [f"# {args.title}", "", "Commands (from the repository root, on one MI355X; one "
             "counter group per run):", "", "```", *args.command, "```", "",
             f"Kernel `{args.kernel}`; values are means per dispatch"
             + (f", median dispatch duration under counters {dur:.2f} us" if dur else "") + ".",
             "", "| counter | per dispatch |", "|---|---|"]
    for k in sorted(k for k in avg if not k.startswith("_") and k != "TA_BUSY_sum_est"):
        lines.append(f"| {k} | {avg[k]:.4g} |")
    lines += ["", "| ratio | value |", "|---|---|"]
    for name, num, den, unit in STALL_RATIOS:
        if num in avg and den in avg and avg[den]:
            v = avg[num] / avg[den]
            lines.append(f"| {name} | {v:.3g} {unit} |" if unit else f"| {name} | {v:.3f} |")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_copy(args):
    kernel = args.kernel or "k_stream"
    fetch, _ = _median_counter(args.summarize_copy[0], kernel, "FETCH_SIZE")
    write, _ = _median_counter(args.summarize_copy[1], kernel, "WRITE_SIZE")
    nbytes = args.copy_mb * (1 << 20)
    d = {"kernel": f"{kernel} (plain streaming copy, libmoe_calib.so)",
         "bytes_read_per_launch": nbytes, "bytes_written_per_launch": nbytes,
         "FETCH_SIZE_KiB_per_dispatch": fetch, "WRITE_SIZE_KiB_per_dispatch": write,
         "fetch_scale": round(nbytes / (fetch * 1024), 4),
         "write_scale": round(nbytes / (write * 1024), 4), "commands": args.command,
         "note": "Kernel traffic = FETCH_SIZE*1024*fetch_scale + WRITE_SIZE*1024*write_scale."}
    with open(args.out, "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")


# ----------------------------------------------------------------- GPU side

def make_set(wl, torch, moe):
    dev = torch.device("cuda")
    c = lambda t: None if t is None else t.contiguous().to(dev)
    s = dict(x=c(wl.x), ids=c(wl.logical_ids), scales=c(wl.scales), table=c(wl.table),
             eout=c(wl.expert_out), shared=c(wl.shared), residual=c(wl.residual),
             gamma=c(wl.gamma))
    s["bal_ids"] = torch.empty((wl.Bs, wl.K), dtype=torch.int32, device=dev)
    s["bal_mask"] = torch.empty((wl.Bs, wl.K), dtype=torch.uint8, device=dev)
    s["d"] = moe.dispatch_buffers(wl.Bs, wl.H, wl.K, wl.E, wl.quant_mode, wl.tile, dev)
    s["y"] = torch.empty((wl.Bs, wl.H), dtype=torch.bfloat16, device=dev)
    s["x_out"] = torch.empty((wl.Bs, wl.H), dtype=torch.bfloat16, device=dev)
    s["rstd"] = torch.empty((wl.Bs,), dtype=torch.float32, device=dev)
    return s


def step_args(wl, s, stream):
    """Pre-marshalled C-ABI argument tuples for one step on buffer set s."""
    d = s["d"]
    p = lambda t: None if t is None else t.data_ptr()
    n_logical, F = wl.table.shape
    upd = (p(s["ids"]), None, p(s["table"]), None, None, wl.Bs, wl.K, n_logical, F, wl.E,
           p(s["bal_ids"]), p(s["bal_mask"]), None, stream)
    dsp = (p(s["x"]), p(s["bal_ids"]), p(s["bal_mask"]), None, wl.Bs, wl.H, wl.K, wl.n_ranks,
           wl.local_experts, wl.quant_mode, wl.tile, None, 0, p(d["expand_x"]),
           p(d["expand_scales"]),
           p(d["expert_counts"]), p(d["expert_offsets"]), p(d["expand_src"]),
           p(d["assist_dst"]), None, stream)
    fused = (p(s["x"]), p(s["ids"]), None, p(s["table"]), None, None, wl.Bs, wl.H, wl.K,
             n_logical, F, wl.n_ranks, wl.local_experts, wl.quant_mode, wl.tile, None, 0,
             p(s["bal_ids"]), p(s["bal_mask"]), p(d["expand_x"]), p(d["expand_scales"]),
             p(d["expert_counts"]), p(d["expert_offsets"]), p(d["expand_src"]),
             p(d["assist_dst"]), None, stream)
    cmb = (p(s["eout"]), p(d["assist_dst"]), p(s["scales"]), p(s["shared"]), p(s["residual"]),
           p(s["gamma"]), wl.eps, wl.Bs, wl.H, wl.K, wl.shared_mode, p(s["y"]), p(s["x_out"]),
           p(s["rstd"]), None, stream)
    return upd, dsp, fused, cmb


# ----------------------------------------------------------------- c5: a chained stack

def make_stack(wls, torch, moe):
    """Device buffers of a chained layer stack: layer l + 1 reads y_l as its
    x and x_out_l as its residual (layer 0 reads the first workload's x and
    residual)."""
    dev = torch.device("cuda")
    c = lambda t: None if t is None else t.contiguous().to(dev)
    layers = []
    for wl in wls:
        s = dict(ids=c(wl.logical_ids), scales=c(wl.scales), table=c(wl.table),
                 eout=c(wl.expert_out), shared=c(wl.shared), gamma=c(wl.gamma))
        s["bal_ids"] = torch.empty((wl.Bs, wl.K), dtype=torch.int32, device=dev)
        s["bal_mask"] = torch.empty((wl.Bs, wl.K), dtype=torch.uint8, device=dev)
        s["d"] = moe.dispatch_buffers(wl.Bs, wl.H, wl.K, wl.E, wl.quant_mode, wl.tile, dev)
        s["y"] = torch.empty((wl.Bs, wl.H), dtype=torch.bfloat16, device=dev)
        s["x_out"] = torch.empty((wl.Bs, wl.H), dtype=torch.bfloat16, device=dev)
        s["rstd"] = torch.empty((wl.Bs,), dtype=torch.float32, device=dev)
        layers.append(s)
    return dict(x0=c(wls[0].x), r0=c(wls[0].residual), layers=layers)


def stack_calls(wls, st, lib, stream):
    """(function, C-ABI arguments) of every call of one pass over the stack:
    per layer the mapping fused into the dispatch, then the combine."""
    p = lambda t: None if t is None else t.data_ptr()
    calls = []
    for l, (wl, s) in enumerate(zip(wls, st["layers"])):
        x = st["x0"] if l == 0 else st["layers"][l - 1]["y"]
        res = st["r0"] if l == 0 else st["layers"][l - 1]["x_out"]
        d = s["d"]
        n_logical, F = wl.table.shape
        calls.append((lib.moe_update_dispatch,
                      (p(x), p(s["ids"]), None, p(s["table"]), None, None, wl.Bs, wl.H, wl.K,
                       n_logical, F, wl.n_ranks, wl.local_experts, wl.quant_mode, wl.tile, None,
                       0, p(s["bal_ids"]), p(s["bal_mask"]), p(d["expand_x"]),
                       p(d["expand_scales"]), p(d["expert_counts"]), p(d["expert_offsets"]),
                       p(d["expand_src"]), p(d["assist_dst"]), None, stream)))
        calls.append((lib.moe_combine_add_rmsnorm,
                      (p(s["eout"]), p(d["assist_dst"]), p(s["scales"]), p(s["shared"]), p(res),
                       p(s["gamma"]), wl.eps, wl.Bs, wl.H, wl.K, wl.shared_mode, p(s["y"]),
                       p(s["x_out"]), p(s["rstd"]), None, stream)))
    return calls


def run_calls(calls):
    for f, a in calls:
        if f(*a):
            raise RuntimeError("a library call returned a non-zero status")


def capture_stack(wls, st, lib, torch):
    """One HIP graph holding every launch of a pass over the stack (the calls
    only enqueue kernels: no allocation, no memset, no host synchronisation)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_calls(stack_calls(wls, st, lib, side.cuda_stream))  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_calls(stack_calls(wls, st, lib, torch.cuda.current_stream().cuda_stream))
    return g


def time_stack(moe, torch, n_layers, replays, warmup):
    """The c5 stack (16 c3-shaped layers, int8 per token, chained) captured in
    one graph: microseconds per replay, per layer, and the stack's bytes."""
    from combine_expert_amd import workloads as W
    wls = W.make_c5_layers(n_layers)
    st = make_stack(wls, torch, moe)
    lib = moe.raw()
    g = capture_stack(wls, st, lib, torch)
    calls = stack_calls(wls, st, lib, torch.cuda.current_stream().cuda_stream)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(replays):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / replays

    t = timed(g.replay)
    t_eager = timed(lambda: run_calls(calls))
    total = 0
    for wl, s in zip(wls, st["layers"]):
        rows = int(s["d"]["expert_offsets"][-1].item())
        nb = algorithmic_bytes(wl.Bs, wl.H, wl.K, wl.E, rows, wl.table.shape[0],
                               wl.table.shape[1], wl.quant_mode,
                               moe.n_scale_entries(wl.quant_mode, wl.H, wl.tile), shared=True)
        total += nb["update_dispatch"] + nb["combine"]
    Bs = wls[0].Bs
    return {"layers": n_layers, "graph_replays": replays, "us_per_replay": round(t * 1e6, 2),
            "us_per_layer": round(t * 1e6 / n_layers, 3),
            "us_per_layer_eager": round(t_eager * 1e6 / n_layers, 3), "bytes": total,
            "GBps": round(total / t / 1e9, 2),
            "frac_of_hbm_peak": round(total / t / 1e9 / HBM_PEAK_GBS, 4),
            "tokens_per_s_per_layer": round(Bs * n_layers / t, 1),
            "workload": "16 chained layers of Bs=512 H=7168 K=8 E=256 (32 x 8), Zipf(1.2), "
                        "int8 per token, 1 shared expert; x_{l+1} = y_l, residual_{l+1} = "
                        "x_out_l; per layer the fused mapping + dispatch and the combine; "
                        "one HIP graph per pass"}


# ----------------------------------------------------------------- dispatch variants

VARIANTS = [  # (quant mode, scales kind, tile) at the c3 shapes; mode 5: mxfp8, exponents
    # in the expert GEMM's group-major order
    (1, 1, 0), (1, 2, 0), (1, 3, 0), (2, 0, 0), (2, 3, 0), (3, 0, 128), (3, 3, 128), (4, 0, 0),
    (5, 0, 0)]


def dispatch_variant_bytes(Bs, H, K, E, rows, mode, kind, tile):
    """Algorithmic bytes of one dispatch: the scales input read once, one byte per code."""
    N = Bs * K
    qs = {0: 0, 1: 4, 2: H * 4, 3: E * H * 4}[kind]
    sc = {1: 0, 2: 4, 3: 4 * -(-H // tile) if tile else 0, 4: H // 32, 5: H // 32}[mode]
    return (Bs * H * 2 + N * 4 + N + qs + rows * H + rows * sc + E * 4 + (E + 1) * 4 + 2 * N * 4)


def dispatch_variants(moe, torch, n):
    """Per-launch duration (HIP events around n back-to-back launches over
    rotating buffer sets) of moe_dispatch in the static and scaled modes, and in mxfp8
    with either exponent layout."""
    from combine_expert_amd import workloads as W
    out = []
    for mode, kind, tile in VARIANTS:
        wl = W.make_c3(seed=3200 + mode, quant_mode=mode, with_expert_out=False)
        wl.tile = tile
        dev = torch.device("cuda")
        sets = cold_sets(wl.Bs * wl.H * 2 + wl.Bs * wl.K * wl.H, hi=64)
        qs = W.make_quant_scales(3300 + mode * 10 + kind, kind, wl.E, wl.H)
        qs = None if qs is None else qs.to(dev)
        ids = wl.logical_ids.to(dev)  # identity table: logical ids are instance ids
        bufs = [(wl.x.to(dev), moe.dispatch_buffers(wl.Bs, wl.H, wl.K, wl.E, mode, tile, dev))
                for _ in range(sets)]
        stream = torch.cuda.current_stream()
        f = moe.raw().moe_dispatch
        p = lambda t: None if t is None else t.data_ptr()
        argv = [(p(x), p(ids), None, None, wl.Bs, wl.H, wl.K, wl.n_ranks, wl.local_experts, mode,
                 tile,
                 p(qs), kind, p(d["expand_x"]), p(d["expand_scales"]), p(d["expert_counts"]),
                 p(d["expert_offsets"]), p(d["expand_src"]), p(d["assist_dst"]), None,
                 stream.cuda_stream) for x, d in bufs]
        for a in argv:
            if f(*a):
                raise RuntimeError("moe_dispatch returned a non-zero status")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(n):
            f(*argv[k % sets])
        e1.record(stream)
        e1.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        rows = int(bufs[0][1]["expert_offsets"][-1].item())
        nb = dispatch_variant_bytes(wl.Bs, wl.H, wl.K, wl.E, rows, mode, kind, tile)
        out.append({"quant_mode": mode, "scales": ["none", "one", "row", "per-instance"][kind],
                    "tile": tile, "avg_us": round(us, 3), "bytes": nb,
                    "GBps": round(nb / (us * 1e-6) / 1e9, 1), "buffer_sets": sets})
        del bufs
    return out


# ----------------------------------------------------------------- other configs

def config_table(moe, torch, n, only=None):
    """Per-launch durations (HIP events around n back-to-back launches over
    rotating buffer sets) of the three calls and the fused call on the other
    workloads at full size, with their algorithmic bytes."""
    from combine_expert_amd import workloads as W
    rows = []
    for name in ("c1", "c2", "c4", "c4b") if only is None else (only,):
        wl = W.make(name)
        if wl.expert_out is None:  # the identity + bias expert: any bf16 rows serve for timing
            wl.expert_out = torch.randn(wl.Bs * wl.K, wl.H).bfloat16()
        stream = torch.cuda.current_stream()
        # the dispatch is the smallest loop: rotate enough sets for its traffic
        est = wl.Bs * wl.H * 2 + wl.Bs * wl.K * wl.H
        sets = cold_sets(est, hi=64)
        bufs = [make_set(wl, torch, moe) for _ in range(sets)]
        prune = wl.prune_thr is not None
        dev = torch.device("cuda")
        extra = dict(sc=wl.scales.to(dev) if prune else None,
                     thr=wl.prune_thr.to(dev) if prune else None,
                     tm=None if wl.token_mask is None else wl.token_mask.to(dev))
        p = lambda t: None if t is None else t.data_ptr()
        argv = []
        for s in bufs:
            upd, dsp, fused, cmb = step_args(wl, s, stream.cuda_stream)
            n_logical, F = wl.table.shape
            upd = (upd[0], p(extra["sc"]), upd[2], p(extra["thr"]), p(extra["tm"])) + upd[5:]
            fused = (fused[0], fused[1], p(extra["sc"]), fused[3], p(extra["thr"]),
                     p(extra["tm"])) + fused[6:]
            argv.append((upd, dsp, fused, cmb))
        lib = moe.raw()
        fns = (lib.moe_update_expert, lib.moe_dispatch, lib.moe_update_dispatch,
               lib.moe_combine_add_rmsnorm)
        for a in argv:  # one full step per set: the dispatch outputs feed the combine
            for j in (0, 1, 3):
                if fns[j](*a[j]):
                    raise RuntimeError(f"{name}: a library call failed")
        us = []
        for j in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for k in range(n):
                fns[j](*argv[k % sets][j])
            e1.record(stream)
            e1.synchronize()
            us.append(e0.elapsed_time(e1) * 1e3 / n)
        nrows = int(bufs[0]["d"]["expert_offsets"][-1].item())
        nb = algorithmic_bytes(wl.Bs, wl.H, wl.K, wl.E, nrows, wl.table.shape[0],
                               wl.table.shape[1], wl.quant_mode,
                               moe.n_scale_entries(wl.quant_mode, wl.H, wl.tile),
                               shared=wl.shared is not None)
        keys = ("update_expert", "dispatch", "update_dispatch", "combine")
        row = {"config": name, "Bs": wl.Bs, "H": wl.H, "K": wl.K, "E": wl.E,
               "quant_mode": wl.quant_mode, "rows_dispatched": nrows, "buffer_sets": sets,
               **{k: {"avg_us": round(u, 3), "bytes": nb[k],
                      "GBps": round(nb[k] / (u * 1e-6) / 1e9, 1),
                      "frac": round(nb[k] / (u * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
                  for k, u in zip(keys, us)}}
        if wl.quant_mode != 0:  # the measurement kernels move 8-bit dispatch rows
            row["shape_ceilings"] = shape_ceilings(torch, wl, bufs[0]["d"]["assist_dst"], nrows, n)
        del bufs, argv
        rows.append(row)
    return rows


def shape_ceilings(torch, wl, assist, nrows, n):
    """The dispatch's and the combine's access shapes on this workload's own routing
    (the measurement kernels of libmoe_calib.so, stores non-temporal as in the library,
    buffers rotating through COLD_BYTES): what the part sustains for each kernel's
    traffic in its block-per-token shape."""
    from combine_expert_amd import calib
    dev = torch.device("cuda")
    Bs, H, K = wl.Bs, wl.H, wl.K
    shared = wl.shared is not None
    res = {}
    db = Bs * H * 2 + Bs * K * 4 + nrows * H
    nsets = cold_sets(db, hi=64)
    xs = [torch.ones((Bs, H), dtype=torch.bfloat16, device=dev) for _ in range(nsets)]
    outs = [torch.empty((nrows, H), dtype=torch.uint8, device=dev) for _ in range(nsets)]
    us = _events_us(torch, lambda k: calib.scatter_shape(xs[k % nsets], assist, nrows,
                                                         outs[k % nsets], calib.STORE_STREAM), n)
    res["dispatch_shape"] = {"avg_us": round(us, 3), "bytes": db,
                             "frac": round(db / us / 1e3 / HBM_PEAK_GBS, 4)}
    del xs, outs
    cb = nrows * H * 2 + (2 if shared else 1) * Bs * H * 2 + H * 2 + Bs * K * 4 + 2 * Bs * H * 2
    nsets = cold_sets(cb, hi=64)
    eo = [torch.ones((nrows, H), dtype=torch.bfloat16, device=dev) for _ in range(nsets)]
    aa = [torch.ones((Bs, H), dtype=torch.bfloat16, device=dev) for _ in range(nsets)]
    bb = [torch.ones((Bs, H), dtype=torch.bfloat16, device=dev) if shared else None
          for _ in range(nsets)]
    o1 = [torch.empty((Bs, H), dtype=torch.bfloat16, device=dev) for _ in range(nsets)]
    o2 = [torch.empty((Bs, H), dtype=torch.bfloat16, device=dev) for _ in range(nsets)]
    g = torch.ones(H, dtype=torch.bfloat16, device=dev)
    us = _events_us(torch, lambda k: calib.gather_shape(
        eo[k % nsets], assist, aa[k % nsets], bb[k % nsets], g, nrows, o1[k % nsets],
        o2[k % nsets], calib.STORE_STREAM), n)
    res["combine_shape"] = {"avg_us": round(us, 3), "bytes": cb,
                            "frac": round(cb / us / 1e3 / HBM_PEAK_GBS, 4)}
    return res


# ----------------------------------------------------------------- ceilings

def _events_us(torch, fn, n, warm=10):
    """Average duration of fn(k), k = 0 .. n-1, enqueued back to back between two
    HIP events on the current stream."""
    stream = torch.cuda.current_stream()
    for k in range(warm):
        fn(k)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for k in range(n):
        fn(k)
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def ceilings(torch, n, wl, step_set, nb, rows):
    """What this device sustains for the same traffic, from the measurement
    kernels of libmoe_calib.so, each over buffers rotating through COLD_BYTES:
    a plain streaming copy, streams with the combine's and the dispatch's
    read/write mix at the c3 sizes, and the two kernels' access shapes (the
    c3 routing of the headline step) with their arithmetic taken out; each
    with its stores in every cache policy (the best is the ceiling)."""
    from combine_expert_amd import calib
    dev = torch.device("cuda")
    out = {"note": "measurement kernels of libmoe_calib.so (include/moe_calib.h); GB/s of the "
                   "bytes each moves, HIP events over back-to-back launches, buffers rotating "
                   "through about 4 GB; per store policy, best first"}

    def entry(bytes_, times):
        res = {"bytes": bytes_}
        for pol, us in sorted(times.items(), key=lambda kv: kv[1]):
            res[pol] = {"avg_us": round(us, 3), "GBps": round(bytes_ / us / 1e3, 1),
                        "frac": round(bytes_ / us / 1e3 / HBM_PEAK_GBS, 4)}
        best = min(times, key=times.get)
        res["best"] = best
        res["frac"] = res[best]["frac"]
        return res

    def stream_case(name, rbytes, wbytes):
        nsets = cold_sets(rbytes + wbytes)
        src = [torch.empty(rbytes, dtype=torch.uint8, device=dev) for _ in range(nsets)]
        dst = [torch.empty(wbytes, dtype=torch.uint8, device=dev) for _ in range(nsets)]
        for t in src:
            t.fill_(3)
        times = {pol: _events_us(torch, lambda k: calib.stream(src[k % nsets], rbytes,
                                                               dst[k % nsets], wbytes, code), n)
                 for pol, code in calib.POLICIES.items()}
        out[name] = entry(rbytes + wbytes, times)
        out[name].update(read_bytes=rbytes, write_bytes=wbytes)
        del src, dst

    stream_case("copy_256MB", 256 << 20, 256 << 20)
    cr = nb["combine"] - 2 * wl.Bs * wl.H * 2 - wl.Bs * 4
    stream_case("stream_combine_mix", cr // 16 * 16, (nb["combine"] - cr) // 16 * 16)
    dr = wl.Bs * wl.H * 2 + wl.Bs * wl.K * 5
    stream_case("stream_dispatch_mix", dr // 16 * 16, (nb["dispatch"] - dr) // 16 * 16)

    # the kernels' access shapes on the headline's routing (c3)
    assist = step_set["d"]["assist_dst"]
    Bs, H, K = wl.Bs, wl.H, wl.K
    nsets = cold_sets(nb["dispatch"], hi=64)
    xs = [torch.empty((Bs, H), dtype=torch.bfloat16, device=dev).fill_(1.0) for _ in range(nsets)]
    outs = [torch.empty((rows, H), dtype=torch.uint8, device=dev) for _ in range(nsets)]
    times = {pol: _events_us(torch, lambda k: calib.scatter_shape(xs[k % nsets], assist, rows,
                                                                  outs[k % nsets], code), n)
             for pol, code in calib.POLICIES.items()}
    out["dispatch_shape"] = entry(Bs * H * 2 + Bs * K * 4 + rows * H, times)
    out["dispatch_shape"]["what"] = ("block per token: its row read, one byte per element "
                                     "written to each of its K rows (no routing, no coding)")
    del xs, outs
    nsets = cold_sets(nb["combine"], hi=64)
    eo = [torch.empty((rows, H), dtype=torch.bfloat16, device=dev).fill_(1.0) for _ in range(nsets)]
    aa = [torch.empty((Bs, H), dtype=torch.bfloat16, device=dev).fill_(1.0) for _ in range(nsets)]
    bb = [torch.empty((Bs, H), dtype=torch.bfloat16, device=dev).fill_(1.0) for _ in range(nsets)]
    o1 = [torch.empty((Bs, H), dtype=torch.bfloat16, device=dev) for _ in range(nsets)]
    o2 = [torch.empty((Bs, H), dtype=torch.bfloat16, device=dev) for _ in range(nsets)]
    g = torch.ones(H, dtype=torch.bfloat16, device=dev)
    times = {pol: _events_us(torch, lambda k: calib.gather_shape(
        eo[k % nsets], assist, aa[k % nsets], bb[k % nsets], g, rows, o1[k % nsets],
        o2[k % nsets], code), n) for pol, code in calib.POLICIES.items()}
    out["combine_shape"] = entry(rows * H * 2 + 2 * Bs * H * 2 + H * 2 + Bs * K * 4
                                 + 2 * Bs * H * 2, times)
    out["combine_shape"]["what"] = ("block per token: its K expert rows, two token rows and "
                                    "gamma read, two rows written, one block barrier (no "
                                    "arithmetic)")
    return out


def step_graph(torch, fns, argv, calls, n, t_eager, step_bytes, Bs):
    """The headline step replayed from a captured HIP graph holding one step
    per buffer set (the same launches, no host issue between them): the
    per-step time next to the eager one shows how much of the eager step is
    host issue."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        sp = side.cuda_stream
        for a in argv:
            for c in calls:
                a2 = a[c][:-1] + (sp,)
                if fns[c](*a2):
                    raise RuntimeError("a library call failed under capture")
    torch.cuda.current_stream().wait_stream(side)
    reps = max(1, n // len(argv))
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / (reps * len(argv))
    return {"steps": reps * len(argv), "ms_per_step": round(t * 1e3, 5),
            "GBps": round(step_bytes / t / 1e9, 2), "tokens_per_s": round(Bs / t, 1),
            "frac_of_hbm_peak": round(step_bytes / t / 1e9 / HBM_PEAK_GBS, 4),
            "host_issue_share_of_eager_step": round(max(0.0, 1.0 - t / t_eager), 4),
            "note": f"one HIP graph of {len(argv)} steps (one per buffer set), replayed"}


def check_parity(wl, s, oracle, np):
    """Step-0 outputs against the oracle: routing/codes exact, y within tolerance."""
    oi, om, _ = oracle.update_expert(wl.logical_ids.numpy(), None, wl.table.numpy(), None, None,
                                     wl.E)
    od = oracle.dispatch(oracle.bf16_bits(wl.x), oi, om, wl.n_ranks, wl.local_experts,
                         wl.quant_mode, wl.tile)
    d = s["d"]
    total = int(od["offsets"][-1])
    ok = (np.array_equal(s["bal_ids"].cpu().numpy(), oi)
          and np.array_equal(s["bal_mask"].cpu().numpy(), om)
          and np.array_equal(d["assist_dst"].cpu().numpy(), od["assist"])
          and np.array_equal(d["expert_offsets"].cpu().numpy(), od["offsets"])
          and np.array_equal(d["expand_x"].view(__import__("torch").uint8).cpu().numpy()[:total],
                             od["expand_x"].view(np.uint8)[:total])
          and np.array_equal(d["expand_scales"].cpu().numpy()[:total], od["scales"][:total]))
    oy, _, _ = oracle.combine(oracle.bf16_bits(wl.expert_out), od["assist"], wl.scales.numpy(),
                              oracle.bf16_bits(wl.shared), oracle.bf16_bits(wl.residual),
                              oracle.bf16_bits(wl.gamma), wl.eps, wl.shared_mode)
    ref = (oy.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = s["y"].float().cpu().numpy()
    ok = ok and bool(np.all(np.abs(got - ref) <= 2e-2 + 1e-2 * np.abs(ref)))
    return ok


def cpu_baseline(wl, oracle, np, budget_s, step_bytes):
    """The oracle as it stands (plain C), the whole step on the same inputs:
    first on one core, then with its per-token loops on every core the process
    may use (the routing stays sequential).  Each for about budget_s / 2."""
    ids = wl.logical_ids.numpy()
    table = wl.table.numpy()
    xb = oracle.bf16_bits(wl.x)
    eob = oracle.bf16_bits(wl.expert_out)
    shb, rsb, gmb = (oracle.bf16_bits(wl.shared), oracle.bf16_bits(wl.residual),
                     oracle.bf16_bits(wl.gamma))
    sc = wl.scales.numpy()
    cores = len(os.sched_getaffinity(0))

    def run(threads, seconds):
        used = oracle.set_threads(threads)
        times = []
        t_end = time.perf_counter() + seconds
        while True:
            t0 = time.perf_counter()
            oi, om, _ = oracle.update_expert(ids, None, table, None, None, wl.E)
            od = oracle.dispatch(xb, oi, om, wl.n_ranks, wl.local_experts, wl.quant_mode, wl.tile)
            oracle.combine(eob, od["assist"], sc, shb, rsb, gmb, wl.eps, wl.shared_mode)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() >= t_end or len(times) >= 50:
                break
        return used, statistics.median(times), len(times)

    one, t1, n1 = run(1, budget_s / 2)
    many, tm, nm = run(cores, budget_s / 2)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         "")
    except OSError:
        pass
    return {"value": round(step_bytes / tm / 1e9, 3), "unit": "GB/s", "cores": many,
            "kind": "oracle", "host_cpu": model, "host_cores_available": cores,
            "sample": f"the full step (update + dispatch + combine) on all {wl.Bs} tokens of the "
                      f"workload, repeated for about {budget_s / 2:.0f} s per thread count, "
                      f"median: {many} threads {tm * 1e3:.1f} ms ({nm} runs), 1 thread "
                      f"{t1 * 1e3:.1f} ms ({n1} runs)",
            "tokens_per_s": round(wl.Bs / tm, 1),
            "single_core": {"value": round(step_bytes / t1 / 1e9, 3), "unit": "GB/s",
                            "cores": one, "tokens_per_s": round(wl.Bs / t1, 1)}}


# ----------------------------------------------------------------- expert GEMM row

FP8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA
INT8_PEAK_TOPS = 5000.0    # MI355X dense int8 MFMA
GEMM_METRIC = "expert GEMM TFLOP/s (mxfp8 x mxfp8 -> bf16, fp32 accumulate)"
GEMM_TAG = "8 instances, 4096 rows (Zipf split), H=7168 -> N=4096, mxfp8 (bench.py --gemm)"


def gemm_sample(g, np, oracle, rows_per_instance=3, n_cols=256, seed=9):
    """Rows (first, middle, last of each instance) and columns of a sub-problem the oracle
    finishes quickly; returns (rows, cols, y64, abs64)."""
    rows, inst = [], []
    for e in range(g.E):
        lo, hi = int(g.offsets[e]), int(g.offsets[e + 1])
        pick = sorted({lo, (lo + hi) // 2, hi - 1})[:rows_per_instance] if hi > lo else []
        rows += pick
        inst += [e] * len(pick)
    rows = np.array(rows)
    cols = np.sort(np.random.default_rng(seed).choice(g.N, min(n_cols, g.N), replace=False))
    off = np.zeros(g.E + 1, np.int32)
    off[1:] = np.cumsum(np.bincount(np.array(inst), minlength=g.E))
    _, y64, abs64 = oracle.expert_gemm_mx(g.a[rows], g.a_sc[rows], off,
                                          np.ascontiguousarray(g.w[:, cols]),
                                          np.ascontiguousarray(g.w_sc[:, cols]))
    return rows, cols, y64, abs64


def gemm_cpu_baseline(g, np, oracle, budget_s):
    """The oracle on whole output rows (all N columns) of the workload, as many rows as fit
    the budget after a one-row probe; TFLOP/s of that sample."""
    e = int(np.argmax(np.diff(g.offsets)))
    lo = int(g.offsets[e])

    def run(n):
        off = np.zeros(g.E + 1, np.int32)
        off[e + 1:] = n
        t0 = time.perf_counter()
        oracle.expert_gemm_mx(g.a[lo:lo + n], g.a_sc[lo:lo + n], off, g.w, g.w_sc)
        return time.perf_counter() - t0

    t1 = run(1)
    n = max(1, min(int(budget_s / t1), int(g.offsets[e + 1]) - lo))
    t = run(n) if n > 1 else t1
    fl = 2.0 * n * g.N * g.Kd
    return {"value": round(fl / t / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} whole output rows (all {g.N} columns, K={g.Kd}) of instance {e}, "
                      f"{t:.1f} s",
            "host_cores_available": len(os.sched_getaffinity(0))}


def ffn_figures(args, g, argv, ys, off, n_sets, K, lib, moe, W, torch, dev, stream):
    """The whole expert FFN of the rank: this launch's output y1 = [gate | up] (N = 2I),
    the activation (moe_expert_swiglu: bf16 silu(gate) * up coded as mxfp8, exponents
    group-major) and the second projection back to H (moe_expert_gemm with K = I), each
    weight set twice so the weights cannot stay in the Infinity Cache.  Reported: the
    activation kernel against the HBM peak (its y1 input was just written by the first
    projection, as in the FFN), the second projection against the fp8 peak, and the three
    launches as one FFN step."""
    I = g.N // 2
    rows = g.rows
    g2 = W.make_gemm_case(3300, g.counts, g.Kd, I, name="g3 second projection")
    w2 = [torch.from_numpy(g2.w).to(dev) for _ in range(n_sets)]
    w2s = [moe.pack_mx_weight_scales(torch.from_numpy(g2.w_sc).to(dev)) for _ in range(n_sets)]
    codes = [torch.empty((rows, I), dtype=torch.uint8, device=dev) for _ in range(n_sets)]
    scs = [torch.empty((-(-I // 512), rows, 16), dtype=torch.uint8, device=dev)
           for _ in range(n_sets)]
    y2 = [torch.empty((rows, g.Kd), dtype=torch.bfloat16, device=dev) for _ in range(n_sets)]
    gm = moe.QUANT_MXFP8_GM
    act_argv = [(ys[k].data_ptr(), off.data_ptr(), g.E, rows, I, gm, codes[k].data_ptr(),
                 scs[k].data_ptr(), None, None, stream.cuda_stream) for k in range(n_sets)]
    g2_argv = [(codes[k].data_ptr(), scs[k].data_ptr(), off.data_ptr(), g.E, rows,
                w2[k].data_ptr(), w2s[k].data_ptr(), g.Kd, I, gm, y2[k].data_ptr(), None,
                stream.cuda_stream) for k in range(n_sets)]
    act, gemm = lib.moe_expert_swiglu, lib.moe_expert_gemm

    def timed(fn):
        for k in range(args.warmup):
            fn(k)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(K):
            fn(k)
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / K

    def step(k):
        a = k % n_sets
        if gemm(*argv[a]) | act(*act_argv[a]) | gemm(*g2_argv[a]):
            raise RuntimeError("an expert FFN call returned a non-zero status")

    def act_only(k):
        gemm(*argv[k % n_sets])   # y1 freshly written, as in the FFN
        if act(*act_argv[k % n_sets]):
            raise RuntimeError("moe_expert_swiglu returned a non-zero status")

    t_step = timed(step)
    t_gemm1_act = timed(act_only)
    t_gemm1 = timed(lambda k: gemm(*argv[k % n_sets]))
    t_act = t_gemm1_act - t_gemm1
    t_act_alone = timed(lambda k: act(*act_argv[k % n_sets]))
    t_g2 = timed(lambda k: gemm(*g2_argv[k % n_sets]))
    n = int(g.offsets[-1])
    f1, f2 = 2.0 * n * g.N * g.Kd, 2.0 * n * g.Kd * I
    act_bytes = n * 2 * I * 2 + n * I + n * (I // 32)
    tf = lambda f, u: f / (u * 1e-6) / 1e12
    return {
        "workload": (f"the rank's expert FFN: {g.E} instances, {n} rows, H={g.Kd} -> 2I={g.N} "
                     f"(gate | up), silu(gate) * up coded as mxfp8, I={I} -> H={g.Kd}"),
        "step_us": round(t_step, 3),
        "TFLOPs": round(tf(f1 + f2, t_step), 1),
        "frac_of_fp8_peak": round(tf(f1 + f2, t_step) / FP8_PEAK_TFLOPS, 4),
        "activation": {"kernel": "k_expert_swiglu", "bound": "hbm",
                       "avg_us": round(t_act, 3), "bytes": act_bytes,
                       "GBps": round(act_bytes / (t_act * 1e-6) / 1e9, 1),
                       "frac": round(act_bytes / (t_act * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                       "how": "first projection + activation minus first projection alone, "
                              "HIP events, y1 read right after the projection wrote it",
                       "alone_us": round(t_act_alone, 3),
                       "alone_GBps": round(act_bytes / (t_act_alone * 1e-6) / 1e9, 1),
                       "alone_how": "back-to-back launches over the two y1 sets (67 MB: "
                                    "partly served by the Infinity Cache)"},
        "second_projection": {"avg_us": round(t_g2, 3), "flops": f2,
                              "TFLOPs": round(tf(f2, t_g2), 1),
                              "frac_of_fp8_peak": round(tf(f2, t_g2) / FP8_PEAK_TFLOPS, 4)},
    }


def gemm_main(args):
    import numpy as np
    import torch

    from combine_expert_amd import build as hip_build
    if hip_build.stale():
        hip_build.build()
    from combine_expert_amd import moe
    from combine_expert_amd import workloads as W

    g = W.make_gemm_case(9001, [4096], 4096, 7168, name="dense") if args.gemm_dense else W.make_g3()
    torch.cuda.init()
    stream = torch.cuda.current_stream()
    lib = moe.raw()
    dev = torch.device("cuda")
    n_sets = 2   # two weight copies (2 x 235 MB) so a launch cannot hit in the 256 MB MALL
    a = torch.from_numpy(g.a).to(dev)
    gm = args.gemm_exponents == "group-major"
    mx_mode = moe.QUANT_MXFP8_GM if gm else moe.QUANT_MXFP8
    asc = torch.from_numpy(g.a_sc).to(dev)
    if gm:   # [rows, H/32] -> [H/512, rows, 16] (H = 7168: whole groups, no pad)
        asc = asc.view(g.rows, g.Kd // 512, 16).permute(1, 0, 2).contiguous()
    off = torch.from_numpy(g.offsets).to(dev)
    ws = [torch.from_numpy(g.w).to(dev) for _ in range(n_sets)]
    wss = [moe.pack_mx_weight_scales(torch.from_numpy(g.w_sc).to(dev)) for _ in range(n_sets)]
    ys = [torch.empty((g.rows, g.N), dtype=torch.bfloat16, device=dev) for _ in range(n_sets)]
    argv = [(a.data_ptr(), asc.data_ptr(), off.data_ptr(), g.E, g.rows, ws[k].data_ptr(),
             wss[k].data_ptr(), g.N, g.Kd, mx_mode, ys[k].data_ptr(), None,
             stream.cuda_stream) for k in range(n_sets)]
    f = lib.moe_expert_gemm

    def launches(n):
        rc = 0
        for k in range(n):
            rc |= f(*argv[k % n_sets])
        if rc:
            raise RuntimeError("moe_expert_gemm returned a non-zero status")

    launches(args.warmup)
    torch.cuda.synchronize()
    ok = True
    if not args.no_check:
        import oracle
        rows, cols, y64, abs64 = gemm_sample(g, np, oracle)
        got = ys[0].float().cpu().numpy()[rows][:, cols].astype(np.float64)
        tol = 2.0 ** -8 * np.abs(y64) + (7 * 2.0 ** -13 + g.Kd * 2.0 ** -26) * abs64
        ok = bool(np.all(np.abs(got - y64) <= tol))
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    launches(K)
    torch.cuda.synchronize()
    t_wall = (time.perf_counter() - t0) / K
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    launches(K)
    e1.record(stream)
    e1.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / K
    # the int8 formats at the same shape (per token, per tile of 128): kernel time only
    variants = {} if args.gemm_formats else None
    for name, mode, per_tile in ((("int8_per_token", moe.QUANT_INT8_TOKEN, False),
                                  ("int8_per_tile", moe.QUANT_INT8_TILE, True))
                                 if args.gemm_formats else ()):
        gi = W.make_gemm_case_i8(3200 + per_tile, g.counts, g.N, g.Kd, per_tile)
        ti = [torch.from_numpy(v).to(dev) for v in (gi.a, gi.a_sc, gi.offsets, gi.w, gi.w_sc)]
        wi2 = ti[3].clone()
        yi = torch.empty((gi.rows, gi.N), dtype=torch.bfloat16, device=dev)
        av = [(ti[0].data_ptr(), ti[1].data_ptr(), ti[2].data_ptr(), gi.E, gi.rows, wt.data_ptr(),
               ti[4].data_ptr(), gi.N, gi.Kd, mode, yi.data_ptr(), None, stream.cuda_stream)
              for wt in (ti[3], wi2)]
        for k in range(args.warmup):
            f(*av[k % 2])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(K):
            f(*av[k % 2])
        e1.record(stream)
        e1.synchronize()
        ui = e0.elapsed_time(e1) * 1e3 / K
        fi = 2.0 * int(gi.offsets[-1]) * gi.N * gi.Kd
        variants[name] = {"avg_us": round(ui, 3), "TOPS": round(fi / (ui * 1e-6) / 1e12, 2),
                          "frac_of_int8_peak": round(fi / (ui * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4)}
        del ti, wi2, yi
    ffn = None if args.gemm_dense else ffn_figures(args, g, argv, ys, off, n_sets, K, lib, moe, W,
                                                    torch, dev, stream)
    rows_total = int(g.offsets[-1])
    flops = 2.0 * rows_total * g.N * g.Kd
    tfs = flops / (us * 1e-6) / 1e12
    alg_bytes = g.a.nbytes + g.a_sc.nbytes + g.w.nbytes + g.w_sc.nbytes + rows_total * g.N * 2
    traffic = None if args.gemm_dense else counter_traffic("expert_gemm_g3_traffic.txt",
                                                          ("expert_gemm.hip", "device.h"))
    line = {
        "metric": GEMM_METRIC, "value": round(tfs, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(t_wall * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": ("one instance of 4096 rows (context, not the headline shape), "
                                "H=7168 -> N=4096, mxfp8 operands with E8M0 block scales, "
                                "bf16 out") if args.gemm_dense else
                               ("expert computation of one expert-parallel rank in a "
                                "DeepSeek-V3-shaped layer: 8 instances, 4096 rows split by a "
                                "Zipf(1.2) draw, H=7168 -> N=4096 (gate and up projections), "
                                "mxfp8 operands with E8M0 block scales, bf16 out"),
                   "E": g.E, "rows": rows_total, "counts": g.counts.tolist(), "N": g.N,
                   "H": g.Kd, "weight_sets": n_sets,
                   "activation_exponents": args.gemm_exponents},
        "roofline": {"kernel": "k_expert_gemm_mx", "bound": "mfma", "achieved": round(tfs, 2),
                     "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tfs / FP8_PEAK_TFLOPS, 4), "traffic": traffic,
                     "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": alg_bytes, "avg_launch_us": round(us, 3)},
        "hbm_GBps_algorithmic": round(alg_bytes / (us * 1e-6) / 1e9, 1),
        "other_formats": variants,
        "ffn": ffn,
        "parity_sample": "ok" if ok else "MISMATCH",
        "cpu_baseline": None,
    }
    if args.cpu_seconds > 0:
        import oracle
        line["cpu_baseline"] = gemm_cpu_baseline(g, np, oracle, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    if not ok:
        sys.exit(1)


def main():
    args = parse()
    if args.summarize_trace:
        return summarize_trace(args)
    if args.summarize_counters:
        return summarize_counters(args)
    if args.summarize_copy:
        return summarize_copy(args)
    if args.summarize_stalls:
        return summarize_stalls(args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py times the single-GPU share of the MoE layer and runs on one GPU only; "
              "--gpus above 1 is not supported.", file=sys.stderr)
        sys.exit(2)

    if args.copy_mb:
        copy_calibration(args.copy_mb, args.steps, args.warmup)
        return
    if args.only_config:
        import torch
        from combine_expert_amd import moe
        torch.cuda.init()
        print(json.dumps({"config_table": config_table(moe, torch, max(args.steps // 5, 50),
                                                       only=args.only_config)}), flush=True)
        return
    if args.gemm:
        return gemm_main(args)

    import numpy as np
    import torch

    from combine_expert_amd import build as hip_build
    if hip_build.stale():
        hip_build.build()
    from combine_expert_amd import moe
    from combine_expert_amd import workloads as W

    wl = W.make_c3()
    torch.cuda.init()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    lib = moe.raw()
    fns = (lib.moe_update_expert, lib.moe_dispatch, lib.moe_update_dispatch,
           lib.moe_combine_add_rmsnorm)
    UPD, DSP, FUSED, CMB = range(4)
    STEP, THREE = (FUSED, CMB), (UPD, DSP, CMB)

    n_sets = args.sets or cold_sets(min(38 << 20, 126 << 20))  # the dispatch's own traffic
    sets = [make_set(wl, torch, moe) for _ in range(n_sets)]
    argv = [step_args(wl, s, sp) for s in sets]
    torch.cuda.synchronize()

    def run_steps(n, calls):
        for k in range(n):
            a = argv[k % len(argv)]
            rc = 0
            for c in calls:
                rc |= fns[c](*a[c])
            if rc:
                raise RuntimeError("a library call returned a non-zero status")

    def timed_steps(n, calls):
        """Exactly n steps, synchronised on both sides."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_steps(n, calls)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n

    def kernel_us(which, n, n_sets=None):
        """Average launch duration of one kernel: HIP events on the launch stream
        bracket n back-to-back launches that rotate over the buffer sets (over the
        first n_sets of them when given: one set stays in the Infinity Cache)."""
        f = fns[which]
        n_sets = len(argv) if n_sets is None else n_sets
        for k in range(n_sets):
            f(*argv[k][which])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(n):
            f(*argv[k % n_sets][which])
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    run_steps(args.warmup, THREE)
    run_steps(args.warmup, STEP)
    torch.cuda.synchronize()
    ok = True
    if not args.no_check:
        import oracle
        ok = check_parity(wl, sets[0], oracle, np)

    # timed region: exactly K steps (mapping + dispatch in one launch, combine)
    K = args.steps
    t_step = timed_steps(K, STEP)
    t_three = timed_steps(K, THREE)  # the same step as the pages' three calls

    # per-kernel launch durations (the dominant kernel's feeds the roofline)
    n_k = max(K, 100)
    us = [kernel_us(j, n_k) for j in range(4)]
    rows = int(sets[0]["d"]["expert_offsets"][-1].item())
    nb = algorithmic_bytes(wl.Bs, wl.H, wl.K, wl.E, rows, wl.table.shape[0], wl.table.shape[1],
                           wl.quant_mode, moe.n_scale_entries(wl.quant_mode, wl.H, wl.tile),
                           shared=True)
    step_bytes = nb["update_dispatch"] + nb["combine"]
    gbs = step_bytes / t_step / 1e9
    three_bytes = nb["update_expert"] + nb["dispatch"] + nb["combine"]
    gbs_3 = three_bytes / t_three / 1e9
    names = ("update_expert", "dispatch", "update_dispatch", "combine")
    rate = {n: nb[n] / (u * 1e-6) / 1e9 for n, u in zip(names, us)}
    us_cmb = us[CMB]
    a_cmb = rate["combine"]

    # launches of each kernel so far: the headline part of a kernel trace of this
    # command is the first this many dispatches of each kernel
    W_, S_ = args.warmup, len(argv)
    launches = {"k_update_expert": W_ + K + S_ + n_k, "k_dispatch": W_ + K + S_ + n_k,
                "k_update_dispatch": W_ + K + S_ + n_k, "k_combine": 2 * W_ + 2 * K + S_ + n_k}

    # hot-cache figures (opt-in): the same launches on one buffer set, which the 256 MB
    # Infinity Cache then serves in part
    hot = None
    if args.hot:
        hot = {"note": "one buffer set reused back to back: inputs partly served from the "
                       "Infinity Cache; not the headline figure",
               **{f"{n}_us": round(kernel_us(j, n_k, 1), 3) for j, n in enumerate(names)}}
    extras = not args.headline_only
    graph = step_graph(torch, fns, argv, STEP, K, t_step, step_bytes, wl.Bs) if extras else None
    configs = config_table(moe, torch, max(K // 5, 50)) if extras else None
    c5 = time_stack(moe, torch, 16, max(10, K // 10), 3) if extras else None
    ceil = ceilings(torch, max(K // 5, 50), wl, sets[0], nb, rows) if extras else None
    variants = dispatch_variants(moe, torch, max(K // 5, 50)) if args.variants else None

    # HBM bytes per launch from the committed counter summaries (null when the
    # kernel source changed since they were taken)
    traffic = {"update_dispatch": counter_traffic("update_dispatch_c3_traffic.txt", DISPATCH_SRC),
               "dispatch": counter_traffic("dispatch_c3_traffic.txt", DISPATCH_SRC),
               "combine": counter_traffic("combine_c3_traffic.txt", COMBINE_SRC)}
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "DeepSeek-V3-shaped MoE layer: Bs=512, H=7168, 256 instances "
                               "(32 ranks x 8), K=8, Zipf(1.2) routing, mxfp8 dispatch, "
                               "1 shared expert, combine + residual + RMSNorm (bf16 in/out)",
                   "Bs": wl.Bs, "H": wl.H, "K": wl.K, "E": wl.E, "quant": "mxfp8",
                   "arithmetic": "bf16 rows in and out, mxfp8 (E4M3 + E8M0) codes, fp32 sums",
                   "rows_dispatched": rows, "buffer_sets": n_sets},
        "tokens_per_s": round(wl.Bs / t_step, 1),
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {
            "kernel": "k_combine", "bound": "hbm", "achieved": round(a_cmb, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(a_cmb / HBM_PEAK_GBS, 4),
            "traffic": traffic["combine"],
            "algorithmic_bytes_per_launch": nb["combine"],
            "avg_launch_us": round(us_cmb, 3),
        },
        "kernels": {
            n: {"avg_us": round(u, 3), "bytes": nb[n], "GBps": round(rate[n], 1),
                "frac": round(rate[n] / HBM_PEAK_GBS, 4), "traffic": traffic.get(n)}
            for n, u in zip(names, us)},
        "step_three_calls": {"ms_per_step": round(t_three * 1e3, 5), "GBps": round(gbs_3, 2),
                             "tokens_per_s": round(wl.Bs / t_three, 1), "bytes": three_bytes},
        "step_graph": graph,
        "hot_cache": hot,
        "c5_stack": c5,
        "dispatch_variants": variants,
        "other_configs": configs,
        "ceilings": ceil,
        "headline_launches": launches,
        "step_bytes": step_bytes,
        "parity_step0": "ok" if ok else "MISMATCH",
        "cpu_baseline": None,
    }
    if args.cpu_seconds > 0:
        import oracle
        line["cpu_baseline"] = cpu_baseline(wl, oracle, np, args.cpu_seconds, step_bytes)
    print(json.dumps(line), flush=True)
    if not ok:
        sys.exit(1)


if __name__ == "__main__":
    main()
