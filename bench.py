#!/usr/bin/env python3
"""Throughput of one D2F denoising step on one MI355X.

A step is the whole hot path over one synthetic batch, through the C ABI:
block-causal window attention for every layer of the workload
(d2f_block_attn), the confidence/commit pass over the window's vocabulary
logits (d2f_confidence_commit), and the append of a completed block to every
layer's KV cache (d2f_kv_commit).  Inputs are resident in HBM before timing.
Input sets rotate so that the timed steps read HBM rather than the 256 MB
Infinity Cache, and every step gets its own pristine mask state.

    python bench.py [--steps K] [--warmup W] [--config llada_batch16]

The default workload is the batched ragged decode at LLaDA-8B shape (16
requests, prefixes ~ U(256, 4096), 1-4 window blocks of 16, 32 layers x 32
heads x 128, vocabulary 126464); --config selects the single step, the
Dream-shaped GQA sweep or the long prefixes.

prints one JSON line.  `value` is the step's compulsory HBM bytes (K/V once
per KV head, Q, O, LSE, the masked rows' logits, the KV append) divided by
the measured step time.  Per call it also reports the back-to-back average
(`avg_us`, a HIP graph of repeated launches) and the spread of single
launches (`p10_us`, `median_us`, `p90_us`); `roofline` for the call with the
largest share of the step (with counter-measured HBM traffic when the
summary under profiles/ was taken on these kernel sources); `near_ties`, the
commit decisions too close to call; and `cpu_baseline`, the fp64 oracle on
a bounded sample of the same workload on the host cores.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "D2F step block-attn TFLOP/s + KV/logit GB/s (frac of peak), LLaDA-8B shape"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3     # MI355X fp32 vector
ROTATE_BYTES = 640 << 20     # > 2x the 256 MB Infinity Cache
SET_BUDGET_BYTES = 64 << 30  # device memory for the rotating input sets of the per-call timings


def input_set_count(read_per_step, smallest_call, set_bytes):
    """Rotating input sets: enough that the bytes streamed between two reads
    of the same set exceed ROTATE_BYTES for the whole step; and, within
    SET_BUDGET_BYTES of sets, also for the smallest single call (the per-call
    timings repeat one call through every set)."""
    n = 1 + math.ceil(ROTATE_BYTES / read_per_step)
    per_call = 1 + math.ceil(ROTATE_BYTES / smallest_call)
    return max(n, min(per_call, SET_BUDGET_BYTES // set_bytes))


def attn_flops(sh):
    """Visible (query, key) pairs x 4 * head_dim (QK^T and PV)."""
    tot = 0.0
    for b in range(sh.batch):
        for k in range(sh.n_win_blocks[b]):
            tot += sh.block_size * (sh.prefix_len[b] + (k + 1) * sh.block_size)
    return tot * sh.n_heads_q * 4.0 * sh.head_dim


def attn_bytes(sh):
    """K and V once per KV head over P + W keys, Q in, O and LSE out."""
    s = 4 if sh.dtype == "f32" else 2
    tot = 0.0
    for b in range(sh.batch):
        w = sh.win_rows(b)
        if w == 0:
            continue  # idle request: nothing is read
        tot += sh.n_heads_kv * (sh.prefix_len[b] + w) * sh.head_dim * 2 * s
        tot += 2 * sh.n_heads_q * w * sh.head_dim * s + sh.n_heads_q * w * 4
    return tot


def attn_kv_bytes(sh):
    s = 4 if sh.dtype == "f32" else 2
    return float(sum(sh.n_heads_kv * (sh.prefix_len[b] + sh.win_rows(b)) * sh.head_dim * 2 * s
                     for b in range(sh.batch) if sh.win_rows(b) > 0))


def commit_bytes(n_masked, rows, vocab):
    """Masked rows' logits once, plus per-row state (mask r/w, token, conf, argmax)."""
    return float(n_masked) * vocab * 4 + rows * (1 + 1 + 4 + 4 + 4)


def kv_commit_bytes(sh, layers):
    s = 4 if sh.dtype == "f32" else 2
    return 2.0 * 2 * sh.block_size * sh.n_heads_kv * sh.head_dim * s * layers  # K+V, read+write


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=None,
                    choices=["llada_p512", "llada_batch16", "dream_gqa", "llada_p32k", "llada_p128k"],
                    help="workload (default llada_batch16; only a run without --config adds "
                         "the per-call figures of the other workloads)")
    ap.add_argument("--block-size", type=int, default=None, help="dream_gqa block size (16/32/64)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of a HIP graph")
    ap.add_argument("--call-reps", type=int, default=20, help="launches per per-call timing graph")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle CPU-baseline budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the per-call figures of the other workloads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy (counter calibration) and exit")
    ap.add_argument("--measure", default="maxprob",
                    choices=["maxprob", "margin", "neg_entropy", "logit_gap"],
                    help="confidence measure of the commit pass")
    ap.add_argument("--early-gap", type=float, default=None,
                    help="Prophet's early-commit threshold (one group per call)")
    ap.add_argument("--paged", action="store_true",
                    help="keep K/V in a paged cache (one page per block; prefixes rounded down "
                         "to whole blocks)")
    ap.add_argument("--round-prefix", action="store_true",
                    help="round prefixes down to whole blocks (the paged layout's workload, "
                         "for a contiguous comparison)")
    ap.add_argument("--reuse", action="store_true",
                    help="also time outside-block reuse: the window-only attention plus the "
                         "log-space join, against the full call and the refresh of the outside "
                         "part")
    ap.add_argument("--decode-loop", action="store_true",
                    help="time complete multi-step decodes (pipelined active window) instead")
    ap.add_argument("--loop-blocks", type=int, default=8, help="blocks decoded per request")
    ap.add_argument("--loop-window", type=int, default=4, help="most blocks in the window")
    ap.add_argument("--loop-reps", type=int, default=3, help="timed complete decodes")
    ap.add_argument("--tau-add", type=float, default=0.25)
    ap.add_argument("--tau-act", type=float, default=0.75)
    ap.add_argument("--summarize-mfma", metavar="DIR",
                    help="turn a rocprofv3 --pmc output dir with the MFMA counters of a bench "
                         "run of --config into profiles/mfma_<config>.txt; needs no GPU")
    ap.add_argument("--summarize-stall", nargs=3, metavar=("DIR_A", "DIR_B", "DIR_C"),
                    help="turn three rocprofv3 --pmc output dirs (the STALL_COUNTERS passes of "
                         "a bench run of --config) into profiles/stall_<config>.txt; needs no "
                         "GPU")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write profiles/kernel_trace_<config>.md from a rocprofv3 --kernel-trace "
                         "--stats output directory")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("COPY_FETCH", "COPY_WRITE",
                                                              "RUN_FETCH", "RUN_WRITE"),
                    help="turn four rocprofv3 --pmc output dirs (FETCH_SIZE / WRITE_SIZE of "
                         "the copy calibration and of a bench run of --config) into "
                         "profiles/traffic_<config>.txt; needs no GPU")
    args = ap.parse_args()
    # The default line (no --config) also times the other workloads per call;
    # a run that names its workload, as the profiling commands do, does not.
    args.other_workloads = args.config is None and not args.no_other_workloads
    if args.config is None:
        args.config = "llada_batch16"
    return args


COPY_BYTES = 512 << 20


def copy_calibration(reps=5):
    """A plain device-to-device copy of known size, the reference for scaling
    the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ms, _ = time_region(lambda: [dst.copy_(src) for _ in range(reps)])
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES,
                      "reps": reps, "gbs": round(2 * COPY_BYTES * reps / (ms * 1e-3) / 1e9, 1)}),
          flush=True)


CALL_OF_KERNEL = (("attn_bf16_kernel", "d2f_block_attn"), ("attn_gqa_kernel", "d2f_block_attn"),
                  ("attn_f32_kernel", "d2f_block_attn"),
                  ("attn_merge_kernel", "d2f_block_attn"),
                  ("vocab_reduce_kernel", "d2f_confidence_commit"),
                  ("commit_decide_kernel", "d2f_confidence_commit"),
                  ("kv_commit_kernel", "d2f_kv_commit"))


def kernel_short_name(name):
    """Readable name of one of the library's kernels as rocprofv3 reports it:
    demangled ("void d2f::(anonymous namespace)::k<128, 2>(d2f::AttnArgs)"),
    or left mangled when it could not demangle a template argument (it leaves
    __bf16, mangled DF16b, alone).  None for other kernels."""
    import re
    if "d2f::" in name:
        short = name.replace("(anonymous namespace)::", "").split("(")[0]
        return short.replace("void ", "").replace("d2f::", "")
    m = re.match(r"_ZN3d2f(?:\d+_GLOBAL__N_1)?(\d+)", name)
    if not m:
        return None
    n = int(m.group(1))
    ident = name[m.end():m.end() + n]
    rest = name[m.end() + n:]
    args = []
    if rest.startswith("I"):
        tok = re.compile(r"Li(-?\d+)E|Lb([01])E|DF16b|f|d")
        i = 1
        while i < len(rest) and rest[i] != "E":
            t = tok.match(rest, i)
            if not t:
                break
            g = t.group(0)
            args.append(t.group(1) if t.group(1) is not None else
                        ("true" if t.group(2) == "1" else "false") if t.group(2) is not None else
                        {"DF16b": "__bf16", "f": "float", "d": "double"}[g])
            i = t.end()
    return ident + (f"<{', '.join(args)}>" if args else "")


def _counter_files(d):
    """The counter csv of a rocprofv3 --pmc output directory.  One run per
    directory: when it holds several (a later run written into the same
    place), only the newest is read."""
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    return sorted(files, key=os.path.getmtime)[-1:]


def _counter_means(d, counter):
    """Average per-dispatch value of `counter` for each kernel in a rocprofv3
    --pmc csv output directory."""
    import csv
    import glob
    sums, counts = {}, {}
    for f in _counter_files(d):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            k = r["Kernel_Name"]
            sums[k] = sums.get(k, 0.0) + float(r["Counter_Value"])
            counts[k] = counts.get(k, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS",
                 "SQ_INSTS_VALU_TRANS_F32", "SQ_VALU_MFMA_BUSY_CYCLES")


def _dispatch_ns(d, counter, name_part):
    """Average duration (ns) of the dispatches of kernels whose name holds
    name_part, from the timestamps of a --pmc csv."""
    import csv
    import glob
    tot, n = 0.0, 0
    for f in _counter_files(d):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                tot += float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
                n += 1
    return tot / n if n else None


def summarize_mfma(args):
    """Instruction mix and MFMA work of the attention kernels from counters."""
    import workloads as W
    d = args.summarize_mfma
    vals = {c: _counter_means(d, c) for c in MFMA_COUNTERS}
    cfg = W.config(args.config, block_size=args.block_size)
    flops_alg = attn_flops(cfg["shape"])
    kernels = {}
    for name, mops in vals["SQ_INSTS_VALU_MFMA_MOPS_BF16"].items():
        if "attn_bf16_kernel" not in name and "attn_gqa_kernel" not in name:
            continue
        short = kernel_short_name(name) or name[:60]
        ns = _dispatch_ns(d, MFMA_COUNTERS[0], short.split("<")[0])
        flops = mops * 512.0
        mfma = vals["SQ_INSTS_MFMA"].get(name, 0.0)
        valu = vals["SQ_INSTS_VALU"].get(name, 0.0)
        lds = vals["SQ_INSTS_LDS"].get(name, 0.0)
        trans = vals["SQ_INSTS_VALU_TRANS_F32"].get(name, 0.0)
        busy = vals["SQ_VALU_MFMA_BUSY_CYCLES"].get(name, 0.0)
        kernels[short] = {
            "mfma_mops_bf16": round(mops), "mfma_flops": flops,
            "algorithmic_flops": flops_alg,
            "mfma_over_algorithmic": round(flops / flops_alg, 3),
            "sq_insts_mfma": round(mfma), "sq_insts_valu": round(valu),
            "sq_insts_lds": round(lds), "sq_insts_valu_trans_f32": round(trans),
            "valu_non_mfma_per_mfma": round((valu - mfma) / mfma, 3) if mfma else None,
            "lds_per_mfma": round(lds / mfma, 3) if mfma else None,
            "trans_per_mfma": round(trans / mfma, 3) if mfma else None,
            "sq_valu_mfma_busy_cycles": round(busy),
            "mfma_busy_cycles_per_mfma": round(busy / mfma, 2) if mfma else None,
            "avg_dispatch_us_under_counters": round(ns / 1e3, 3) if ns else None,
            "mfma_tflops_under_counters": round(flops / ns / 1e3, 1) if ns else None,
            "frac_of_bf16_peak_under_counters":
                round(flops / ns / 1e3 / PEAK_BF16_TFLOPS, 4) if ns else None}
    key = traffic_key(args)
    bs = "" if args.block_size is None else f" --block-size {args.block_size}"
    hdr = (f"MFMA work and instruction mix of the bf16 attention kernels, workload {key}.\n"
           "Per-dispatch averages (counters summed over the device).  mfma_flops =\n"
           "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; its rate over the dispatch time is the MFMA\n"
           "utilisation against the 2500 TFLOP/s bf16 peak.  algorithmic_flops counts visible\n"
           "(query, key) pairs only (4 x head_dim each), so mfma_over_algorithmic > 1 is padded\n"
           "rows and masked keys of partial tiles.  SQ_INSTS_VALU includes the MFMA\n"
           "instructions; the per-MFMA ratios give the vector, LDS and transcendental (exp)\n"
           "instructions issued per v_mfma_f32_16x16x32_bf16.  SQ_VALU_MFMA_BUSY_CYCLES per\n"
           "MFMA is the matrix core's occupancy per instruction (16 cycles at full rate).\n"
           "Command (repo root on the MI355X machine, after `cd /tmp && export TMPDIR=/tmp`):\n"
           f"  rocprofv3 --pmc {' '.join(MFMA_COUNTERS)} --output-format csv -d <dir> -- "
           f"python3 bench.py --config {args.config}{bs} --steps 2 --warmup 1 --call-reps 2 "
           "--no-cpu-baseline\n"
           f"  python3 bench.py --config {args.config}{bs} --summarize-mfma <dir>\n")
    path = os.path.join(ROOT, "profiles", f"mfma_{key}.txt")
    with open(path, "w") as f:
        f.write(hdr + "\n---\n" + json.dumps({"config": key, "source_hash": kernel_source_hash(),
                                                "kernels": kernels}, indent=1) + "\n")
    print(path)


# Three counter passes (at most 8 SQ counters each) on where the waves of the
# attention kernels spend their cycles.
STALL_COUNTERS = (
    ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
     "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_VALU_MFMA_COEXEC_CYCLES"),
    ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAIT_INST_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_DATA_FIFO_FULL",
     "SQ_LDS_CMD_FIFO_FULL", "SQ_IFETCH", "SQ_ACTIVE_INST_MISC", "SQ_ACTIVE_INST_SCA"),
    ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_SMEM", "SQ_WAVES",
     "SQ_INST_LEVEL_LDS", "SQ_ACTIVE_INST_FLAT"))
N_SIMDS = 1024  # 256 CUs x 4


def stall_breakdown(v):
    """Derived figures from the per-dispatch means v (counter -> value) of the
    STALL_COUNTERS of one kernel.  The wave-cycle counters share one unit
    (quad-cycles), so their ratios are plain shares of the waves' lifetime."""
    wave = v["SQ_WAVE_CYCLES"]
    waves = v["SQ_WAVES"]
    busy = v["SQ_VALU_MFMA_BUSY_CYCLES"]
    share = {k: round(v[c] / wave, 4) for k, c in (
        ("issuing_any", "SQ_ACTIVE_INST_ANY"), ("waiting_on_counters_or_barrier", "SQ_WAIT_ANY"),
        ("waiting_to_issue", "SQ_WAIT_INST_ANY"), ("valu", "SQ_ACTIVE_INST_VALU"),
        ("lds", "SQ_ACTIVE_INST_LDS"), ("scalar", "SQ_ACTIVE_INST_SCA"),
        ("branch", "SQ_ACTIVE_INST_MISC"), ("waiting_for_lds_issue", "SQ_WAIT_INST_LDS"))}
    per_wave = {k: round(v[c] / waves, 1) for k, c in (
        ("valu_incl_mfma", "SQ_INSTS_VALU"), ("mfma", "SQ_INSTS_MFMA"), ("lds", "SQ_INSTS_LDS"),
        ("salu", "SQ_INSTS_SALU"), ("smem", "SQ_INSTS_SMEM"))}
    return {"share_of_wave_cycles": share,
            "instructions_per_wave": per_wave,
            "mfma_busy_cycles_per_simd": round(busy / N_SIMDS),
            "coexec_share_of_mfma_busy": round(v["SQ_VALU_MFMA_COEXEC_CYCLES"] / busy, 4)
            if busy else None,
            "lds_bank_conflict_cycles": round(v["SQ_LDS_BANK_CONFLICT"]),
            "lds_cmd_fifo_full_cycles": round(v["SQ_LDS_CMD_FIFO_FULL"]),
            "lds_data_fifo_full_cycles": round(v["SQ_LDS_DATA_FIFO_FULL"])}


def summarize_stall(args):
    """Where the attention kernels' waves spend their cycles, from three
    counter passes of one bench run each."""
    vals, ns = {}, {}
    for d, cs in zip(args.summarize_stall, STALL_COUNTERS):
        for c in cs:
            for name, x in _counter_means(d, c).items():
                if "attn_bf16_kernel" not in name and "attn_gqa_kernel" not in name:
                    continue
                short = kernel_short_name(name) or name[:60]
                vals.setdefault(short, {})[c] = x
                if short not in ns:
                    ns[short] = _dispatch_ns(d, c, short.split("<")[0])
    kernels = {}
    for short, v in vals.items():
        if any(c not in v for cs in STALL_COUNTERS for c in cs):
            continue
        rec = stall_breakdown(v)
        rec["avg_dispatch_us_under_counters"] = round(ns[short] / 1e3, 3) if ns[short] else None
        rec["raw_means"] = {c: round(v[c], 1) for cs in STALL_COUNTERS for c in cs}
        kernels[short] = rec
    key = traffic_key(args)
    bs = "" if args.block_size is None else f" --block-size {args.block_size}"
    run = (f"python3 bench.py --config {args.config}{bs} --steps 1 --warmup 1 --call-reps 1 "
           "--no-cpu-baseline")
    cmds = "".join(f"  rocprofv3 --pmc {' '.join(cs)} --output-format csv -d <dir{i}> -- {run}\n"
                   for i, cs in enumerate(STALL_COUNTERS, 1))
    hdr = (f"Where the waves of the attention kernels spend their cycles, workload {key}.\n"
           "Per-dispatch averages of SQ counters summed over the device, from three passes.\n"
           "share_of_wave_cycles divides SQ_ACTIVE_INST_* (cycles issuing each kind of\n"
           "instruction), SQ_WAIT_ANY (waiting on a wait counter or a barrier), SQ_WAIT_INST_ANY\n"
           "(an instruction ready but not issued) and SQ_WAIT_INST_LDS by SQ_WAVE_CYCLES (all in\n"
           "quad-cycles).  coexec_share_of_mfma_busy = SQ_VALU_MFMA_COEXEC_CYCLES /\n"
           "SQ_VALU_MFMA_BUSY_CYCLES: the part of the matrix core's busy cycles in which a\n"
           "vector instruction was issued alongside.  instructions_per_wave divides the\n"
           "SQ_INSTS_* counts by SQ_WAVES.\n"
           "Commands (repo root on the MI355X machine, after `cd /tmp && export TMPDIR=/tmp`):\n"
           f"{cmds}"
           f"  python3 bench.py --config {args.config}{bs} --summarize-stall <dir1> <dir2> <dir3>\n")
    path = os.path.join(ROOT, "profiles", f"stall_{key}.txt")
    with open(path, "w") as f:
        f.write(hdr + "\n---\n" + json.dumps({"config": key, "source_hash": kernel_source_hash(),
                                                "kernels": kernels}, indent=1) + "\n")
    print(path)


def summarize_trace(args):
    """Per-kernel durations of the library's kernels from a rocprofv3
    --kernel-trace --stats run of this benchmark."""
    import csv
    import glob
    files = glob.glob(os.path.join(args.summarize_trace, "**", "*kernel_stats.csv"), recursive=True)
    rows = []
    for f in files:
        for r in csv.DictReader(open(f)):
            short = kernel_short_name(r["Name"])
            if short is None:
                continue
            rows.append((short, int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
                         float(r["MaxNs"])))
    rows.sort(key=lambda x: -x[1] * x[2])
    if args.decode_loop:
        key = "decode_loop_llada_batched"
        run = "--decode-loop --loop-reps 1"
        what = ["Per-kernel durations of the library's kernels over the pipelined decoding",
                "loop (bench.py --decode-loop: one warm-up, one timed and one phase-timed decode",
                "of the batched ragged LLaDA-8B-shaped workload; rocprofv3 kernel trace)."]
    else:
        key = traffic_key(args)
        bs = "" if args.block_size is None else f" --block-size {args.block_size}"
        extra = "".join(f" --{k.replace('_', '-')}" for k in ("paged", "round_prefix")
                        if getattr(args, k, False))
        run = f"--config {args.config}{bs}{extra} --steps 5 --warmup 2 --no-cpu-baseline"
        what = ["Per-kernel durations of the library's kernels (rocprofv3 kernel trace; each",
                "call of the benchmark's timed graphs, its per-call graphs and the eager spread",
                "launches counted)."]
    lines = [f"# Kernel trace: {key}", "", *what, "",
             "Command (repo root on the MI355X machine, after `cd /tmp && export TMPDIR=/tmp`):", "",
             "    rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o kt -- \\",
             f"        python3 bench.py {run}",
             f"    python3 bench.py {run.split(' --steps')[0]} --summarize-trace <dir>", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
    for short, calls, avg, mn, mx in rows:
        lines.append(f"| {short} | {calls} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} |")
    lines += ["", f"source_hash: {kernel_source_hash()}", ""]
    path = os.path.join(ROOT, "profiles", f"kernel_trace_{key}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    print(path)


def summarize_counters(args):
    cf = _counter_means(args.summarize_counters[0], "FETCH_SIZE")
    cw = _counter_means(args.summarize_counters[1], "WRITE_SIZE")
    rf = _counter_means(args.summarize_counters[2], "FETCH_SIZE")
    rw = _counter_means(args.summarize_counters[3], "WRITE_SIZE")
    copy_kernel = max(cf, key=cf.get)  # the 512 MiB copy dominates the calibration run
    f_fetch = (COPY_BYTES / 1024) / cf[copy_kernel]
    f_write = (COPY_BYTES / 1024) / cw[copy_kernel]
    calls = {}
    for name in rf:
        call = next((c for k, c in CALL_OF_KERNEL if k in name), None)
        if call is None:
            continue
        e = calls.setdefault(call, {"kernels": {}, "bytes_per_call": 0.0})
        fb = rf[name] * 1024 * f_fetch
        wb = rw.get(name, 0.0) * 1024 * f_write
        short = kernel_short_name(name) or name[:60]
        e["kernels"][short] = {"fetch_kib": round(rf[name], 1),
                                                  "write_kib": round(rw.get(name, 0.0), 1),
                                                  "bytes": round(fb + wb)}
        e["bytes_per_call"] += fb + wb
    key = traffic_key(args)
    rec = {"config": key, "source_hash": kernel_source_hash(),
           "calibration": {"kernel": copy_kernel[:60], "copy_bytes": COPY_BYTES,
                           "fetch_kib": round(cf[copy_kernel], 1),
                           "write_kib": round(cw[copy_kernel], 1),
                           "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4)},
           "calls": calls}
    path = os.path.join(ROOT, "profiles", f"traffic_{key}.txt")
    bs = "" if args.block_size is None else f" --block-size {args.block_size}"
    hdr = (f"HBM traffic per call for workload {key} from rocprofv3 counters.\n"
           "FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are averaged per kernel and scaled by\n"
           "what the same counters read for a plain 512 MiB device copy (calibration).\n"
           "Commands (repo root on the MI355X machine, after `cd /tmp && export TMPDIR=/tmp`, each\n"
           "counter in its own run):\n"
           "  rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -- python3 bench.py --copy-calibration\n"
           "  rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -- python3 bench.py --copy-calibration\n"
           f"  rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -- python3 bench.py --config {args.config}{bs} --steps 2 --warmup 1 --call-reps 2 --no-cpu-baseline\n"
           f"  rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -- python3 bench.py --config {args.config}{bs} --steps 2 --warmup 1 --call-reps 2 --no-cpu-baseline\n"
           f"  python3 bench.py --config {args.config}{bs} --summarize-counters <4 dirs>\n"
           "bench.py reports bytes_per_call as roofline.traffic only while source_hash (the kernel\n"
           "sources without comments or whitespace) matches.\n")
    with open(path, "w") as f:
        f.write(hdr + "\n---\n" + json.dumps(rec, indent=1) + "\n")
    print(path)


# Sources the three per-step calls are built from (planner, kernels, shared
# declarations); the multi-step bookkeeping (window.hip, decode.hip) is not
# among them.
STEP_SOURCES = ("api.hip", "attn_bf16.hip", "attn_gqa.hip", "attn_lds.h", "attn_f32.hip",
                "attn_merge.h", "attn_merge.hip", "commit.hip", "kv_commit.hip", "d2f_internal.h")


def kernel_source_hash():
    """Hash of the HIP sources of the per-step calls, comments and whitespace
    left out: counter-derived traffic is only reported for the code it was
    measured on."""
    import hashlib
    import re
    h = hashlib.sha256()
    d = os.path.join(ROOT, "block_causal_attention_d2f_amd", "csrc")
    for f in STEP_SOURCES:
        text = open(os.path.join(d, f), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(f.encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_key(args):
    """Name of a workload's counter summary: the config, plus the block size
    when one is chosen explicitly (the GQA config is measured per B) and the
    confidence measure when it is not the maximum probability."""
    key = args.config if args.block_size is None else f"{args.config}_b{args.block_size}"
    if getattr(args, "measure", "maxprob") != "maxprob":
        key += f"_{args.measure}"
    if getattr(args, "paged", False):
        key += "_paged"
    elif getattr(args, "round_prefix", False):
        key += "_whole_blocks"
    return key


def measured_traffic(config_name, call):
    """HBM bytes per launch of `call` from the committed counter summary
    (profiles/traffic_<config>.txt), or None when absent or measured on other
    kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{config_name}.txt")
    try:
        rec = json.loads(open(path).read().split("\n---\n")[-1])
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    c = rec.get("calls", {}).get(call)
    return None if c is None else c.get("bytes_per_call")


class Workload:
    """Rotating input sets of one configuration, resident on the GPU."""

    def __init__(self, name, block_size, n_masks, measure="maxprob", early_gap=None,
                 paged=False, round_prefix=False):
        import torch
        import workloads as W
        self.measure, self.early_gap, self.paged = measure, early_gap, paged
        self.cfg = W.config(name, block_size=block_size)
        sh = self.cfg["shape"]
        if paged or round_prefix:
            B = sh.block_size
            sh = W.make_shape(sh.batch, sh.n_heads_q, sh.n_heads_kv, sh.head_dim, B,
                              [p // B * B for p in sh.prefix_len], sh.n_win_blocks,
                              dtype=sh.dtype, max_win_blocks=sh.max_win_blocks,
                              cache_capacity=sh.cache_capacity)
            self.cfg["shape"] = sh
        self.sh = sh
        self.layers = self.cfg["layers"]
        self.tau = self.cfg["taus"][0]
        self.k_aggr = self.cfg["k_aggr"]
        dev = "cuda"
        self.rows = W.total_rows(sh)
        es = 4 if sh.dtype == "f32" else 2
        read_per_step = (self.layers * attn_bytes(sh) + self.rows * self.cfg["vocab"] * 4)
        self.set_bytes = (self.layers * es * sh.head_dim *
                          (sh.batch * sh.n_heads_q * sh.w_max + 2 * sh.batch * sh.n_heads_kv *
                           (sh.cache_capacity + sh.w_max)) + self.rows * self.cfg["vocab"] * 4)
        # A workload whose sets exceed the budget keeps the per-step count;
        # its calls are then far larger than the cache anyway.
        smallest = min(read_per_step, attn_bytes(sh), self.rows * self.cfg["vocab"] * 4)
        self.n_sets = input_set_count(read_per_step, smallest, self.set_bytes)
        self.sets = []
        for r in range(self.n_sets):
            xs = [W.attn_inputs(sh, layer=l, device=dev, seed=r * 7919) for l in range(self.layers)]
            st = {n: torch.stack([x[n] for x in xs]) for n in xs[0]}
            ci = W.config_commit_inputs(self.cfg, device=dev, seed=r * 7919)
            st["logits"] = ci.logits
            if paged:
                self._to_pages(st)
            self.sets.append(st)
            del xs
        self.phases = ci.block_phase
        self.mask_token_id = ci.mask_token_id
        self.n_masked = int((ci.mask_state == W.MASKED).sum())
        self.mask0, self.tok0 = ci.mask_state.clone(), ci.tokens.clone()
        self.masks = ci.mask_state.unsqueeze(0).repeat(n_masks, 1).contiguous()
        self.tokens = ci.tokens.unsqueeze(0).repeat(n_masks, 1).contiguous()
        # Outputs and workspaces, allocated once.
        import block_causal_attention_d2f_amd as d2f
        q0 = self.sets[0]["q"][0]
        self.out = torch.empty((self.layers,) + tuple(q0.shape), dtype=q0.dtype, device=dev)
        self.lse = torch.empty((self.layers,) + tuple(q0.shape[:3]), dtype=torch.float32,
                               device=dev)
        desc = d2f.make_desc(sh.batch, sh.n_heads_q, sh.n_heads_kv, sh.head_dim, sh.block_size,
                             sh.max_win_blocks, sh.cache_capacity + sh.w_max, q0.dtype)
        need = d2f.d2f_block_attn_workspace_size(desc, sh.prefix_len, sh.n_win_blocks)
        self.ws_attn = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        need = d2f.d2f_confidence_commit_workspace_size(self.rows, self.cfg["vocab"])
        self.ws_commit = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        nb = self.rows // sh.block_size
        self.n_committed = torch.empty(nb, dtype=torch.int32, device=dev)
        self.block_complete = torch.empty(nb, dtype=torch.uint8, device=dev)
        self.conf = torch.empty(self.rows, dtype=torch.float32, device=dev)
        self.argmax = torch.empty(self.rows, dtype=torch.int32, device=dev)
        self.prefix_dev = torch.tensor(sh.prefix_len, dtype=torch.int32, device=dev)
        self.early_gap_dev = (None if early_gap is None else
                              torch.tensor([early_gap], dtype=torch.float32, device=dev))
        torch.cuda.synchronize()

    def _to_pages(self, st):
        """Move one input set's caches and windows into page pools (one pool
        per layer, page ids shared by the layers, randomly numbered)."""
        import torch
        sh, B = self.sh, self.sh.block_size
        L, nb, hkv, _, d = st["k_cache"].shape
        if not hasattr(self, "page_table"):
            n_cache = [p // B for p in sh.prefix_len]
            self.n_pages = sum(n_cache) + sum(sh.n_win_blocks)
            perm = torch.randperm(self.n_pages, generator=torch.Generator().manual_seed(1)).tolist()
            ts = max(n_cache) + 1
            pt = torch.full((nb, ts), -1, dtype=torch.int32)
            wp = torch.full((nb, sh.max_win_blocks), -1, dtype=torch.int32)
            for b in range(nb):
                for i in range(n_cache[b]):
                    pt[b, i] = perm.pop()
                for k in range(sh.n_win_blocks[b]):
                    wp[b, k] = perm.pop()
            self.page_table, self.win_pages = pt.cuda(), wp.cuda()
            self.pt_scratch, self.wp_scratch = self.page_table.clone(), self.win_pages.clone()
        pt, wp = self.page_table.cpu(), self.win_pages.cpu()
        for name, cname, wname in (("k_pages", "k_cache", "k_win"), ("v_pages", "v_cache", "v_win")):
            pool = torch.empty((L, self.n_pages, hkv, B, d), dtype=st[cname].dtype, device="cuda")
            for b in range(nb):
                for i in range(sh.prefix_len[b] // B):
                    pool[:, int(pt[b, i])] = st[cname][:, b, :, i * B:(i + 1) * B]
                for k in range(sh.n_win_blocks[b]):
                    pool[:, int(wp[b, k])] = st[wname][:, b, :, k * B:(k + 1) * B]
            st[name] = pool
            del st[cname], st[wname]

    # --- the three calls ---------------------------------------------------
    def ensure_masks(self, n):
        """At least n pristine mask/token rows (one per commit call)."""
        if self.masks.shape[0] < n:
            self.masks = self.mask0.unsqueeze(0).repeat(n, 1).contiguous()
            self.tokens = self.tok0.unsqueeze(0).repeat(n, 1).contiguous()

    def attn(self, r, l):
        import block_causal_attention_d2f_amd as d2f
        s, sh = self.sets[r], self.sh
        if self.paged:
            d2f.d2f_block_attn_paged(s["q"][l], s["k_pages"][l], s["v_pages"][l], self.page_table,
                                     self.win_pages, sh.prefix_len, sh.n_win_blocks,
                                     out=self.out[l], lse=self.lse[l], workspace=self.ws_attn)
            return
        d2f.d2f_block_attn(s["q"][l], s["k_cache"][l], s["v_cache"][l], s["k_win"][l],
                           s["v_win"][l], sh.prefix_len, sh.n_win_blocks, sh.block_size,
                           out=self.out[l], lse=self.lse[l], workspace=self.ws_attn)

    def commit(self, r, m):
        import block_causal_attention_d2f_amd as d2f
        d2f.d2f_confidence_commit(self.sets[r]["logits"], self.masks[m], self.tokens[m],
                                  self.phases, self.sh.block_size, self.tau, self.k_aggr,
                                  self.mask_token_id, conf_out=self.conf, argmax_out=self.argmax,
                                  n_committed=self.n_committed,
                                  block_complete=self.block_complete, workspace=self.ws_commit,
                                  measure=self.measure, early_gap=self.early_gap_dev)

    def kv(self, r):
        import block_causal_attention_d2f_amd as d2f
        s = self.sets[r]
        prefix = list(self.sh.prefix_len)  # the workload stays fixed from step to step
        if self.paged:
            # the persist moves page ids only: scratch tables keep the ones
            # attention reads intact from step to step
            d2f.d2f_kv_commit_paged(self.pt_scratch, self.wp_scratch, prefix, 0,
                                    self.sh.block_size, n_heads_kv=self.sh.n_heads_kv,
                                    head_dim=self.sh.head_dim, prefix_len_dev=self.prefix_dev)
            return
        d2f.d2f_kv_commit(s["k_cache"], s["v_cache"], s["k_win"], s["v_win"], prefix, 0,
                          self.sh.block_size, prefix_len_dev=self.prefix_dev)

    def step(self, i):
        r = i % self.n_sets
        for l in range(self.layers):
            self.attn(r, l)
        self.commit(r, i)
        self.kv(r)

    def kv_bytes(self):
        """The append's compulsory bytes: K/V rows copied, or, paged, the
        page ids moved."""
        if self.paged:
            return 4.0 * 2 * (self.sh.max_win_blocks + 1)
        return kv_commit_bytes(self.sh, self.layers)

    def step_bytes(self):
        return (self.layers * attn_bytes(self.sh) +
                commit_bytes(self.n_masked, self.rows, self.cfg["vocab"]) + self.kv_bytes())


def capture(fn, use_graph):
    """A callable that replays fn (captured into a HIP graph) or runs it."""
    import torch
    if not use_graph:
        return fn
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g.replay


def time_region(run):
    import torch
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1), (time.perf_counter() - t0) * 1e3


def per_call_times(wl, reps, use_graph):
    """Average duration of each call, from HIP events around a graph of
    `reps` back-to-back launches on the current stream (rotating inputs)."""
    n_sets = wl.n_sets
    base = wl.masks.shape[0] - reps  # spare pristine masks reserved for this

    def attn_run():
        for i in range(reps):
            wl.attn(i % n_sets, 0)

    def commit_run():
        for i in range(reps):
            wl.commit(i % n_sets, base + i)

    def kv_run():
        for i in range(reps):
            wl.kv(i % n_sets)

    out = {}
    for name, fn in (("d2f_block_attn", attn_run), ("d2f_confidence_commit", commit_run),
                     ("d2f_kv_commit", kv_run)):
        run = capture(fn, use_graph)
        if name == "d2f_confidence_commit":
            wl.masks[base:] = wl.mask0
            wl.tokens[base:] = wl.tok0
        run()  # warm
        if name == "d2f_confidence_commit":
            wl.masks[base:] = wl.mask0
            wl.tokens[base:] = wl.tok0
        ms, _ = time_region(run)
        out[name] = ms / reps
    return out


# Width of the band around a threshold inside which the fp32 confidence and
# the exact one may fall on different sides (the parity tests exclude these
# decisions from the bit-exact comparison and count them).
NEAR_BAND = {"maxprob": 1e-6, "margin": 1e-6, "neg_entropy": 5e-5, "logit_gap": 1e-5}


# Workloads timed after the default line, per call, so that one default run
# also covers the calls the other targets are set on: the Dream-7B-shaped
# grouped-query attention (MFMA-bound) and its commit pass at three block
# sizes, and the 32K-token prefix (KV-read-bound).
OTHER_WORKLOADS = (("dream_gqa", 16), ("dream_gqa", 32), ("dream_gqa", 64), ("llada_p32k", None))


def other_workloads(args, use_graph):
    """Per-call attention and commit figures of OTHER_WORKLOADS (HIP graphs of
    back-to-back launches over rotating input sets, as for the default line).
    A workload that fails records its error instead of ending the run."""
    import torch
    res = {}
    for name, bs in OTHER_WORKLOADS:
        key = name if bs is None else f"{name}_b{bs}"
        wl = None
        try:
            wl = Workload(name, bs, 1)
            reps = max(args.call_reps, wl.n_sets)
            wl.ensure_masks(reps + 1)
            calls = per_call_times(wl, reps, use_graph)
            sh = wl.sh
            t_a = calls["d2f_block_attn"] * 1e-3
            t_c = calls["d2f_confidence_commit"] * 1e-3
            a_flops, a_bytes = attn_flops(sh), attn_bytes(sh)
            c_bytes = commit_bytes(wl.n_masked, wl.rows, wl.cfg["vocab"])
            tflops, gbs, cgbs = a_flops / t_a / 1e12, a_bytes / t_a / 1e9, c_bytes / t_c / 1e9
            res[key] = {
                "workload": wl.cfg["workload"],
                "attn": {"avg_us": round(t_a * 1e6, 3), "tflops": round(tflops, 3),
                         "frac_mfma": round(tflops / PEAK_BF16_TFLOPS, 4), "gbs": round(gbs, 2),
                         "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "flops": a_flops,
                         "bytes": a_bytes},
                "commit": {"avg_us": round(t_c * 1e6, 3), "logit_gbs": round(cgbs, 2),
                           "frac_hbm": round(cgbs / PEAK_HBM_GBS, 4), "bytes": c_bytes},
                "per_call_graph_launches": reps, "input_sets": wl.n_sets}
        except Exception as e:  # a failure here must not cost the default line
            res[key] = {"error": f"{type(e).__name__}: {e}"[:300]}
        finally:
            del wl
            torch.cuda.empty_cache()
    return res


def near_ties(wl):
    """Commit decisions too close to call, from the GPU's own fp32 confidences
    of the last commit call: MASKED rows within the measure's band of the
    threshold (as the interface receives it, in float32), and aggressive
    blocks whose k_aggr-th and (k_aggr+1)-th masked confidences are that close
    while the latter does not clear the threshold."""
    import numpy as np
    import workloads as W
    band = NEAR_BAND[wl.measure]
    conf = wl.conf.cpu().double().numpy()
    live = wl.mask0.cpu().numpy() == W.MASKED
    tau = float(np.float32(wl.tau))
    near_tau = int((live & (np.abs(conf - tau) <= band)).sum())
    near_topk = 0
    B, k = wl.sh.block_size, wl.k_aggr
    if k > 0:
        for j in np.flatnonzero(wl.phases.cpu().numpy() == W.AGGRESSIVE):
            c = np.sort(conf[j * B:(j + 1) * B][live[j * B:(j + 1) * B]])[::-1]
            if len(c) > k and c[k] <= tau and c[k - 1] - c[k] <= band:
                near_topk += 1
    return {"near_tau": near_tau, "near_topk": near_topk, "band": band,
            "masked_rows": int(live.sum()), "source": "GPU fp32 confidences of the eager step"}


def per_call_spread(wl, reps):
    """Per-launch duration spread of each call, in us: (p10, median, p90).

    The host enqueues `reps` eager launches of the call, each between its own
    pair of HIP events, behind a bounded spin kernel, so the queue is full
    before the GPU reaches the first launch: the launches then run
    back-to-back and each event pair brackets one call's GPU time (with the
    event packets' own cost)."""
    import numpy as np
    import torch
    n_sets = wl.n_sets
    base = wl.masks.shape[0] - reps
    calls = (("d2f_block_attn", lambda i: wl.attn(i % n_sets, 0)),
             ("d2f_confidence_commit", lambda i: wl.commit(i % n_sets, base + i)),
             ("d2f_kv_commit", lambda i: wl.kv(i % n_sets)))
    out = {}
    for name, call in calls:
        wl.masks[base:] = wl.mask0
        wl.tokens[base:] = wl.tok0
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        torch.cuda.synchronize()
        torch.cuda._sleep(20_000_000)
        for i in range(reps):
            ev[i][0].record()
            call(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
        out[name] = tuple(round(float(x), 3) for x in np.percentile(us, [10, 50, 90]))
    return out


def reuse_times(wl, reps, use_graph):
    """Per-layer times of outside-block reuse: the full call, the outside part
    (cache keys only, the refresh), the window-only part and the join."""
    import torch
    import block_causal_attention_d2f_amd as d2f
    sh, n_sets = wl.sh, wl.n_sets
    zero = [0] * sh.batch
    lo = [0] * sh.batch
    o_out, l_out = torch.empty_like(wl.out[0]), torch.empty_like(wl.lse[0])
    o_win, l_win = torch.empty_like(wl.out[0]), torch.empty_like(wl.lse[0])
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")

    def full():
        for i in range(reps):
            wl.attn(i % n_sets, 0)

    def outside():
        for i in range(reps):
            s = wl.sets[i % n_sets]
            d2f.d2f_block_attn_range(s["q"][0], s["k_cache"][0], s["v_cache"][0], lo,
                                     sh.prefix_len, sh.n_win_blocks, sh.block_size, out=o_out,
                                     lse=l_out, workspace=ws)

    def window():
        for i in range(reps):
            s = wl.sets[i % n_sets]
            d2f.d2f_block_attn(s["q"][0], s["k_cache"][0], s["v_cache"][0], s["k_win"][0],
                               s["v_win"][0], zero, sh.n_win_blocks, sh.block_size, out=o_win,
                               lse=l_win, workspace=ws)

    def join():
        for i in range(reps):
            d2f.d2f_attn_combine(o_out, l_out, o_win, l_win, sh.n_win_blocks, sh.block_size,
                                 out=wl.out[0], lse=wl.lse[0])

    out = {}
    for name, fn in (("full", full), ("outside_refresh", outside), ("window_only", window),
                     ("join", join)):
        run = capture(fn, use_graph)
        run()
        ms, _ = time_region(run)
        out[name + "_us"] = round(ms / reps * 1e3, 3)
    out["reuse_step_us"] = round(out["window_only_us"] + out["join_us"], 3)
    out["speedup_when_reused"] = round(out["full_us"] / out["reuse_step_us"], 2)
    return out


def cpu_baseline(wl, budget_s):
    """The fp64 oracle on a bounded sample of the same workload, timed on the
    host cores.  The sample is one layer's attention for a subset of query
    heads plus the commit pass on a subset of blocks; its compulsory bytes
    are scaled the same way as the GPU step's."""
    import numpy as np
    import torch
    from oracle import attention as OA
    from oracle import commit as OC
    sh = wl.sh
    s = wl.sets[0]
    # Copy the sample to host memory first so that only the oracle is timed.
    heads = list(range(min(sh.n_heads_q, 8)))
    pairs = [(b, h) for b in range(sh.batch) for h in heads]
    host = {n: s[n][0].cpu() for n in ("q", "k_cache", "v_cache", "k_win", "v_win")}
    nb_blocks = min(wl.rows // sh.block_size, 4)
    rows = nb_blocks * sh.block_size
    logits = s["logits"][:rows].cpu()
    masks, toks = wl.mask0[:rows].cpu(), wl.tok0[:rows].cpu()
    phases = wl.phases[:nb_blocks].cpu()
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    # bytes the sample covers, counted like the GPU step
    frac_heads = len(heads) / sh.n_heads_q
    bytes_attn = attn_bytes(sh) * frac_heads
    bytes_commit = commit_bytes(int((masks == 0).sum()), rows, wl.cfg["vocab"])
    reps, t0 = 0, time.perf_counter()
    while True:
        OA.block_attn(host["q"], host["k_cache"], host["v_cache"], host["k_win"], host["v_win"],
                      sh.prefix_len, sh.n_win_blocks, sh.block_size, pairs=pairs)
        OC.confidence_commit(logits, masks, toks, phases, sh.block_size, wl.tau, wl.k_aggr,
                             wl.mask_token_id)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    gbs = reps * (bytes_attn + bytes_commit) / el / 1e9
    return dict(value=round(gbs, 4), unit="GB/s", cores=int(blas), kind="oracle",
                sample=(f"{reps} x (attention of layer 0 for query heads {heads[0]}..{heads[-1]} "
                        f"of every request + commit pass over {rows} rows x "
                        f"{wl.cfg['vocab']} logits), numpy fp64, {el:.1f} s; "
                        f"host affinity {len(os.sched_getaffinity(0))} cpus"))


LOOP_METRIC = "D2F pipelined decoding: hot-path decoded tokens/s, LLaDA-8B shape"


class DecodeLoop:
    """Complete multi-step decodes of the batched ragged LLaDA-8B-shaped
    workload (16 requests, prompts ~ U(256, 4096), 32 layers x 32 heads x
    128, B = 16, vocab 126464) with the active-window schedule: per step,
    attention of every layer over each request's window, the commit pass
    over every window slot, and d2f_decode_advance (the step's one
    device-to-host transfer).  Q, the window K/V and the logits are resident
    synthetic tensors (the model that would produce them is not part of the
    path); the logits rotate through a pool of independent N(0, 3) sets with
    one boosted column per row, so every row's confidence is redrawn each
    step."""

    def __init__(self, args):
        import torch
        import workloads as W
        import block_causal_attention_d2f_amd as d2f
        self.paged = args.paged
        self.cfg = cfg = W.config("llada_batch16")
        sh = cfg["shape"]
        self.nb, self.hq, self.hkv, self.d, self.B = (sh.batch, sh.n_heads_q, sh.n_heads_kv,
                                                      sh.head_dim, sh.block_size)
        self.L, self.vocab = cfg["layers"], cfg["vocab"]
        self.mw, self.total = args.loop_window, args.loop_blocks
        self.tau, self.k_aggr = cfg["taus"][0], cfg["k_aggr"]
        self.tau_add, self.tau_act = args.tau_add, args.tau_act
        self.prompt = list(sh.prefix_len)
        if self.paged:  # the paged cache holds whole blocks
            self.prompt = [p // self.B * self.B for p in self.prompt]
        self.cap = max(self.prompt) + self.total * self.B
        self.wmax = self.mw * self.B
        self.mask_id = self.vocab
        dev = "cuda"
        g = torch.Generator(device=dev).manual_seed(1234)
        bf = torch.bfloat16

        def randn(*shape):
            return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(bf)
        L, nb, hq, hkv, d = self.L, self.nb, self.hq, self.hkv, self.d
        if self.paged:
            # pages for the prompts, the first block of each window and one
            # per later block; ids in random order
            self.n_pages = sum(p // self.B for p in self.prompt) + nb * (self.total + 1)
            self.kc = torch.empty((L, self.n_pages, hkv, self.B, d), dtype=bf, device=dev)
            self.vc = torch.empty_like(self.kc)
            for l in range(L):
                self.kc[l] = randn(self.n_pages, hkv, self.B, d)
                self.vc[l] = randn(self.n_pages, hkv, self.B, d)
            self.page_order = torch.randperm(
                self.n_pages, generator=torch.Generator().manual_seed(5)).tolist()
            self.table_stride = max(self.prompt) // self.B + self.total
            self.page_table = torch.empty((nb, self.table_stride), dtype=torch.int32, device=dev)
            self.win_pages = torch.empty((nb, self.mw), dtype=torch.int32, device=dev)
        else:
            self.kc = torch.empty((L, nb, hkv, self.cap, d), dtype=bf, device=dev)
            self.vc = torch.empty_like(self.kc)
            for l in range(L):  # layer by layer keeps the fp32 staging small
                self.kc[l] = randn(nb, hkv, self.cap, d)
                self.vc[l] = randn(nb, hkv, self.cap, d)
        self.q = randn(L, nb, hq, self.wmax, d)
        self.kw = randn(L, nb, hkv, self.wmax, d)
        self.vw = randn(L, nb, hkv, self.wmax, d)
        self.out = torch.empty((nb, hq, self.wmax, d), dtype=bf, device=dev)
        self.lse = torch.empty((nb, hq, self.wmax), dtype=torch.float32, device=dev)
        rows = nb * self.wmax
        self.pool = [W.logits_normal(rows, self.vocab, cfg["logit_std"], True, device=dev,
                                     seed=100 + r) for r in range(3)]
        desc = d2f.make_desc(nb, hq, hkv, d, self.B, self.mw, self.cap, bf)
        need = d2f.d2f_block_attn_workspace_size(desc, [max(self.prompt)] * nb, [self.mw] * nb)
        self.ws_attn = torch.empty(max(need, 1 << 20) * 4, dtype=torch.uint8, device=dev)
        self.ws_commit = torch.empty(d2f.d2f_confidence_commit_workspace_size(rows, self.vocab),
                                     dtype=torch.uint8, device=dev)
        self.ms = torch.empty(rows, dtype=torch.uint8, device=dev)
        self.tk = torch.empty(rows, dtype=torch.int32, device=dev)
        self.ph = torch.empty(nb * self.mw, dtype=torch.uint8, device=dev)
        self.ncd = torch.empty(nb * self.mw, dtype=torch.int32, device=dev)
        self.bcd = torch.empty(nb * self.mw, dtype=torch.uint8, device=dev)
        self.outt = torch.empty((nb, self.total * self.B), dtype=torch.int32, device=dev)
        self.prefix_dev = torch.empty(nb, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()

    def reset(self):
        import torch
        import block_causal_attention_d2f_amd as d2f
        ms = torch.full((self.nb, self.wmax), d2f.COMMITTED, dtype=torch.uint8)
        ms[:, :self.B] = d2f.MASKED
        self.ms.copy_(ms.reshape(-1))
        self.tk.fill_(self.mask_id)
        ph = torch.zeros((self.nb, self.mw), dtype=torch.uint8)
        ph[:, 0] = d2f.AGGRESSIVE
        self.ph.copy_(ph.reshape(-1))
        self.outt.fill_(-1)
        self.P = list(self.prompt)
        self.prefix_dev.copy_(torch.tensor(self.P, dtype=torch.int32))
        self.wins = [d2f.Window(self.B, self.mw, self.total, self.tau_add, self.tau_act)
                     for _ in range(self.nb)]
        if self.paged:
            import numpy as np
            order = list(self.page_order)
            pt = np.full((self.nb, self.table_stride), -1, dtype=np.int32)
            wp = np.full((self.nb, self.mw), -1, dtype=np.int32)
            for b in range(self.nb):
                n = self.prompt[b] // self.B
                pt[b, :n] = order[len(order) - n:][::-1]
                del order[len(order) - n:]
                wp[b, 0] = order.pop()
            self.page_table.copy_(torch.from_numpy(pt))
            self.win_pages.copy_(torch.from_numpy(wp))
            self.free = order
        torch.cuda.synchronize()

    def step(self, i, ev=None):
        import block_causal_attention_d2f_amd as d2f
        nwin = [w.n_win for w in self.wins]
        rec = (lambda k: ev[k].record()) if ev is not None else (lambda k: None)
        rec(0)
        for l in range(self.L):
            if self.paged:   # the window's K/V are the resident random pages
                d2f.d2f_block_attn_paged(self.q[l], self.kc[l], self.vc[l], self.page_table,
                                         self.win_pages, self.P, nwin, out=self.out,
                                         lse=self.lse, workspace=self.ws_attn)
            else:
                d2f.d2f_block_attn(self.q[l], self.kc[l], self.vc[l], self.kw[l], self.vw[l],
                                   self.P, nwin, self.B, out=self.out, lse=self.lse,
                                   workspace=self.ws_attn)
        rec(1)
        d2f.d2f_confidence_commit(self.pool[i % len(self.pool)], self.ms, self.tk, self.ph,
                                  self.B, self.tau, self.k_aggr, self.mask_id, n_committed=self.ncd,
                                  block_complete=self.bcd, workspace=self.ws_commit,
                                  want_conf=False)
        rec(2)
        if self.paged:
            new = [self.free.pop() for _ in range(self.nb)]
            _, app = d2f.d2f_decode_advance_paged(
                self.page_table, self.win_pages, new, self.wins, self.P, self.ncd, self.ms,
                self.tk, self.ph, self.outt, self.mask_id, n_heads_kv=self.hkv, head_dim=self.d,
                prefix_len_dev=self.prefix_dev)
            self.free.extend(pg for pg, a in zip(new, app) if not a)
        else:
            d2f.d2f_decode_advance(self.kc, self.vc, self.kw, self.vw, self.wins, self.P,
                                   self.ncd, self.ms, self.tk, self.ph, self.outt, self.mask_id,
                                   prefix_len_dev=self.prefix_dev)
        rec(3)
        return nwin

    def decode(self, events=False):
        """One complete decode; returns the per-step windows and events, and
        the wall time of the steps (the set-up of the decode is not timed)."""
        import torch
        self.reset()
        t0 = time.perf_counter()
        steps = []
        while not all(w.done for w in self.wins):
            if len(steps) > 100 * self.total:
                raise RuntimeError("decoding did not finish")
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if events else None
            prefix = list(self.P)
            nwin = self.step(len(steps), ev)
            steps.append((prefix, nwin, ev))
        torch.cuda.synchronize()
        self.wall = time.perf_counter() - t0
        return steps


def decode_loop_main(args):
    import torch
    import workloads as W
    lp = DecodeLoop(args)
    lp.decode()                                   # warm-up decode (untimed)
    outs = lp.outt.clone()
    walls, n_steps = [], []
    for _ in range(args.loop_reps):
        st = lp.decode()
        walls.append(lp.wall)
        n_steps.append(len(st))
        assert torch.equal(lp.outt, outs), "decodes of the same inputs differ"
    assert (outs >= 0).all() and (outs != lp.mask_id).all(), "undecoded positions left"
    # One more decode with events around the three phases of every step.
    st = lp.decode(events=True)
    t_attn = t_commit = t_adv = 0.0
    a_bytes = a_flops = 0.0
    for prefix, nwin, ev in st:
        t_attn += ev[0].elapsed_time(ev[1]) * 1e-3
        t_commit += ev[1].elapsed_time(ev[2]) * 1e-3
        t_adv += ev[2].elapsed_time(ev[3]) * 1e-3
        sh = W.make_shape(lp.nb, lp.hq, lp.hkv, lp.d, lp.B, prefix, nwin, dtype="bf16",
                          max_win_blocks=lp.mw, cache_capacity=lp.cap)
        a_bytes += attn_bytes(sh) * lp.L
        a_flops += attn_flops(sh) * lp.L
    tokens = lp.nb * lp.total * lp.B
    wall = sum(walls) / len(walls)
    steps = sum(n_steps) / len(n_steps)
    attn_gbs = a_bytes / t_attn / 1e9
    rec = {
        "metric": LOOP_METRIC,
        "value": round(tokens / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": int(round(steps)),
        "warmup": 1,
        "ms_per_step": round(wall / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "pipelined decoding of the batched ragged LLaDA-8B-shaped batch",
                   "batch": lp.nb, "heads_q": lp.hq, "heads_kv": lp.hkv, "head_dim": lp.d,
                   "layers": lp.L, "block_size": lp.B, "blocks_per_request": lp.total,
                   "max_window_blocks": lp.mw, "prompt_len": f"U(256, 4096), mean "
                   f"{sum(lp.prompt) / lp.nb:.0f}", "vocab": lp.vocab, "tau": lp.tau,
                   "k_aggr": lp.k_aggr, "tau_add": lp.tau_add, "tau_act": lp.tau_act,
                   "timed_decodes": args.loop_reps, "launch": "eager",
                   "kv_layout": "paged" if lp.paged else "contiguous"},
        "tokens_per_decode": tokens,
        "tokens_per_step": round(tokens / steps, 2),
        "wall_s_per_decode": round(wall, 5),
        "phase_ms_per_step": {"attention_all_layers": round(t_attn / len(st) * 1e3, 4),
                              "commit": round(t_commit / len(st) * 1e3, 4),
                              "advance_incl_sync": round(t_adv / len(st) * 1e3, 4)},
        "roofline": {"kernel": "d2f_block_attn", "bound": "hbm", "achieved": round(attn_gbs, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "tflops": round(a_flops / t_attn / 1e12, 3)},
    }
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.summarize_mfma:
        summarize_mfma(args)
        return
    if args.summarize_trace:
        summarize_trace(args)
        return
    if args.summarize_stall:
        summarize_stall(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the D2F step here runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration()
        return
    import block_causal_attention_d2f_amd as d2f
    d2f.load()
    if args.decode_loop:
        decode_loop_main(args)
        return
    K, Wu = args.steps, args.warmup
    n_masks = Wu + K + args.call_reps + 1
    wl = Workload(args.config, args.block_size, n_masks, args.measure, args.early_gap,
                  args.paged, args.round_prefix)
    # A per-call graph visits every input set, so that a repeated call reads
    # HBM rather than the Infinity Cache.
    call_reps = max(args.call_reps, wl.n_sets)
    n_masks = Wu + K + call_reps + 1
    wl.ensure_masks(n_masks)
    sh = wl.sh
    use_graph = not args.no_graph

    # One eager step first (it also proves the path runs) on a spare mask set.
    wl.step(n_masks - 1)
    torch.cuda.synchronize()
    ties = near_ties(wl)

    warm = capture(lambda: [wl.step(i) for i in range(Wu)], use_graph)
    timed = capture(lambda: [wl.step(Wu + i) for i in range(K)], use_graph)
    torch.cuda.synchronize()
    warm()
    torch.cuda.synchronize()
    ms_total, wall_ms = time_region(timed)
    ms_step = ms_total / K

    calls = per_call_times(wl, call_reps, use_graph)
    spread = per_call_spread(wl, args.call_reps)
    a_bytes = attn_bytes(sh)
    a_flops = attn_flops(sh)
    c_bytes = commit_bytes(wl.n_masked, wl.rows, wl.cfg["vocab"])
    kv_b = wl.kv_bytes()
    t_attn = calls["d2f_block_attn"] * 1e-3
    t_commit = calls["d2f_confidence_commit"] * 1e-3
    t_kv = calls["d2f_kv_commit"] * 1e-3
    attn_gbs = a_bytes / t_attn / 1e9
    attn_tflops = a_flops / t_attn / 1e12
    commit_gbs = c_bytes / t_commit / 1e9
    shares = {"d2f_block_attn": t_attn * wl.layers, "d2f_confidence_commit": t_commit,
              "d2f_kv_commit": t_kv}
    dom = max(shares, key=shares.get)
    ai = a_flops / a_bytes
    if dom == "d2f_block_attn":
        if ai * PEAK_HBM_GBS / 1e3 >= PEAK_BF16_TFLOPS:
            roof = dict(kernel=dom, bound="mfma", achieved=round(attn_tflops, 3),
                        peak=PEAK_BF16_TFLOPS, unit="TFLOP/s")
        else:
            roof = dict(kernel=dom, bound="hbm", achieved=round(attn_gbs, 2), peak=PEAK_HBM_GBS,
                        unit="GB/s")
        per_launch = a_bytes
    elif dom == "d2f_confidence_commit":
        roof = dict(kernel=dom, bound="hbm", achieved=round(commit_gbs, 2), peak=PEAK_HBM_GBS,
                    unit="GB/s")
        per_launch = c_bytes
    else:
        roof = dict(kernel=dom, bound="hbm", achieved=round(kv_b / t_kv / 1e9, 2),
                    peak=PEAK_HBM_GBS, unit="GB/s")
        per_launch = kv_b
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(traffic_key(args), dom)
    roof["avg_us"] = round(shares[dom] / (wl.layers if dom == "d2f_block_attn" else 1) * 1e6, 3)
    roof["algorithmic_bytes_per_launch"] = per_launch

    step_bytes = wl.step_bytes()
    value = step_bytes / (ms_step * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wu,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if sh.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.cfg["workload"], "name": args.config, "batch": sh.batch,
                   "heads_q": sh.n_heads_q, "heads_kv": sh.n_heads_kv, "head_dim": sh.head_dim,
                   "block_size": sh.block_size, "prefix_len": (sh.prefix_len if sh.batch <= 4 else
                                                               f"ragged, mean {sum(sh.prefix_len) / sh.batch:.0f}"),
                   "n_win_blocks": (sh.n_win_blocks if sh.batch <= 4 else
                                    f"ragged, {sum(sh.n_win_blocks)} blocks"),
                   "layers": wl.layers, "vocab": wl.cfg["vocab"], "commit_rows": wl.rows,
                   "tau": wl.tau, "measure": args.measure, "early_gap": args.early_gap,
                   "kv_layout": "paged" if args.paged else "contiguous",
                   "prefix_whole_blocks": bool(args.paged or args.round_prefix),
                   "input_sets": wl.n_sets, "per_call_graph_launches": call_reps,
                   "input_set_bytes": wl.set_bytes,
                   "launch": "hip-graph" if use_graph else "eager"},
        "step_bytes": step_bytes,
        "wall_ms_per_step": round(wall_ms / K, 5),
        "attn": {"avg_us": round(t_attn * 1e6, 3),
                 "p10_us": spread["d2f_block_attn"][0], "median_us": spread["d2f_block_attn"][1],
                 "p90_us": spread["d2f_block_attn"][2], "tflops": round(attn_tflops, 3),
                 "frac_mfma": round(attn_tflops / PEAK_BF16_TFLOPS, 5),
                 "gbs": round(attn_gbs, 2), "frac_hbm": round(attn_gbs / PEAK_HBM_GBS, 4),
                 "kv_read_gbs": round(attn_kv_bytes(sh) / t_attn / 1e9, 2),
                 "flops": a_flops, "bytes": a_bytes, "intensity": round(ai, 2)},
        "commit": {"avg_us": round(t_commit * 1e6, 3),
                   "p10_us": spread["d2f_confidence_commit"][0], "median_us": spread["d2f_confidence_commit"][1],
                   "p90_us": spread["d2f_confidence_commit"][2], "logit_gbs": round(commit_gbs, 2),
                   "frac_hbm": round(commit_gbs / PEAK_HBM_GBS, 4), "bytes": c_bytes,
                   "masked_rows": wl.n_masked},
        "kv_commit": {"avg_us": round(t_kv * 1e6, 3),
                      "p10_us": spread["d2f_kv_commit"][0], "median_us": spread["d2f_kv_commit"][1],
                      "p90_us": spread["d2f_kv_commit"][2], "gbs": round(kv_b / t_kv / 1e9, 2),
                      "bytes": kv_b},
        "roofline": roof,
        "near_ties": ties,
    }
    if args.reuse and not args.paged:
        rec["reuse"] = reuse_times(wl, call_reps, use_graph)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    if args.other_workloads and not (args.paged or args.round_prefix or args.reuse):
        del wl, warm, timed
        torch.cuda.empty_cache()
        rec["other_workloads"] = other_workloads(args, use_graph)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
