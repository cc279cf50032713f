#!/usr/bin/env python3
"""Benchmark of the MI355X flash-attention forward path; prints one JSON line.

Headline (value): long-context GQA decode, bf16, B=1 Hq=32 Hkv=4 Sq=1
Sk=32768 d=128 -- KV bytes read per second over whole steps (forward kernel
plus log-sum-exp combine), with the KV cache rotated over enough copies that
every step reads HBM rather than the 256 MB last-level cache.
Secondary (prefill): causal prefill, bf16, B=1 H=32 S=8192 d=128 -- TFLOP/s
over visible (query, key) pairs only.

A step is one call of the library on one batch of synthetic inputs already
resident in GPU memory. Per-kernel durations come from HIP events the library
records around each launch (on the launch stream) in a separate pass.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
LLC_BYTES = 256 << 20       # MI355X Infinity Cache

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "tiled_prefill_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
TIMES_FILE = os.path.join(ROOT, "profiles", "kernel_times.json")
# kernel -> source file it is compiled from
KERNEL_SOURCES = {"attn_decode_kernel": "attn_decode.hip", "attn_decode_kdma_kernel": "attn_decode.hip",
                  "lse_combine_kernel": "attn_decode.hip", "lse_combine_cols_kernel": "attn_decode.hip",
                  "lse_combine_cols_small_kernel": "attn_decode.hip",
                  "lse_combine_rows_kernel": "attn_decode.hip",
                  "attn_prefill_kernel": "attn_prefill.hip", "attn_fwd_kernel": "attn_fwd.hip",
                  "attn_mla_kernel": "attn_mla.hip", "stream_read_kernel": "attn_tools.hip",
                  "attn_bwd_dkdv_dma_kernel": "attn_bwd.hip", "attn_bwd_dq_dma_kernel": "attn_bwd.hip",
                  "attn_fwd_f32_dma_kernel": "attn_fwd_f32.hip", "attn_decode_kv_kernel": "attn_decode.hip"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only", choices=["decode", "prefill", "backward"], default=None,
                    help="run one leg only (for profiling)")
    ap.add_argument("--suite", action="store_true",
                    help="time every workload (one JSON line each) instead of the headline line")
    ap.add_argument("--workload", default=None, help="with --suite: time only this workload")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="first copy a buffer of this many MiB three times (a plain copy "
                         "of known size, to calibrate HBM byte counters)")
    ap.add_argument("--summarize-rocprof", default=None, metavar="DIR",
                    help="summarise the rocprofv3 kernel trace under DIR into "
                         "profiles/kernel_trace_<workload>.md and profiles/kernel_times.json")
    ap.add_argument("--rocprof-cmd", default="", help="with --summarize-rocprof: the command that made DIR")
    ap.add_argument("--title", default="", help="with --summarize-rocprof: what the trace covers")
    ap.add_argument("--summarize-counters", nargs="+", default=None, metavar="DIR",
                    help="summarise rocprofv3 --pmc runs (one DIR per pass) into "
                         "profiles/counters_<workload>.md; --rocprof-cmd names each pass's command, '|'-separated")
    ap.add_argument("--summarize-traffic", nargs=2, default=None, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="HBM bytes per launch from a rocprofv3 --pmc FETCH_SIZE pass and a WRITE_SIZE pass "
                         "(each run with --copy-mb), calibrated on the copies: profiles/hbm_traffic_<workload>.md "
                         "and profiles/traffic.json")
    return ap.parse_args()


# the decode kernel the planner selects (ATTN_DECODE_KDMA: 0 the register-K form with
# 16-row V tiles, 2 K in registers with whole-block V; default 1, K and V through LDS)
DECODE_KERNEL = {"0": "attn_decode_kernel", "2": "attn_decode_kv_kernel"}.get(
    os.environ.get("ATTN_DECODE_KDMA", "").strip(), "attn_decode_kdma_kernel")


# headers whose inline device code every kernel source compiles in
SHARED_SOURCES = ("attn_device.h", "attn_plan.h")


def source_hash(kernel: str) -> str:
    """sha256[:16] over the kernel's source file and the shared device headers."""
    h = hashlib.sha256()
    for name in (KERNEL_SOURCES[kernel],) + SHARED_SOURCES:
        h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """Counter-derived HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated),
    if they were recorded for the current source of that kernel; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = rec.get(f"{kernel}:{workload}")
    if not e or e.get("source_sha") != source_hash(kernel):
        return None
    return e.get("bytes_per_launch")


def kernel_time_for(kernel: str, workload: str):
    """rocprofv3 kernel-trace durations (us: mean, median, ...) of a kernel on a
    workload, if they were recorded for the current source of that kernel; else None."""
    try:
        rec = json.load(open(TIMES_FILE))
    except (OSError, ValueError):
        return None
    e = rec.get(f"{kernel}:{workload}")
    if not e or e.get("source_sha") != source_hash(kernel):
        return None
    return e


def summarize_rocprof(args):
    """Per-kernel duration statistics of a rocprofv3 --kernel-trace run (every
    dispatch in the trace): a markdown summary under profiles/ and, for the
    kernels bench.py reports, an entry in profiles/kernel_times.json keyed on the
    kernel's source hash."""
    import csv
    import glob
    import re
    import statistics
    files = glob.glob(os.path.join(args.summarize_rocprof, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        sys.exit(f"no kernel_trace.csv under {args.summarize_rocprof}")
    durs = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            name = re.sub(r"\(.*\)$", "", r["Kernel_Name"]).replace("void ", "").replace("tpa::", "")
            durs.setdefault(name, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in durs.values())
    lines = [f"# Kernel trace: {args.title or args.workload}", "",
             "command (from the repository root on one MI355X, TMPDIR=/tmp), then this summary:", "",
             f"    {args.rocprof_cmd}",
             f"    python3 bench.py --summarize-rocprof {args.summarize_rocprof} --workload {args.workload}",
             "", "Durations in us over every dispatch of the run (warm-up and timed steps alike).", "",
             "| kernel | calls | mean | median | p10 | p90 | min | max | share % |",
             "|---|---|---|---|---|---|---|---|---|"]
    try:
        times = json.load(open(TIMES_FILE))
    except (OSError, ValueError):
        times = {}
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        v = sorted(v)
        q = lambda f: v[min(len(v) - 1, int(f * len(v)))]
        st = {"calls": len(v), "mean_us": round(statistics.fmean(v), 3),
              "median_us": round(statistics.median(v), 3), "p10_us": round(q(0.1), 3),
              "p90_us": round(q(0.9), 3), "min_us": round(v[0], 3), "max_us": round(v[-1], 3)}
        lines.append(f"| {name} | {st['calls']} | {st['mean_us']:.2f} | {st['median_us']:.2f} | "
                     f"{st['p10_us']:.2f} | {st['p90_us']:.2f} | {st['min_us']:.2f} | {st['max_us']:.2f} | "
                     f"{100 * sum(v) / total:.1f} |")
        base = name.split("<")[0]
        if base in KERNEL_SOURCES:
            times[f"{base}:{args.workload}"] = dict(st, kernel=name, source=KERNEL_SOURCES[base],
                                                    source_sha=source_hash(base))
    out = os.path.join(ROOT, "profiles", f"kernel_trace_{args.workload}.md")
    open(out, "w").write("\n".join(lines) + "\n")
    json.dump(times, open(TIMES_FILE, "w"), indent=1, sort_keys=True)
    print(out)


def summarize_counters(args, num_cus=256, num_xcd=8):
    """Per-kernel means of rocprofv3 --pmc counters (values summed over the GPU's
    instances, averaged over a kernel's dispatches), plus derived shares:
      cycles per XCD     = GRBM_GUI_ACTIVE / 8
      MFMA busy          = SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x 256 CUs x cycles per XCD)
      VALU / MFMA per wave = SQ_INSTS_VALU / SQ_WAVES, SQ_INSTS_MFMA / SQ_WAVES
      waiting            = SQ_WAIT_ANY / SQ_WAVE_CYCLES (share of wave lifetime)
      VALU active        = SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES
      LDS bank conflicts = SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS"""
    import csv
    import glob
    import re
    vals = {}
    for d in args.summarize_counters:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                name = re.sub(r"\(.*\)$", "", r["Kernel_Name"]).replace("void ", "").replace("tpa::", "")
                vals.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    cmds = [c.strip() for c in args.rocprof_cmd.split("|") if c.strip()]
    lines = [f"# Counters: {args.title or args.workload}", "",
             "commands (from the repository root on one MI355X, TMPDIR=/tmp; one pass each), then this summary:", ""]
    lines += [f"    {c}" for c in cmds]
    lines += [f"    python3 bench.py --summarize-counters {' '.join(args.summarize_counters)} "
              f"--workload {args.workload}", "",
              "Mean per dispatch of each counter (summed over the GPU). Derived: cycles per XCD = "
              "GRBM_GUI_ACTIVE / 8; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (4 x 256 x cycles per XCD); "
              "per wave = SQ_INSTS_* / SQ_WAVES; waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES; VALU active = "
              "SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES; LDS conflicts = SQ_LDS_BANK_CONFLICT / "
              "SQ_ACTIVE_INST_LDS.", ""]
    mean = lambda v: sum(v) / len(v)
    for name, cs in sorted(vals.items()):
        if name.startswith("__amd"):
            continue
        m = {c: mean(v) for c, v in cs.items()}
        lines += [f"## {name}", "", "| counter | dispatches | mean |", "|---|---|---|"]
        lines += [f"| {c} | {len(cs[c])} | {m[c]:.6g} |" for c in sorted(m)]
        der = []
        if "GRBM_GUI_ACTIVE" in m:
            cyc = m["GRBM_GUI_ACTIVE"] / num_xcd
            der.append(f"cycles per XCD {cyc:.4g}")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                der.append(f"MFMA busy {100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * num_cus * cyc):.1f}%")
        if "SQ_WAVES" in m and m["SQ_WAVES"] > 0:
            for c, lab in (("SQ_INSTS_VALU", "VALU"), ("SQ_INSTS_MFMA", "MFMA"), ("SQ_INSTS_LDS", "LDS"),
                           ("SQ_INSTS_VMEM_RD", "VMEM reads")):
                if c in m:
                    der.append(f"{lab} per wave {m[c] / m['SQ_WAVES']:.1f}")
        if "SQ_WAVE_CYCLES" in m and m["SQ_WAVE_CYCLES"] > 0:
            for c, lab in (("SQ_WAIT_ANY", "waiting"), ("SQ_ACTIVE_INST_VALU", "VALU active"),
                           ("SQ_WAIT_INST_LDS", "waiting on LDS")):
                if c in m:
                    der.append(f"{lab} {100 * m[c] / m['SQ_WAVE_CYCLES']:.1f}% of wave cycles")
        if "SQ_LDS_BANK_CONFLICT" in m and m.get("SQ_ACTIVE_INST_LDS", 0) > 0:
            der.append(f"LDS conflicts {m['SQ_LDS_BANK_CONFLICT'] / m['SQ_ACTIVE_INST_LDS']:.3f} per LDS active cycle")
        lines += ["", "derived: " + "; ".join(der), ""]
    out = os.path.join(ROOT, "profiles", f"counters_{args.workload}.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print(out)


def algorithmic_bytes(kernel: str, workload: str):
    """(read, write) bytes one launch of `kernel` needs on `workload` if every
    input were read and every output written exactly once: forward kernels read
    Q and the K/V rows that exist (variable lengths: the sum of the key lengths)
    and write O + lse, or the split partials; the combine reads the partials and
    writes O + lse; the backward's key-block and query-block kernels read Q, dO,
    K, V and the two per-row vectors and write dK + dV, or dQ."""
    from workloads import WORKLOADS, BWD_WORKLOADS, LATENT_WORKLOADS, make_inputs
    import tiled_prefill_amd as tpa
    if workload in LATENT_WORKLOADS:  # keys 576 wide, values 512, one shared KV head
        B, Hq, Sq, Sk = LATENT_WORKLOADS[workload]
        rows = B * Sq * Hq
        plan = tpa.plan_dv(B, Hq, 1, Sq, Sk, 576, 512, True, -1, 0, "bf16")
        part = plan["num_splits"] * rows * (512 + 1) * 4 if plan["num_splits"] > 1 else 0
        o_bytes = rows * 512 * 2 + rows * 4
        if kernel.startswith("lse_combine"):
            return part, o_bytes
        return rows * 576 * 2 + B * Sk * (576 + 512) * 2, part or o_bytes
    w = WORKLOADS.get(workload) or BWD_WORKLOADS.get(workload)
    if w is None:
        return None
    esz = 4 if w.dtype == "fp32" else 2
    q_bytes = w.B * w.Sq * w.Hq * w.d * esz
    rows = w.B * w.Sq * w.Hq
    keys = w.B * w.Sk
    if getattr(w, "varlen", False):
        keys = int(make_inputs(w, seed=0)[3].sum())
    kv_bytes = 2 * keys * w.Hkv * w.d * esz
    o_bytes = q_bytes + rows * 4
    if kernel.startswith("attn_bwd_"):
        reads = 2 * q_bytes + kv_bytes + 2 * rows * 4
        return reads, (kv_bytes if "dkdv" in kernel else q_bytes)
    if kernel == "stream_read_kernel":  # the decode leg's reference: K and V bytes, read only
        return kv_bytes, 0
    plan = tpa.plan(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.causal, w.window_left, 0, w.dtype,
                    varlen=getattr(w, "varlen", False), sum_seqlens_k=keys if getattr(w, "varlen", False) else -1)
    part = plan["num_splits"] * rows * (w.d + 1) * 4 if plan["num_splits"] > 1 else 0
    if kernel.startswith("lse_combine"):
        return part, o_bytes
    return q_bytes + kv_bytes, part or o_bytes


def summarize_traffic(args):
    """HBM bytes per launch from FETCH_SIZE and WRITE_SIZE (KiB per dispatch,
    summed over the GPU), each scaled by what the same counter reads for the
    plain copies of --copy-mb MiB that the profiled run made first (the largest
    copy dispatches of the pass): scale = copied bytes / counter bytes."""
    import csv
    import glob
    import re
    copy = args.copy_mb << 20
    if copy <= 0:
        sys.exit("--summarize-traffic needs --copy-mb (the size of the calibration copies)")
    per = {}
    scales = {}
    for d, counter in zip(args.summarize_traffic, ("FETCH_SIZE", "WRITE_SIZE")):
        vals, copies = {}, []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                name = re.sub(r"\(.*\)$", "", r["Kernel_Name"]).replace("void ", "").replace("tpa::", "")
                v = float(r["Counter_Value"]) * 1024
                if name.startswith("__amd_rocclr_copyBuffer"):
                    copies.append(v)
                else:
                    vals.setdefault(name, []).append(v)
        if not copies:
            sys.exit(f"no copy dispatches in {d}: run the pass with --copy-mb")
        big = [v for v in copies if v > 0.9 * max(copies)]
        scales[counter] = copy / (sum(big) / len(big))
        for name, v in vals.items():
            per.setdefault(name, {})[counter] = (len(v), sum(v) / len(v) * scales[counter])
    cmds = [c.strip() for c in args.rocprof_cmd.split("|") if c.strip()]
    lines = [f"# HBM traffic per launch: {args.title or args.workload}", "",
             "commands (from the repository root on one MI355X, TMPDIR=/tmp; one pass per counter), then this summary:",
             ""] + [f"    {c}" for c in cmds] + [
             f"    python3 bench.py --summarize-traffic {' '.join(args.summarize_traffic)} --workload {args.workload} "
             f"--copy-mb {args.copy_mb}", "",
             f"Each pass first copies a {args.copy_mb} MiB buffer three times; a counter's scale is the copied bytes "
             f"over what it reads for those copies (FETCH_SIZE {scales['FETCH_SIZE']:.4f}, "
             f"WRITE_SIZE {scales['WRITE_SIZE']:.4f}). Bytes are per launch, averaged over the kernel's dispatches; "
             "algorithmic bytes read every input and write every output once.", "",
             "| kernel | dispatches | fetched MB | written MB | algorithmic read MB | algorithmic write MB | fetch / algorithmic read |",
             "|---|---|---|---|---|---|---|"]
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        rec = {}
    for name, c in sorted(per.items(), key=lambda kv: -kv[1].get("FETCH_SIZE", (0, 0))[1]):
        if "FETCH_SIZE" not in c or "WRITE_SIZE" not in c or name.startswith("at::"):
            continue  # (torch's own kernels: input fills and copies)
        fb, wb = c["FETCH_SIZE"][1], c["WRITE_SIZE"][1]
        base = name.split("<")[0]
        alg = algorithmic_bytes(base, args.workload) if base in KERNEL_SOURCES else None
        ratio = f"{fb / alg[0]:.2f}" if alg and alg[0] else "-"
        lines.append(f"| {name} | {c['FETCH_SIZE'][0]} | {fb / 1e6:.2f} | {wb / 1e6:.2f} | "
                     f"{alg[0] / 1e6 if alg else float('nan'):.2f} | {alg[1] / 1e6 if alg else float('nan'):.2f} | {ratio} |")
        if base in KERNEL_SOURCES:
            rec[f"{base}:{args.workload}"] = {
                "kernel": name, "source": KERNEL_SOURCES[base], "source_sha": source_hash(base),
                "bytes_per_launch": int(fb + wb), "fetch_bytes": int(fb), "write_bytes": int(wb),
                "fetch_scale": round(scales["FETCH_SIZE"], 4), "write_scale": round(scales["WRITE_SIZE"], 4),
                "algorithmic_read_bytes": alg[0] if alg else None, "algorithmic_write_bytes": alg[1] if alg else None}
    out = os.path.join(ROOT, "profiles", f"hbm_traffic_{args.workload}.md")
    open(out, "w").write("\n".join(lines) + "\n")
    json.dump(rec, open(TRAFFIC_FILE, "w"), indent=1, sort_keys=True)
    print(out)


def warm(step, n_steps, min_seconds=0.3):
    """Untimed warmup: n_steps steps, then more until min_seconds of GPU work have
    run, so that the GPU clocks have settled before the timed region."""
    import torch
    i = 0
    for i in range(n_steps):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_seconds:
        for _ in range(8):
            i += 1
            step(i)
        torch.cuda.synchronize()


def visible_pairs(w, seqlens=None):
    """Visible (query, key) pairs of workload w: sum over rows of the key interval
    length (bottom-right aligned causal / window mask)."""
    total = 0
    for b in range(w.B):
        skb = int(seqlens[b]) if seqlens is not None else w.Sk
        delta = skb - w.Sq
        for i in range(w.Sq):
            hi = min(skb - 1, i + delta) if w.causal else skb - 1
            lo = max(0, i + delta - w.window_left) if w.window_left >= 0 else 0
            total += max(0, hi - lo + 1)
    return total * w.Hq


def visible_kv_rows(w, seqlens=None):
    """Key rows some query row of a (batch, KV head) can see, summed over batches."""
    total = 0
    for b in range(w.B):
        skb = int(seqlens[b]) if seqlens is not None else w.Sk
        delta = skb - w.Sq
        hi = min(skb - 1, w.Sq - 1 + delta) if w.causal else skb - 1
        lo = max(0, delta - w.window_left) if w.window_left >= 0 else 0
        total += max(0, hi - lo + 1)
    return total


def run_suite(args):
    import torch
    import tiled_prefill_amd as tpa
    from workloads import WORKLOADS, make_inputs
    dev = "cuda:0"
    for name, w in WORKLOADS.items():
        if args.workload and name != args.workload:
            continue
        q, k, v, seqlens = make_inputs(w, seed=0, device=dev)
        esz = 4 if w.dtype == "fp32" else 2
        sl = seqlens.cpu() if seqlens is not None else None
        kv_bytes = 2 * visible_kv_rows(w, sl) * w.Hkv * w.d * esz
        flops = 4.0 * w.d * visible_pairs(w, sl)
        memory_bound = w.Sq * (w.Hq // w.Hkv) <= 32
        n_rot = max(1, min(16, math.ceil(2 * LLC_BYTES / max(1, 2 * w.B * w.Sk * w.Hkv * w.d * esz)))) \
            if memory_bound else 1
        ks = [k] + [k.clone() for _ in range(n_rot - 1)]
        vs = [v] + [v.clone() for _ in range(n_rot - 1)]
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
        total_k = int(seqlens.sum()) if seqlens is not None else -1

        def step(i):
            if seqlens is not None:
                tpa.fwd_varlen(q, ks[i % n_rot], vs[i % n_rot], seqlens, causal=w.causal,
                               window_left=w.window_left, sum_seqlens_k=total_k, out=o, lse=lse)
            else:
                tpa.fwd(q, ks[i % n_rot], vs[i % n_rot], causal=w.causal,
                        window_left=w.window_left, out=o, lse=lse)

        warm(step, 10)
        t0 = time.perf_counter()
        step(0)
        torch.cuda.synchronize()
        one = time.perf_counter() - t0
        steps = max(5, min(2000, int(0.3 / max(one, 1e-6))))
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        tpa.profile_begin(2 * steps + 8)
        for i in range(steps):
            step(i)
        prof = tpa.profile_end()
        plan = tpa.plan(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.causal, w.window_left, dtype=w.dtype,
                        varlen=w.varlen, sum_seqlens_k=total_k)
        rec = {"workload": name, "dtype": w.dtype, "ms_per_step": round(ms, 5),
               "kv_GBps": round(kv_bytes / (ms * 1e-3) / 1e9, 1),
               "pct_hbm": round(100 * kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
               "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
               "fwd_us": round(1e3 * prof["fwd_ms"] / max(1, prof["fwd_launches"]), 2),
               "combine_us": round(1e3 * prof["combine_ms"] / max(1, prof["combine_launches"]), 2),
               "num_splits": plan["num_splits"], "pack_gqa": plan["pack_gqa"],
               "block_m": plan["block_m"], "block_n": plan["block_n"], "kv_copies": n_rot,
               "kv_bytes": kv_bytes, "flops": flops, "steps": steps}
        if w.dtype == "bf16" and not memory_bound:
            rec["pct_mfma_bf16"] = round(100 * rec["TFLOPs"] / BF16_PEAK_TFLOPS, 2)
        print(json.dumps(rec), flush=True)
        del ks, vs, q, k, v, o
    run_latent_suite(args)
    run_bwd_suite(args)


def run_bwd_suite(args):
    """Backward workloads (attn_bwd) on the prefill shapes: TFLOP/s over the five
    matrix products of the backward (10 d flops per visible pair)."""
    import torch
    import tiled_prefill_amd as tpa
    from workloads import BWD_WORKLOADS, make_inputs, output_grad
    dev = "cuda:0"
    for name, w in BWD_WORKLOADS.items():
        if args.workload and name != args.workload:
            continue
        q, k, v, _ = make_inputs(w, seed=0, device=dev)
        g = output_grad(0, q.shape, w.dtype, device=dev)
        o, lse = tpa.fwd(q, k, v, causal=w.causal, window_left=w.window_left)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        flops = 10.0 * w.d * visible_pairs(w)

        def step(i=0):
            tpa.bwd(q, k, v, o, g, lse, causal=w.causal, window_left=w.window_left,
                    dq=dq, dk=dk, dv=dv)

        warm(step, 3)
        steps = max(5, min(200, args.prefill_steps * 2))
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        tpa.profile_begin(4 * steps + 8)
        for i in range(steps):
            step(i)
        prof = tpa.profile_end_kinds()
        plan = tpa.plan_bwd(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.causal, w.window_left, w.dtype)
        n = max(1, prof["bwd_launches"])
        rec = {"workload": name, "dtype": w.dtype, "ms_per_step": round(ms, 5),
               "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
               "pct_mfma_bf16": round(100 * flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 2),
               "dkdv_us": round(1e3 * prof["bwd_ms"] / n, 2),
               "dq_us": round(1e3 * prof["bwd_dq_ms"] / n, 2),
               "pre_us": round(1e3 * prof["bwd_prepost_ms"] / n, 2),
               "block_n": plan["block_n"], "block_m": plan["block_m"],
               "dq_block_m": plan["dq_block_m"], "flops": flops, "steps": steps}
        print(json.dumps(rec), flush=True)
        del q, k, v, g, o, dq, dk, dv


def run_latent_suite(args):
    """Latent-attention verify workloads (values of their own width, attn_fwd_dv)."""
    import torch
    import tiled_prefill_amd as tpa
    from workloads import LATENT_WORKLOADS, latent_case
    dev = "cuda:0"
    for name, (B, Hq, Sq, Sk) in LATENT_WORKLOADS.items():
        if args.workload and name != args.workload:
            continue
        q, k, v = (t.to(dev) for t in latent_case(0, B, Hq, Sq, Sk))
        kv_bytes = B * Sk * (576 + 512) * 2
        pairs = B * Hq * sum(min(i + 1 + Sk - Sq, Sk) for i in range(Sq))
        flops = 2.0 * (576 + 512) * pairs
        n_rot = max(1, min(16, math.ceil(2 * LLC_BYTES / kv_bytes)))
        ks = [k] + [k.clone() for _ in range(n_rot - 1)]
        vs = [v] + [v.clone() for _ in range(n_rot - 1)]
        o = torch.empty((B, Sq, Hq, 512), dtype=q.dtype, device=dev)
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)

        def step(i):
            tpa.fwd_dv(q, ks[i % n_rot], vs[i % n_rot], causal=True, out=o, lse=lse)

        warm(step, args.warmup)
        steps = max(20, args.steps)
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        tpa.profile_begin(2 * steps + 8)
        for i in range(steps):
            step(i)
        prof = tpa.profile_end()
        plan = tpa.plan_dv(B, Hq, 1, Sq, Sk, 576, 512, causal=True)
        rec = {"workload": name, "dtype": "bf16", "B": B, "Hq": Hq, "Hkv": 1, "Sq": Sq, "Sk": Sk,
               "d": 576, "d_v": 512, "ms_per_step": round(ms, 5),
               "kv_GBps": round(kv_bytes / (ms * 1e-3) / 1e9, 1),
               "pct_hbm": round(100 * kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
               "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
               "pct_mfma_bf16": round(100 * flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 2),
               "fwd_us": round(1e3 * prof["fwd_ms"] / max(1, prof["fwd_launches"]), 2),
               "combine_us": round(1e3 * prof["combine_ms"] / max(1, prof["combine_launches"]), 2),
               "num_splits": plan["num_splits"], "grid": plan["grid_x"], "kv_copies": n_rot,
               "kv_bytes": kv_bytes, "flops": flops, "steps": steps}
        print(json.dumps(rec), flush=True)
        del ks, vs, q, k, v, o


def main():
    args = parse()
    if args.summarize_rocprof:
        summarize_rocprof(args)
        return
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.summarize_traffic:
        summarize_traffic(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(every workload fits one MI355X); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import tiled_prefill_amd as tpa
    from workloads import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    tpa.load()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_mb > 0:  # plain copies of known size, to calibrate HBM byte counters
        src = torch.ones(args.copy_mb << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.suite:
        run_suite(args)
        return
    out = {}

    # ------------------------------------------------------------------ decode
    w = WORKLOADS["gqa_decode_bf16"]
    esz = 2
    kv_bytes = 2 * w.B * w.Sk * w.Hkv * w.d * esz            # K and V, every row visible
    q_bytes = w.B * w.Sq * w.Hq * w.d * esz
    o_bytes = q_bytes + w.B * w.Hq * w.Sq * 4                 # O plus lse
    plan = tpa.plan(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.causal, w.window_left, dtype=w.dtype)
    if args.only in (None, "decode"):
        q, k, v, _ = make_inputs(w, seed=0, device=dev)
        n_rot = max(2, math.ceil(2 * LLC_BYTES / kv_bytes))
        ks = [k] + [k.clone() for _ in range(n_rot - 1)]
        vs = [v] + [v.clone() for _ in range(n_rot - 1)]
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)

        def step(i):
            tpa.fwd(q, ks[i % n_rot], vs[i % n_rot], causal=False, out=o, lse=lse)

        warm(step, args.warmup)
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        ms = dt * 1e3 / args.steps
        value = kv_bytes / (dt / args.steps) / 1e9
        # per-kernel durations (events around each launch, on the launch stream)
        tpa.profile_begin(2 * args.steps + 8)
        for i in range(args.steps):
            step(i)
        prof = tpa.profile_end()
        fwd_ms = prof["fwd_ms"] / max(1, prof["fwd_launches"])
        comb_ms = prof["combine_ms"] / max(1, prof["combine_launches"])
        achieved = (kv_bytes + q_bytes) / (fwd_ms * 1e-3) / 1e9
        traffic = traffic_for(DECODE_KERNEL, w.name)
        # distribution of single steps, each bracketed by events on the launch stream
        stream = torch.cuda.current_stream()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(100)]
        for i, (e0, e1) in enumerate(evs):
            e0.record(stream)
            step(i)
            e1.record(stream)
        torch.cuda.synchronize()
        us = sorted(1e3 * e0.elapsed_time(e1) for e0, e1 in evs)
        pct = {"p10": round(us[10], 2), "p50": round(us[50], 2), "p90": round(us[90], 2)}
        out["decode"] = dict(value=value, ms_per_step=ms, fwd_ms=fwd_ms, combine_ms=comb_ms,
                             achieved=achieved, traffic=traffic, n_rot=n_rot, step_us=pct)
        del ks, vs, q, k, v
        # the reference: a plain streaming read of the same bytes (one launch of 512
        # workgroups with the decode kernel's 16-byte non-temporal loads), rotated
        # over as many buffers and timed the same way as the decode steps
        bufs = [torch.empty(kv_bytes, dtype=torch.uint8, device=dev) for _ in range(n_rot)]
        sink = torch.zeros(512, dtype=torch.int32, device=dev)

        def sstep(i):
            tpa.stream_read(bufs[i % n_rot], sink, 512)

        warm(sstep, args.warmup)
        t0 = time.perf_counter()
        for i in range(args.steps):
            sstep(i)
        torch.cuda.synchronize()
        sdt = (time.perf_counter() - t0) / args.steps
        out["stream"] = dict(GBps=kv_bytes / sdt / 1e9, us=sdt * 1e6)
        del bufs

    # ----------------------------------------------------------------- prefill
    wp = WORKLOADS["causal_prefill_bf16"]
    pairs = wp.B * wp.Hq * sum(min(i + 1 + wp.Sk - wp.Sq, wp.Sk) for i in range(wp.Sq))
    flops = 4.0 * wp.d * pairs
    if not args.no_prefill and args.only in (None, "prefill"):
        q, k, v, _ = make_inputs(wp, seed=0, device=dev)
        o = torch.empty_like(q)
        lse = torch.empty((wp.B, wp.Hq, wp.Sq), dtype=torch.float32, device=dev)

        def pstep(i=0):
            tpa.fwd(q, k, v, causal=True, out=o, lse=lse)

        warm(pstep, args.warmup)
        t0 = time.perf_counter()
        for _ in range(args.prefill_steps):
            pstep()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        pms = dt * 1e3 / args.prefill_steps
        tpa.profile_begin(args.prefill_steps + 4)
        for _ in range(args.prefill_steps):
            pstep()
        prof = tpa.profile_end()
        pf_ms = prof["fwd_ms"] / max(1, prof["fwd_launches"])
        out["prefill"] = dict(value=flops / (pms * 1e-3) / 1e12, ms_per_step=pms, fwd_ms=pf_ms,
                              achieved=flops / (pf_ms * 1e-3) / 1e12)
        del q, k, v

    # ---------------------------------------------------------------- backward
    from workloads import BWD_WORKLOADS, output_grad
    wb = BWD_WORKLOADS["causal_prefill_bwd_bf16"]
    bflops = 10.0 * wb.d * pairs  # five products of 2 d flops per visible pair
    if not args.no_backward and args.only in (None, "backward"):
        q, k, v, _ = make_inputs(wb, seed=0, device=dev)
        g = output_grad(0, q.shape, wb.dtype, device=dev)
        o, lse = tpa.fwd(q, k, v, causal=True)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

        def bstep(i=0):
            tpa.bwd(q, k, v, o, g, lse, causal=True, dq=dq, dk=dk, dv=dv)

        warm(bstep, 3)
        nb = max(5, args.prefill_steps)
        t0 = time.perf_counter()
        for _ in range(nb):
            bstep()
        torch.cuda.synchronize()
        bms = (time.perf_counter() - t0) * 1e3 / nb
        tpa.profile_begin(4 * nb + 8)
        for _ in range(nb):
            bstep()
        prof = tpa.profile_end_kinds()
        n = max(1, prof["bwd_launches"])
        kv_ms, dq_ms = prof["bwd_ms"] / n, prof["bwd_dq_ms"] / n
        out["backward"] = dict(value=bflops / (bms * 1e-3) / 1e12, ms_per_step=bms, dkdv_ms=kv_ms,
                               dq_ms=dq_ms, pre_ms=prof["bwd_prepost_ms"] / n,
                               achieved=bflops / ((kv_ms + dq_ms) * 1e-3) / 1e12)
        del q, k, v, g, o, dq, dk, dv

    # ------------------------------------------------------------ cpu baseline
    cpu = None
    if not args.no_cpu_baseline and args.only is None:
        import oracle
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
        q, k, v, _ = make_inputs(w, seed=0)
        oracle.attn_ref(q, k, v, False, -1, w.scale, n_threads=threads)  # warm (build, pages)
        runs, t0 = 0, time.perf_counter()
        while True:
            oracle.attn_ref(q, k, v, False, -1, w.scale, n_threads=threads)
            runs += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        cpu = {"value": kv_bytes * runs / dt / 1e9, "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"the whole decode workload (all 32 query heads, 32768 keys), "
                         f"{runs} oracle runs in {dt:.1f} s, fp64"}
        # prefill: 16 query rows spread over the sequence, all heads, oracle fp64
        qp, kp, vp, _ = make_inputs(wp, seed=0)
        rows = [int(x) for x in torch.linspace(0, wp.Sq - 1, 16).round()]
        t0 = time.perf_counter()
        pf = 0.0
        for i in rows:
            kl = i + 1
            oracle.attn_ref(qp[:, i:i + 1], kp[:, :kl], vp[:, :kl], True, -1, wp.scale,
                            n_threads=threads)
            pf += 4.0 * wp.d * kl * wp.Hq
        dtp = time.perf_counter() - t0
        cpu["prefill"] = {"value": pf / dtp / 1e12, "unit": "TFLOP/s",
                          "sample": f"{len(rows)} causal query rows x 32 heads, {dtp:.1f} s"}
        if not args.no_backward:
            # backward: the whole gradient of one of the 32 heads (full 8192 rows)
            from workloads import output_grad
            gp = output_grad(0, qp.shape, wp.dtype)
            t0 = time.perf_counter()
            oracle.attn_bwd_ref(qp[:, :, :1], kp[:, :, :1], vp[:, :, :1], gp[:, :, :1], True, -1,
                                wp.scale, n_threads=threads)
            dtb = time.perf_counter() - t0
            cpu["backward"] = {"value": 10.0 * wp.d * (pairs / wp.Hq) / dtb / 1e12, "unit": "TFLOP/s",
                               "sample": f"the backward of 1 of the 32 heads (8192 causal rows), {dtb:.1f} s"}
        try:
            model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo")
                         if l.startswith("model name"))
        except (OSError, StopIteration):
            model = "unknown"
        cpu["cpu_model"] = model

    dec = out.get("decode")
    pre = out.get("prefill")
    line = {
        "metric": "decode KV GB/s (% of HBM peak); causal prefill TFLOP/s (% MFMA peak), 1 GPU",
        "value": round(dec["value"], 2) if dec else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5) if dec else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) tensors; KV rotated over copies to defeat the LLC)",
        "config": {"workload": "gqa_decode_bf16: B=1 Hq=32 Hkv=4 Sq=1 Sk=32768 d=128, "
                               "non-causal, split-KV + LSE combine",
                   "num_splits": plan["num_splits"], "pack_gqa": plan["pack_gqa"],
                   "grid": [plan["grid_x"], plan["grid_y"], plan["grid_z"]],
                   "kv_copies": dec["n_rot"] if dec else None},
    }
    if dec:
        line["pct_of_hbm_peak"] = round(100 * dec["value"] / HBM_PEAK_GBS, 2)
        line["roofline"] = {"bound": "hbm", "kernel": DECODE_KERNEL + "<128, 4, false>",
                            "achieved": round(dec["achieved"], 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(dec["achieved"] / HBM_PEAK_GBS, 4),
                            "traffic": dec["traffic"],
                            "avg_launch_ms": round(dec["fwd_ms"], 5),
                            "combine_avg_launch_ms": round(dec["combine_ms"], 5)}
        kt = kernel_time_for(DECODE_KERNEL, w.name)
        if kt:  # the same fraction from the committed rocprofv3 kernel trace
            line["roofline"]["rocprof_median_us"] = kt["median_us"]
            line["roofline"]["frac_rocprof"] = round(
                (kv_bytes + q_bytes) / (kt["median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        line["step_us"] = dec["step_us"]
        st = out.get("stream")
        if st:
            line["stream_read"] = {"GBps": round(st["GBps"], 1), "us_per_read": round(st["us"], 2),
                                   "pct_of_hbm_peak": round(100 * st["GBps"] / HBM_PEAK_GBS, 2),
                                   "decode_step_vs_stream_read": round(dec["value"] / st["GBps"], 4)}
    if pre:
        line["prefill"] = {
            "metric": "causal prefill TFLOP/s", "value": round(pre["value"], 2),
            "unit": "TFLOP/s", "ms_per_step": round(pre["ms_per_step"], 4),
            "pct_of_mfma_peak": round(100 * pre["value"] / BF16_PEAK_TFLOPS, 2),
            "config": {"workload": "causal_prefill_bf16: B=1 H=32 S=8192 d=128, causal, "
                                   "visible pairs only", "flops_per_step": flops},
            "roofline": {"bound": "mfma", "kernel": "attn_prefill_kernel<128, 8, 32, 0, 0>",
                         "achieved": round(pre["achieved"], 2),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(pre["achieved"] / BF16_PEAK_TFLOPS, 4),
                         "traffic": traffic_for("attn_prefill_kernel", wp.name),
                         "avg_launch_ms": round(pre["fwd_ms"], 4)},
        }
        kt = kernel_time_for("attn_prefill_kernel", wp.name)
        if kt:
            line["prefill"]["roofline"]["rocprof_median_us"] = kt["median_us"]
            line["prefill"]["roofline"]["frac_rocprof"] = round(
                flops / (kt["median_us"] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)
    bwd = out.get("backward")
    if bwd:
        # counter bytes of the two matrix kernels together, when both are recorded
        t_kv = traffic_for("attn_bwd_dkdv_dma_kernel", wb.name)
        t_dq = traffic_for("attn_bwd_dq_dma_kernel", wb.name)
        bwd_traffic = t_kv + t_dq if t_kv is not None and t_dq is not None else None
        line["backward"] = {
            "metric": "causal backward TFLOP/s", "value": round(bwd["value"], 2),
            "unit": "TFLOP/s", "ms_per_step": round(bwd["ms_per_step"], 4),
            "pct_of_mfma_peak": round(100 * bwd["value"] / BF16_PEAK_TFLOPS, 2),
            "config": {"workload": "causal_prefill_bwd_bf16: B=1 H=32 S=8192 d=128, causal, "
                                   "dq/dk/dv, 10 d flops per visible pair", "flops_per_step": bflops},
            "roofline": {"bound": "mfma",
                         "kernel": "attn_bwd_dkdv_dma_kernel<128, 16, 2> + attn_bwd_dq_dma_kernel<128, 2, 2>",
                         "achieved": round(bwd["achieved"], 2), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(bwd["achieved"] / BF16_PEAK_TFLOPS, 4),
                         "traffic": bwd_traffic,
                         "avg_launch_ms": {"dkdv": round(bwd["dkdv_ms"], 4), "dq": round(bwd["dq_ms"], 4),
                                           "row_sums": round(bwd["pre_ms"], 4)}},
        }
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
