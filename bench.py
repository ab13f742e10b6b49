"""Benchmark of the canvas denoising attention hot path on one MI355X.

One step = one block cycle of the L=8192 workload: 12 canvas denoising steps
(dg_canvas_step_loop, fresh seeded Q/K/V per step, fixed cache) followed by the
causal commit of the block with its cache append (dg_commit_block), batch 1,
Hq=16, Hkv=8, head_dim=128, bf16 storage with fp32 accumulation.

Prints one JSON line.  value = algorithmic TFLOP/s of the whole cycle
(canvas step 4*B*Hq*256*(L+256)*D, commit 4*B*Hq*D*(256*L + 256*257/2), exp
and max not counted).  The roofline object is for the dominant kernel (the
split-key canvas attention kernel), timed with HIP events that the library
records on its launch stream.  cpu_baseline times the CPU fp64 oracle on a
bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "canvas-step attn TFLOP/s + canvas positions/s at L=8k, bs=1; % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


# HBM traffic of the dominant kernel comes from rocprofv3 counter runs
# (FETCH_SIZE and WRITE_SIZE per dispatch, calibrated against a plain copy of
# known size) recorded in this file together with a hash of the kernel source;
# it is reported only while the source still matches.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "canvas_attn_l8k_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "canvas_attention_amd", "csrc", f)
                  for f in ("dg_attn_mfma.hip", "dg_internal.h")]


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """Bytes per launch of the canvas attention kernel from the counter file, or
    None when the file is absent or was taken on another version of the kernel."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    try:
        if kv["kernel_source_hash"] != kernel_source_hash():
            return None
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def copy_probe(mib):
    """A plain device-to-device copy of known size (the counter calibration run)."""
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)


def _counter_per_dispatch(folder, counter, name_part):
    """Mean value of one counter over the dispatches of kernels whose name holds
    name_part, from a rocprofv3 --pmc csv folder."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                    vals[(f, r["Dispatch_Id"])] = vals.get((f, r["Dispatch_Id"]), 0.0) + \
                        float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for '{name_part}' under {folder}")
    return sum(vals.values()) / len(vals), len(vals)


ATTN_KERNEL = "attn_bf16_kernel<128, false"


def summarize_counters(fetch_dir, write_dir, cfetch_dir, cwrite_dir, copy_mib):
    copy_bytes = int(copy_mib) * (1 << 20)
    f_kib, nf = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", ATTN_KERNEL)
    w_kib, nw = _counter_per_dispatch(write_dir, "WRITE_SIZE", ATTN_KERNEL)
    cf_kib, _ = _counter_per_dispatch(cfetch_dir, "FETCH_SIZE", "copyBuffer")
    cw_kib, _ = _counter_per_dispatch(cwrite_dir, "WRITE_SIZE", "copyBuffer")
    f_scale = copy_bytes / (cf_kib * 1024.0)
    w_scale = copy_bytes / (cw_kib * 1024.0)
    fetch = f_kib * 1024.0 * f_scale
    write = w_kib * 1024.0 * w_scale
    lines = [
        "# HBM traffic of the canvas attention kernel (canvas step, L=8192, B=1, Hq=16, Hkv=8, D=128)",
        "# from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE runs of",
        "#   python3 bench.py --steps 2 --warmup 1 --profile-steps",
        "# calibrated with the same counters on a plain device-to-device copy of known size",
        f"#   python3 bench.py --copy-probe {copy_mib}",
        "# (each scale = copy bytes / counter bytes of that copy); written by",
        "#   python3 bench.py --summarize-counters FETCH WRITE COPY_FETCH COPY_WRITE MIB",
        f"kernel: {ATTN_KERNEL}...>",
        f"kernel_source_hash: {kernel_source_hash()}",
        f"dispatches_fetch: {nf}",
        f"dispatches_write: {nw}",
        f"fetch_kib_per_dispatch: {f_kib:.1f}",
        f"write_kib_per_dispatch: {w_kib:.1f}",
        f"copy_bytes: {copy_bytes}",
        f"copy_fetch_kib: {cf_kib:.1f}",
        f"copy_write_kib: {cw_kib:.1f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        f"fetch_bytes_per_launch: {fetch:.0f}",
        f"write_bytes_per_launch: {write:.0f}",
        f"traffic_bytes_per_launch: {fetch + write:.0f}",
    ]
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_mfma(pass1_dir, pass2_dir, trace_txt):
    """MFMA work of the canvas attention kernel from two rocprofv3 --pmc runs of
    `bench.py --steps 2 --warmup 1 --profile-steps` (SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_INSTS_MFMA; SQ_INSTS_VALU_MFMA_MOPS_BF16), set against the kernel's average
    duration from the kernel-trace summary.  Writes profiles/canvas_attn_l8k_mfma.txt."""
    import csv
    import collections

    def per_dispatch(d):
        vals = collections.defaultdict(lambda: collections.defaultdict(float))
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            if ATTN_KERNEL in r["Kernel_Name"]:
                vals[r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
        return {c: (sum(v.values()) / len(v), len(v)) for c, v in vals.items()}

    c = {**per_dispatch(pass1_dir), **per_dispatch(pass2_dir)}
    avg_us = None
    for line in open(trace_txt):
        if ATTN_KERNEL in line:
            avg_us = float(line.split()[1])
    busy = c["SQ_VALU_MFMA_BUSY_CYCLES"][0] / 1024.0  # per SIMD (256 CUs x 4)
    mops = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"][0]
    out = os.path.join(ROOT, "profiles", "canvas_attn_l8k_mfma.txt")
    with open(out, "w") as f:
        f.write("# MFMA work of the canvas attention kernel (canvas step, L=8192, B=1, Hq=16, Hkv=8, D=128)\n")
        f.write("# from rocprofv3 --pmc runs (each in its own process) of\n")
        f.write("#   python3 bench.py --steps 2 --warmup 1 --profile-steps\n")
        f.write("#   pass 1: SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_MFMA\n")
        f.write("#   pass 2: SQ_INSTS_VALU_MFMA_MOPS_BF16\n")
        f.write("# per-dispatch means over the dispatches of the kernel; written by\n")
        f.write("#   python3 bench.py --summarize-mfma PASS1 PASS2 profiles/canvas_attn_l8k_kernel_trace.txt\n")
        f.write(f"kernel: {ATTN_KERNEL}...>\n")
        f.write(f"kernel_source_hash: {kernel_source_hash()}\n")
        f.write(f"dispatches: {c['SQ_INSTS_MFMA'][1]}\n")
        f.write(f"mfma_instructions: {c['SQ_INSTS_MFMA'][0]:.0f}\n")
        f.write(f"mfma_flop (MOPS_BF16 x 512): {mops * 512:.4e}\n")
        f.write(f"algorithmic_flop: {step_flops(1, 16, 8192, 128):.4e}\n")
        f.write(f"mfma_busy_cycles_per_simd: {busy:.0f}\n")
        if avg_us:
            f.write(f"kernel_avg_us (kernel trace): {avg_us}\n")
            f.write(f"mfma_busy_frac_at_2.4GHz: {busy / (avg_us * 1e-6 * 2.4e9):.4f}\n")
    print(open(out).read())


def summarize_trace(stats_csv, out_txt):
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    keep = [r for r in rows if "dg::" in r["Name"] or "copyBuffer" in r["Name"]]
    lines = ["# rocprofv3 --kernel-trace --stats summary (kernels of this library)",
             "# command: cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv "
             "-d <dir> -o run -- python3 <repo>/bench.py --steps 10 --warmup 2 --no-cpu-baseline",
             f"{'calls':>7} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_pct':>9}  kernel"]
    for r in keep:
        lines.append(f"{int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.3f} "
                     f"{float(r['MinNs']) / 1e3:10.3f} {float(r['MaxNs']) / 1e3:10.3f} "
                     f"{float(r['Percentage']):9.2f}  {r['Name'][:110]}")
    with open(out_txt, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def step_flops(B, Hq, L, D, Nc=256):
    return 4.0 * B * Hq * Nc * (L + Nc) * D


def commit_flops(B, Hq, L, D, Nc=256):
    return 4.0 * B * Hq * D * (Nc * L + Nc * (Nc + 1) / 2)


def step_bytes(B, Hq, Hkv, L, D, Nc=256):
    # cache K and V once, canvas Q/K/V, output
    return 2.0 * B * (2 * L * Hkv * D + Nc * Hq * D + 2 * Nc * Hkv * D + Nc * Hq * D)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--profile-steps", action="store_true",
                    help="only run the timed cycles (for rocprofv3 runs)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device to device 5 times (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=5, metavar=("FETCH", "WRITE", "COPY_FETCH",
                                                              "COPY_WRITE", "COPY_MIB"),
                    help="write the traffic file from four rocprofv3 --pmc output folders")
    ap.add_argument("--summarize-mfma", nargs=3, metavar=("PASS1", "PASS2", "TRACE_TXT"),
                    help="write profiles/canvas_attn_l8k_mfma.txt from two rocprofv3 --pmc runs")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("STATS_CSV", "OUT_TXT"),
                    help="write a kernel summary from a rocprofv3 --stats kernel_stats.csv")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the canvas "
              "attention path has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    import canvas_attention_amd.dg as dg
    from canvas_attention_amd import synth

    torch.cuda.set_device(0)
    name = "cycle_l8k"
    w = synth.WORKLOADS[name]
    B, Hq, Hkv, D, seed = w["batch"], w["hq"], w["hkv"], w["d"], w["seed"]
    n_steps = w["steps"]
    L = synth.prefix_lengths(name)
    Lv = int(L[0])
    cap = Lv + 256

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    kc, vc = synth.cache(seed, L, cap, Hkv, D, "bf16")
    kc_d, vc_d = dev(kc), dev(vc)
    canv = [synth.canvas(seed, B, Hq, Hkv, D, "bf16", step=s) for s in range(n_steps)]
    qs = torch.stack([dev(c[0]) for c in canv])
    ks = torch.stack([dev(c[1]) for c in canv])
    vs = torch.stack([dev(c[2]) for c in canv])
    qb, kb, vb = (dev(x) for x in synth.block(seed, B, Hq, Hkv, D, "bf16"))
    out_steps = torch.empty_like(qs)
    out_blk = torch.empty_like(qb)
    ws = dg.alloc_workspace(qs[0], Hkv, cap)
    stream = torch.cuda.current_stream()

    def cycle():
        dg.canvas_step_loop(qs, ks, vs, kc_d, vc_d, L, out=out_steps, workspace=ws)
        dg.commit_block(qb, kb, vb, kc_d, vc_d, L, out=out_blk, workspace=ws)

    for _ in range(args.warmup):
        cycle()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        cycle()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    if args.profile_steps:
        print(json.dumps({"ms_per_step": ms}), flush=True)
        return

    fl_step = step_flops(B, Hq, Lv, D)
    fl_commit = commit_flops(B, Hq, Lv, D)
    fl_cycle = n_steps * fl_step + fl_commit
    value = fl_cycle / (ms * 1e-3) / 1e12

    # per-kernel durations: a second pass over the same canvas steps with the
    # library's HIP events around every launch (same stream as the launches)
    dg.kernel_timing_read()
    dg.kernel_timing_enable(True)
    for _ in range(args.steps):
        dg.canvas_step_loop(qs, ks, vs, kc_d, vc_d, L, out=out_steps, workspace=ws)
    n_attn, attn_ms, n_merge, merge_ms = dg.kernel_timing_read()
    for _ in range(args.steps):
        dg.commit_block(qb, kb, vb, kc_d, vc_d, L, out=out_blk, workspace=ws)
    n_cattn, cattn_ms, n_cmerge, cmerge_ms = dg.kernel_timing_read()
    dg.kernel_timing_enable(False)
    attn_us = attn_ms / max(n_attn, 1) * 1e3
    merge_us = merge_ms / max(n_merge, 1) * 1e3 if n_merge else 0.0
    achieved = fl_step / (attn_us * 1e-6) / 1e12

    # canvas steps alone (whole step incl. merge), for positions/s
    t0.record(stream)
    for _ in range(args.steps):
        dg.canvas_step_loop(qs, ks, vs, kc_d, vc_d, L, out=out_steps, workspace=ws)
    t1.record(stream)
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / (args.steps * n_steps)

    # per-launch kernel durations (the library's events around each launch), median
    # over calls of one canvas step (attention + merge): warm (the fixed cache stays
    # in the 256 MB last-level cache, as in a block's step loop) and cold (a 512 MB
    # scratch fill before every call, outside the timed kernels)
    reps = max(args.steps, 50)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")

    def one_step(i):
        s = i % n_steps
        dg.canvas_attn(qs[s], kc_d, vc_d, L, ks[s], vs[s], out=out_steps[s], workspace=ws)

    medians = {}
    for mode in ("warm", "cold"):
        dg.kernel_timing_read()
        dg.kernel_timing_enable(True)
        for i in range(reps):
            if mode == "cold":
                flush.fill_(i & 255)
            one_step(i)
        a_ms, m_ms = dg.kernel_timing_samples(reps)
        dg.kernel_timing_enable(False)
        m_ms = m_ms if len(m_ms) == len(a_ms) else [0.0] * len(a_ms)
        medians[mode] = {"attn": round(float(np.median(a_ms)) * 1e3, 3),
                         "step": round(float(np.median(np.add(a_ms, m_ms))) * 1e3, 3)}
    del flush

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "block cycle: 12 canvas steps + commit at prefix L=8192",
                   "batch": B, "prefix_len": Lv, "n_canvas": 256, "n_heads_q": Hq,
                   "n_heads_kv": Hkv, "head_dim": D, "steps_per_block": n_steps},
        "canvas_step_us": round(step_ms * 1e3, 3),
        "canvas_step_tflops": round(fl_step / (step_ms * 1e-3) / 1e12, 2),
        "canvas_positions_per_s": round(B * 256 / (step_ms * 1e-3), 1),
        "canvas_step_mfma_frac": round(fl_step / (step_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "canvas_call_us_median": {"warm": medians["warm"], "cold": medians["cold"],
                                  "calls": reps},
        "kernels_us": {"canvas_attn": round(attn_us, 3), "canvas_merge": round(merge_us, 3),
                       "commit_attn": round(cattn_ms / max(n_cattn, 1) * 1e3, 3),
                       "commit_merge": round(cmerge_ms / max(n_cmerge, 1) * 1e3, 3)
                       if n_cmerge else 0.0},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "attn_bf16_kernel<128,false> (canvas step, L=8192)",
                     "algorithmic_flop_per_launch": fl_step,
                     "hbm_frac": round(step_bytes(B, Hq, Hkv, Lv, D) / (attn_us * 1e-6) / 1e9
                                       / PEAK_HBM_GBS, 4)},
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(name, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline(name, budget_s):
    """The CPU fp64 oracle on a bounded sample of the same workload: whole canvas
    steps of the block cycle (each with its own seeded canvas Q/K/V, all 256
    positions and all heads), one after another until the time budget is spent."""
    import oracle
    from canvas_attention_amd import synth
    w = synth.WORKLOADS[name]
    B, Hq, Hkv, D, seed = w["batch"], w["hq"], w["hkv"], w["d"], w["seed"]
    L = synth.prefix_lengths(name)
    Lv = int(L[0])
    kc, vc = synth.cache(seed, L, Lv + 256, Hkv, D, "bf16")
    steps = [synth.canvas(seed, B, Hq, Hkv, D, "bf16", step=s) for s in range(w["steps"])]
    done = 0
    t_start = time.perf_counter()
    elapsed = 0.0
    while elapsed < budget_s:
        q, kn, vn = steps[done % len(steps)]
        oracle.canvas_attn(q, kc, vc, L, kn, vn)
        done += 1
        elapsed = time.perf_counter() - t_start
    flops = done * step_flops(B, Hq, Lv, D)
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{done} whole canvas steps of the L={Lv} block cycle (B={B}, 256 "
                      f"positions, Hq={Hq}, Hkv={Hkv}, D={D}) in {elapsed:.1f} s: "
                      f"{done * B * 256 / elapsed:.1f} canvas positions/s"}


if __name__ == "__main__":
    main()
