"""Benchmark of the canvas denoising attention hot path on one MI355X.

One step = one block cycle of the L=8192 workload: 12 canvas denoising steps
(dg_canvas_step_loop, fresh seeded Q/K/V per step, fixed cache) followed by the
causal commit of the block with its cache append (dg_commit_block), batch 1,
Hq=16, Hkv=8, head_dim=128, bf16 storage with fp32 accumulation (--dtype fp8:
OCP e4m3 storage with tensor scales 1, fp32 accumulation, bf16 output).

Prints one JSON line.  value = algorithmic TFLOP/s of the canvas step (the
metric's quantity: 4*B*Hq*256*(L+256)*D per step, exp and max not counted),
taken from the timed block cycles themselves: an event pair brackets the 12
steps of every cycle, so the step time holds attention and merge.  Beside it:
canvas positions per second, the fraction of the bf16 MFMA peak, and the whole
cycle's TFLOP/s (commit: 4*B*Hq*D*(256*L + 256*257/2)).  ms_per_step is the
block cycle.  The roofline object is for the dominant kernel (the split-key
canvas attention kernel), timed with HIP events that the library's launches
record with their own dispatch, on the launch stream.  cpu_baseline times the CPU fp64 oracle on bounded samples
of the L=2048, L=8192 and L=131072 canvas steps, on all host threads and on
one.  The default (bf16) line also carries the
fp8 canvas step's kernel time and its fraction of the fp8 MFMA peak, the
canvas sampler's time per call over one step's logits (--sampler: only that),
decode attention (AR mode, 1 or 16 new tokens over the same cache) on four
workloads with its own HBM roofline object (--decode [WORKLOAD]: only that), and
the self-conditioning input z = FFW(softmax(logits) E) of one canvas with the
roofline of its embedding product (--selfcond: only that).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--dtype fp8]
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
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}  # MI355X dense MFMA
PEAK_BF16_TFLOPS = PEAK_TFLOPS["bf16"]
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
ELEM_BYTES = {"bf16": 2, "fp8": 1}

# the canvas attention kernel of each format, as rocprofv3 names it, and the
# profile files of its counter summaries
ATTN_KERNELS = {"bf16": "attn_bf16_kernel<128, false", "fp8": "attn_fp8_kernel<128, false",
                "sampler": "row_stats_kernel", "decode": "decode_kernel<dg::(anonymous namespace)::FmtBf16, 128",
                "selfcond": "gemm_kernel<256>", "long": "attn_bf16_kernel<128, false"}
PROFILE_TAG = {"bf16": "canvas_attn_l8k", "fp8": "canvas_attn_fp8_l8k", "sampler": "canvas_sample_v262k",
               "decode": "decode_attn_b32_l8k", "selfcond": "selfcond_v262k_d2048",
               "long": "canvas_attn_l128k"}
PROFILE_WHAT = {"bf16": "the canvas attention kernel (bf16; canvas step, L=8192, B=1, Hq=16, Hkv=8, D=128)",
                "fp8": "the canvas attention kernel (fp8; canvas step, L=8192, B=1, Hq=16, Hkv=8, D=128)",
                "sampler": "the sampler's row statistics kernel (B=1, 256 positions, V=262144 bf16 logits)",
                "decode": "the decode attention kernel (bf16; 32 sequences at L=8192, one new token each, "
                          "Hq=16, Hkv=8, D=128)",
                "selfcond": "the self-conditioning embedding product (256 x 262144 softmax weights times "
                            "E [262144 x 2048], bf16)",
                "long": "the canvas attention kernel (bf16; canvas step, L=131072, B=1, Hq=16, Hkv=8, D=128)"}
PROFILE_RUN = {"bf16": "--steps 2 --warmup 1 --profile-steps", "fp8": "--steps 2 --warmup 1 --profile-steps --dtype fp8",
               "sampler": "--sampler --steps 10", "decode": "--decode b32_l8k_k1 --steps 10",
               "selfcond": "--selfcond --steps 10", "long": "--long-context --steps 5"}

# Decode attention workloads (AR mode over the same cache; the concurrency
# crossover of the pages sits near 32 sequences): Hq=16, Hkv=8, D=128, bf16.
DECODE_WORKLOADS = {
    "b1_l8k_k1": dict(batch=1, prefix=8192, k=1),
    "b32_l8k_k1": dict(batch=32, prefix=8192, k=1),
    "b1_l128k_k1": dict(batch=1, prefix=131072, k=1),
    "b1_l8k_k16": dict(batch=1, prefix=8192, k=16),
}
DECODE_ROOFLINE = "b32_l8k_k1"  # the decode shape whose kernel the roofline object describes
MOPS_COUNTER = {"bf16": "SQ_INSTS_VALU_MFMA_MOPS_BF16", "fp8": "SQ_INSTS_VALU_MFMA_MOPS_F8"}


def traffic_file(dtype):
    return os.path.join(ROOT, "profiles", PROFILE_TAG[dtype] + "_traffic.txt")


# HBM traffic of the dominant kernel comes from rocprofv3 counter runs
# (FETCH_SIZE and WRITE_SIZE per dispatch, calibrated against a plain copy of
# known size) recorded in a profile file together with a hash of the kernel
# source; it is reported only while the source still matches.
# The attention kernels' counted traffic also depends on the split plan (dg_plan.cpp
# sets how many partial rows a launch writes) and on the merge that reads them.
KERNEL_SOURCES = [os.path.join(ROOT, "canvas_attention_amd", "csrc", f)
                  for f in ("dg_attn_mfma.hip", "dg_internal.h", "dg_plan.h", "dg_plan.cpp",
                            "dg_merge.hip")]
SAMPLER_SOURCES = [os.path.join(ROOT, "canvas_attention_amd", "csrc", f)
                   for f in ("dg_sample.hip", "dg_internal.h", "dg_plan.h")]
SELFCOND_SOURCES = [os.path.join(ROOT, "canvas_attention_amd", "csrc", f)
                    for f in ("dg_selfcond.hip", "dg_internal.h", "dg_plan.h")]
# the decode kernel shares its source file with the canvas kernels


def kernel_source_hash(dtype="bf16"):
    h = hashlib.sha256()
    srcs = {"sampler": SAMPLER_SOURCES, "selfcond": SELFCOND_SOURCES}.get(dtype, KERNEL_SOURCES)
    for f in srcs:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(dtype="bf16"):
    """Bytes per launch of the kernel behind `dtype` (bf16, fp8, sampler, decode)
    from its counter file, or None when the file is absent or was taken on
    another version of the kernel."""
    path = traffic_file(dtype)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    try:
        if kv["kernel_source_hash"] != kernel_source_hash(dtype):
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


def summarize_counters(fetch_dir, write_dir, cfetch_dir, cwrite_dir, copy_mib, dtype="bf16"):
    ATTN_KERNEL = ATTN_KERNELS[dtype]
    flag = {"bf16": "", "fp8": " --dtype fp8", "sampler": " --sampler", "decode": " --decode",
            "selfcond": " --selfcond", "long": " --long-context"}[dtype]
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
        f"# HBM traffic of {PROFILE_WHAT[dtype]}",
        "# from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE runs of",
        f"#   python3 bench.py {PROFILE_RUN[dtype]}",
        "# calibrated with the same counters on a plain device-to-device copy of known size",
        f"#   python3 bench.py --copy-probe {copy_mib}",
        "# (each scale = copy bytes / counter bytes of that copy); written by",
        f"#   python3 bench.py --summarize-counters FETCH WRITE COPY_FETCH COPY_WRITE MIB{flag}",
        f"kernel: {ATTN_KERNEL}...>",
        f"kernel_source_hash: {kernel_source_hash(dtype)}",
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
    os.makedirs(os.path.dirname(traffic_file(dtype)), exist_ok=True)
    with open(traffic_file(dtype), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_mfma(pass1_dir, pass2_dir, trace_txt, dtype="bf16"):
    """MFMA work of the canvas attention kernel from two rocprofv3 --pmc runs of
    `bench.py --steps 2 --warmup 1 --profile-steps` (SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_INSTS_MFMA; SQ_INSTS_VALU_MFMA_MOPS_BF16 or _F8), set against the kernel's
    average duration from the kernel-trace summary.  Writes
    profiles/<tag>_mfma.txt."""
    import csv
    import collections
    ATTN_KERNEL = ATTN_KERNELS[dtype]
    flag = "" if dtype == "bf16" else f" --dtype {dtype}"

    def per_dispatch(d):
        vals = collections.defaultdict(lambda: collections.defaultdict(float))
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            if ATTN_KERNEL in r["Kernel_Name"]:
                vals[r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
        return {c: (sum(v.values()) / len(v), len(v)) for c, v in vals.items()}

    c = {**per_dispatch(pass1_dir), **per_dispatch(pass2_dir)}
    avg_us = None
    for line in open(trace_txt):
        if ATTN_KERNEL in line and "L=131072 leg" not in line and not line.startswith("#"):
            avg_us = float(line.split()[1])  # the L=8192 leg line, when present, comes last
    busy = c["SQ_VALU_MFMA_BUSY_CYCLES"][0] / 1024.0  # per SIMD (256 CUs x 4)
    mops = c[MOPS_COUNTER[dtype]][0]
    tag = PROFILE_TAG[dtype]
    out = os.path.join(ROOT, "profiles", f"{tag}_mfma.txt")
    with open(out, "w") as f:
        f.write(f"# MFMA work of the canvas attention kernel ({dtype}; canvas step, L=8192, B=1, Hq=16, "
                "Hkv=8, D=128)\n")
        f.write("# from rocprofv3 --pmc runs (each in its own process) of\n")
        f.write(f"#   python3 bench.py --steps 2 --warmup 1 --profile-steps{flag}\n")
        f.write("#   pass 1: SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_MFMA\n")
        f.write(f"#   pass 2: {MOPS_COUNTER[dtype]}\n")
        f.write("# per-dispatch means over the dispatches of the kernel; written by\n")
        f.write(f"#   python3 bench.py --summarize-mfma PASS1 PASS2 profiles/{tag}_kernel_trace.txt{flag}\n")
        f.write(f"kernel: {ATTN_KERNEL}...>\n")
        f.write(f"kernel_source_hash: {kernel_source_hash()}\n")
        f.write(f"dispatches: {c['SQ_INSTS_MFMA'][1]}\n")
        f.write(f"mfma_instructions: {c['SQ_INSTS_MFMA'][0]:.0f}\n")
        f.write(f"mfma_flop ({MOPS_COUNTER[dtype][19:]} x 512): {mops * 512:.4e}\n")
        f.write(f"algorithmic_flop: {step_flops(1, 16, 8192, 128):.4e}\n")
        f.write(f"mfma_flop / algorithmic_flop: {mops * 512 / step_flops(1, 16, 8192, 128):.4f}"
                + (" (the fp8 kernel adds one row-sum MFMA per 8 score and value MFMAs)\n"
                   if dtype == "fp8" else "\n"))
        f.write(f"mfma_busy_cycles_per_simd: {busy:.0f}\n")
        if avg_us:
            f.write(f"kernel_avg_us (kernel trace): {avg_us}\n")
            f.write(f"mfma_busy_frac_at_2.4GHz: {busy / (avg_us * 1e-6 * 2.4e9):.4f}\n")
    print(open(out).read())


def summarize_trace(stats_csv, out_txt, dtype="bf16", sampler=False, decode=None, selfcond=False,
                    long_context=False):
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    keep = [r for r in rows if "dg::" in r["Name"] or "copyBuffer" in r["Name"]]
    flag = "" if dtype == "bf16" else f" --dtype {dtype}"
    run = "--sampler --steps 50" if sampler else f"--steps 10 --warmup 2 --no-cpu-baseline{flag}"
    if decode:
        run = f"--decode {decode} --steps 20"
        flag = f" --decode {decode}"
    if selfcond:
        run = "--selfcond --steps 20"
        flag = " --selfcond"
    if long_context:
        run = "--long-context --steps 10"
        flag = " --long-context"
    tag = ("sampler" if sampler else "decode" if decode else "selfcond" if selfcond
           else "long" if long_context else dtype)
    lines = ["# rocprofv3 --kernel-trace --stats summary (kernels of this library)",
             f"# kernel_source_hash: {kernel_source_hash(tag)}",
             "# command: cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv "
             f"-d <dir> -o run -- python3 <repo>/bench.py {run}",
             "# (written by: python3 bench.py --summarize-trace <dir>/run_kernel_stats.csv OUT"
             f"{' --sampler' if sampler else flag})",
             f"{'calls':>7} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_pct':>9}  kernel"]
    for r in keep:
        lines.append(f"{int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.3f} "
                     f"{float(r['MinNs']) / 1e3:10.3f} {float(r['MaxNs']) / 1e3:10.3f} "
                     f"{float(r['Percentage']):9.2f}  {r['Name'][:110]}")
    # The default run times the same canvas kernel at L=8192 and (its long_context
    # object) at L=131072; the per-dispatch trace separates the two legs by launch
    # time (about 20-30 us against 250-370 us).
    trace_csv = os.path.join(os.path.dirname(stats_csv), "run_kernel_trace.csv")
    if tag == "bf16" and os.path.exists(trace_csv):
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                for r in csv.DictReader(open(trace_csv)) if ATTN_KERNELS["bf16"] in r["Kernel_Name"]]
        lines.append("# attn_bf16_kernel<128, false> by leg (per-dispatch trace, split at 100 us):")
        for leg, sel in (("L=8192", [d for d in durs if d < 100.0]),
                         ("L=131072", [d for d in durs if d >= 100.0])):
            if sel:
                lines.append(f"{len(sel):7d} {sum(sel) / len(sel):10.3f} {min(sel):10.3f} "
                             f"{max(sel):10.3f} {'':>9}  attn_bf16_kernel<128, false> {leg} leg")
    with open(out_txt, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def step_flops(B, Hq, L, D, Nc=256):
    return 4.0 * B * Hq * Nc * (L + Nc) * D


def commit_flops(B, Hq, L, D, Nc=256):
    return 4.0 * B * Hq * D * (Nc * L + Nc * (Nc + 1) / 2)


def step_bytes(B, Hq, Hkv, L, D, esz=2, Nc=256):
    # cache K and V once, canvas Q/K/V (esz bytes per element), bf16 output
    return B * (esz * (2 * L * Hkv * D + Nc * Hq * D + 2 * Nc * Hkv * D) + 2.0 * Nc * Hq * D)


def dev(a):
    """numpy -> GPU tensor (uint16 bf16 bits or uint8 e4m3 bytes)."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda().view(torch.float8_e4m3fn)


class Cycle:
    """Device inputs of the L=8192 block cycle in one storage format."""

    def __init__(self, dtype, name="cycle_l8k"):
        import torch
        import canvas_attention_amd.dg as dg
        from canvas_attention_amd import synth
        self.dg, self.dtype = dg, dtype
        w = synth.WORKLOADS[name]
        self.B, self.Hq, self.Hkv, self.D = w["batch"], w["hq"], w["hkv"], w["d"]
        seed, self.n_steps = w["seed"], w["steps"]
        self.L = synth.prefix_lengths(name)
        self.Lv = int(self.L[0])
        cap = self.Lv + 256
        kc, vc = synth.cache(seed, self.L, cap, self.Hkv, self.D, dtype)
        self.kc, self.vc = dev(kc), dev(vc)
        canv = [synth.canvas(seed, self.B, self.Hq, self.Hkv, self.D, dtype, step=s)
                for s in range(self.n_steps)]
        self.qs = dev(np.stack([c[0] for c in canv]))
        self.ks = dev(np.stack([c[1] for c in canv]))
        self.vs = dev(np.stack([c[2] for c in canv]))
        self.qb, self.kb, self.vb = (dev(x) for x in synth.block(seed, self.B, self.Hq, self.Hkv,
                                                                 self.D, dtype))
        self.out_steps = torch.empty(self.qs.shape, dtype=torch.bfloat16, device="cuda")
        self.out_blk = torch.empty(self.qb.shape, dtype=torch.bfloat16, device="cuda")
        self.ws = dg.alloc_workspace(self.qs[0], self.Hkv, cap)

    def steps(self):
        self.dg.canvas_step_loop(self.qs, self.ks, self.vs, self.kc, self.vc, self.L,
                                 out=self.out_steps, workspace=self.ws)

    def commit(self):
        self.dg.commit_block(self.qb, self.kb, self.vb, self.kc, self.vc, self.L,
                             out=self.out_blk, workspace=self.ws)

    def one_step(self, i):
        s = i % self.n_steps
        self.dg.canvas_attn(self.qs[s], self.kc, self.vc, self.L, self.ks[s], self.vs[s],
                            out=self.out_steps[s], workspace=self.ws)


class Flush:
    """Evicts L2 and the 256 MB last-level cache by reading a 512 MB buffer (a
    clean eviction: a write would leave dirty lines whose write-back then runs
    during the timed kernel and takes about a quarter of its read bandwidth)."""

    def __init__(self):
        import torch
        self.buf = torch.ones(128 << 20, dtype=torch.int32, device="cuda")

    def __call__(self):
        self.buf.max()


def call_medians(cy, reps, modes=("warm", "cold")):
    """Per-launch kernel durations (the library's events around each launch),
    median over calls of one canvas step (attention + merge): warm (the fixed
    cache stays in the 256 MB last-level cache, as in a block's step loop) and
    cold (a 512 MB read before every call, outside the timed kernels)."""
    dg = cy.dg
    flush = Flush() if "cold" in modes else None
    medians = {}
    for mode in modes:
        dg.kernel_timing_read()
        dg.kernel_timing_enable(True)
        for i in range(reps):
            if mode == "cold":
                flush()
            cy.one_step(i)
        a_ms, m_ms = dg.kernel_timing_samples(reps)
        dg.kernel_timing_enable(False)
        m_ms = m_ms if len(m_ms) == len(a_ms) else [0.0] * len(a_ms)
        medians[mode] = {"attn": round(float(np.median(a_ms)) * 1e3, 3),
                         "step": round(float(np.median(np.add(a_ms, m_ms))) * 1e3, 3)}
    del flush
    return medians


def measure(dtype, steps, warmup, profile_steps=False):
    """Times the block cycle in one format; returns the bench fields."""
    import torch
    cy = Cycle(dtype)
    dg = cy.dg
    B, Hq, Hkv, D, Lv, n_steps = cy.B, cy.Hq, cy.Hkv, cy.D, cy.Lv, cy.n_steps
    stream = torch.cuda.current_stream()

    def cycle():
        cy.steps()
        cy.commit()

    for _ in range(warmup):
        cycle()
    torch.cuda.synchronize()
    # the timed region: `steps` block cycles back to back; within it one more
    # event after each cycle's 12 canvas steps splits steps from commit
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps + 1)]
    evs[0].record(stream)
    for i in range(steps):
        cy.steps()
        evs[2 * i + 1].record(stream)
        cy.commit()
        evs[2 * i + 2].record(stream)
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / steps
    if profile_steps:
        return {"ms_per_step": ms}
    steps_ms = sum(evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(steps))
    step_ms = steps_ms / (steps * n_steps)

    fl_step = step_flops(B, Hq, Lv, D)
    fl_commit = commit_flops(B, Hq, Lv, D)
    fl_cycle = n_steps * fl_step + fl_commit
    peak = PEAK_TFLOPS[dtype]

    # per-kernel durations: a second pass over the same canvas steps with the
    # library's HIP events, recorded by every launch with its dispatch
    dg.kernel_timing_read()
    dg.kernel_timing_enable(True)
    for _ in range(steps):
        cy.steps()
    n_attn, attn_ms, n_merge, merge_ms = dg.kernel_timing_read()
    for _ in range(steps):
        cy.commit()
    n_cattn, cattn_ms, n_cmerge, cmerge_ms = dg.kernel_timing_read()
    dg.kernel_timing_enable(False)
    attn_us = attn_ms / max(n_attn, 1) * 1e3
    merge_us = merge_ms / max(n_merge, 1) * 1e3 if n_merge else 0.0
    achieved = fl_step / (attn_us * 1e-6) / 1e12

    reps = max(steps, 50)
    medians = call_medians(cy, reps)
    kname = ATTN_KERNELS[dtype].replace(", ", ",")
    return {
        "value": round(fl_step / (step_ms * 1e-3) / 1e12, 2),
        "ms_per_step": round(ms, 5),
        "block_cycle_tflops": round(fl_cycle / (ms * 1e-3) / 1e12, 2),
        "canvas_step_us": round(step_ms * 1e3, 3),
        "canvas_positions_per_s": round(B * 256 / (step_ms * 1e-3), 1),
        "canvas_step_mfma_frac": round(fl_step / (step_ms * 1e-3) / 1e12 / peak, 4),
        "canvas_call_us_median": {"warm": medians["warm"], "cold": medians["cold"],
                                  "calls": reps},
        "kernels_us": {"canvas_attn": round(attn_us, 3), "canvas_merge": round(merge_us, 3),
                       "commit_attn": round(cattn_ms / max(n_cattn, 1) * 1e3, 3),
                       "commit_merge": round(cmerge_ms / max(n_cmerge, 1) * 1e3, 3)
                       if n_cmerge else 0.0},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(dtype),
                     "kernel": f"{kname}> (canvas step, L=8192)",
                     "algorithmic_flop_per_launch": fl_step,
                     "hbm_frac": round(step_bytes(B, Hq, Hkv, Lv, D, ELEM_BYTES[dtype])
                                       / (attn_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
        "_config": {"batch": B, "prefix_len": Lv, "n_canvas": 256, "n_heads_q": Hq,
                    "n_heads_kv": Hkv, "head_dim": D, "steps_per_block": n_steps},
    }


def long_context_summary(reps=20):
    """The canvas step of the long-context workload (B=1, L=131072, Hq=16, Hkv=8,
    D=128, bf16): median per call of the attention kernel (the library's events)
    and of attention + merge, warm, with the kernel's fraction of the bf16 MFMA
    peak -- the same kernel as the headline step, with 16x the keys per unit, so
    its fixed costs weigh less."""
    import torch
    import canvas_attention_amd.dg as dg
    from canvas_attention_amd import synth
    w = synth.WORKLOADS["long_l128k"]
    B, Hq, Hkv, D, seed = w["batch"], w["hq"], w["hkv"], w["d"], w["seed"]
    L = synth.prefix_lengths("long_l128k")
    Lv = int(L[0])
    kc, vc = (dev(x) for x in synth.cache(seed, L, Lv, Hkv, D, "bf16"))
    q, kn, vn = (dev(x) for x in synth.canvas(seed, B, Hq, Hkv, D, "bf16"))
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    ws = dg.alloc_workspace(q, Hkv, Lv)
    for _ in range(3):
        dg.canvas_attn(q, kc, vc, L, kn, vn, out=out, workspace=ws)
    torch.cuda.synchronize()
    dg.kernel_timing_read()
    dg.kernel_timing_enable(True)
    for _ in range(reps):
        dg.canvas_attn(q, kc, vc, L, kn, vn, out=out, workspace=ws)
    a_ms, m_ms = dg.kernel_timing_samples(reps)
    dg.kernel_timing_enable(False)
    attn_us = float(np.median(a_ms)) * 1e3
    step_us = float(np.median(np.add(a_ms, m_ms if len(m_ms) == len(a_ms) else 0.0))) * 1e3
    fl = step_flops(B, Hq, Lv, D)
    alg = step_bytes(B, Hq, Hkv, Lv, D)
    gbs = alg / (attn_us * 1e-6) / 1e9
    del kc, vc
    return {"prefix_len": Lv, "canvas_attn_us": round(attn_us, 2), "canvas_step_us": round(step_us, 2),
            "canvas_attn_tflops": round(fl / (attn_us * 1e-6) / 1e12, 1),
            "frac_of_bf16_peak": round(fl / (attn_us * 1e-6) / 1e12 / PEAK_TFLOPS["bf16"], 4),
            "hbm_GBps": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "algorithmic_bytes_per_launch": int(alg),
            # FETCH_SIZE + WRITE_SIZE per launch (calibrated counters), while they match the kernel
            "traffic": measured_traffic("long"),
            "kernel": "attn_bf16_kernel<128,false>", "timing": f"median of {reps} calls, warm"}


def fp8_summary(reps=100):
    """The fp8 canvas step at L=8192 (warm median per call) for the bf16 line."""
    cy = Cycle("fp8")
    for i in range(10):
        cy.one_step(i)
    med = call_medians(cy, reps, modes=("warm",))["warm"]
    fl = step_flops(cy.B, cy.Hq, cy.Lv, cy.D)
    return {"canvas_attn_us": med["attn"], "canvas_step_us": med["step"],
            "canvas_attn_tflops": round(fl / (med["attn"] * 1e-6) / 1e12, 2),
            "frac_of_fp8_peak": round(fl / (med["attn"] * 1e-6) / 1e12 / PEAK_TFLOPS["fp8"], 4),
            "kernel": "attn_fp8_kernel<128,false>", "timing": f"median of {reps} calls, warm"}


def back_to_back(call, reps, stream):
    """Milliseconds of each of `reps` calls enqueued back to back, one pair of events
    around each, one synchronisation at the end (a wait per call would add the
    host's launch latency to every interval)."""
    import torch
    evs = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def measure_sampler(reps=50, batch=1):
    """The canvas sampler (dg_canvas_sample) on one step's logits: B canvases of
    256 positions over the 262144-token vocabulary, tau 0.8 (the start of the
    annealing), budget 0.1, stop threshold 0.005.  Median per call over `reps`
    calls (both launches, torch events on the launch stream); the logits (bf16)
    are the algorithmic bytes."""
    import torch
    import canvas_attention_amd.dg as dg
    from canvas_attention_amd import synth
    lg = torch.from_numpy(synth.sampler_logits(1006, batch).view(np.int16)).view(torch.bfloat16).cuda()
    nz = torch.from_numpy(synth.noise_tokens(1006, batch)).cuda()
    # outputs allocated once, so that the host's work per call stays below the
    # kernels' and the calls queue up back to back
    outs = (torch.empty(batch, 256, dtype=torch.float32, device="cuda"),
            *[torch.empty(batch, 256, dtype=torch.int32, device="cuda") for _ in range(3)],
            torch.empty(batch, dtype=torch.int32, device="cuda"))
    for _ in range(5):
        dg.canvas_sample(lg, nz, None, 0.8, 0.1, 0.005, out=outs)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ts = back_to_back(lambda: dg.canvas_sample(lg, nz, None, 0.8, 0.1, 0.005, out=outs), reps,
                      stream)
    us = float(np.median(ts)) * 1e3
    nbytes = batch * 256 * synth.VOCAB * 2
    return {"batch": batch, "vocab": synth.VOCAB, "call_us_median": round(us, 3),
            "logits_bytes": nbytes, "call_GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "call_hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "kernels": "row_stats_kernel + select_kernel", "timing": f"median of {reps} calls"}



def decode_bytes(B, L, k, Hq, Hkv, D, esz=2):
    """Algorithmic bytes of one decode call: the prefix's cache K and V once, the
    new tokens' Q, K and V, the bf16 output and the appended K/V rows."""
    return B * (esz * (2 * L * Hkv * D + k * Hq * D + 2 * k * Hkv * D)
                + 2 * k * Hq * D + esz * 2 * k * Hkv * D)


def measure_decode(reps=50, names=None):
    """Decode attention (dg_decode_attn) per workload: median per call of the decode
    kernel and of the whole call (kernel + merge) from the library's HIP events,
    warm (the cache stays in the 256 MB last-level cache between calls) and cold (a
    512 MB read before every call, outside the timed kernels, as when the model's
    other layers run between two decode steps).  GB/s and the HBM fraction are the
    algorithmic bytes over the cold kernel time."""
    import torch
    import canvas_attention_amd.dg as dg
    from canvas_attention_amd import synth
    Hq, Hkv, D = 16, 8, 128
    flush = Flush()
    out = {}
    for name in names or DECODE_WORKLOADS:
        w = DECODE_WORKLOADS[name]
        B, Lv, k = w["batch"], w["prefix"], w["k"]
        L = np.full(B, Lv, np.int32)
        kc, vc = synth.cache(1300, L, Lv + k, Hkv, D, "bf16")
        kc, vc = dev(kc), dev(vc)
        q, kn, vn = (dev(x) for x in synth.decode(1300, B, k, Hq, Hkv, D, "bf16"))
        o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
        ws = torch.zeros(max(dg.decode_workspace_bytes(B, k, Hq, Hkv, D, Lv), 16), dtype=torch.uint8,
                         device="cuda")

        def call():
            dg.decode_attn(q, kn, vn, kc, vc, L, out=o, workspace=ws)

        for _ in range(5):
            call()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        med = {}
        for mode in ("warm", "cold"):
            # the decode kernel alone (library events around its launch) ...
            dg.kernel_timing_read()
            dg.kernel_timing_enable(True)
            for i in range(reps):
                if mode == "cold":
                    flush()
                call()
            a_ms, _ = dg.kernel_timing_samples(reps)
            dg.kernel_timing_enable(False)
            # ... and the whole call (kernel + merge when there is one), one pair of
            # events around it, without the per-launch events
            if mode == "cold":
                c_ms = []
                for _ in range(reps):  # the flush stays outside the timed interval
                    flush()
                    c_ms += back_to_back(call, 1, stream)
            else:
                c_ms = back_to_back(call, reps, stream)
            med[mode] = {"kernel": round(float(np.median(a_ms)) * 1e3, 3),
                         "call": round(float(np.median(c_ms)) * 1e3, 3)}
        nbytes = decode_bytes(B, Lv, k, Hq, Hkv, D)
        gbs = nbytes / (med["cold"]["kernel"] * 1e-6) / 1e9
        out[name] = {"batch": B, "prefix_len": Lv, "new_tokens": k, "algorithmic_bytes": nbytes,
                     "kernel_us": {m: med[m]["kernel"] for m in med},
                     "call_us": {m: med[m]["call"] for m in med},
                     "cold_kernel_GBps": round(gbs, 1), "cold_kernel_hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
        del kc, vc, q, kn, vn, o, ws
    del flush
    res = {"workloads": out, "heads": {"n_heads_q": Hq, "n_heads_kv": Hkv, "head_dim": D},
           "dtype": "bf16", "timing": f"median of {reps} calls per mode"}
    if DECODE_ROOFLINE in out:
        r = out[DECODE_ROOFLINE]
        res["roofline"] = {"bound": "hbm", "achieved": r["cold_kernel_GBps"], "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": r["cold_kernel_hbm_frac"],
                           "traffic": measured_traffic("decode"),
                           "kernel": "decode_kernel<FmtBf16,128,4,2> (32 sequences, L=8192, 1 token)",
                           "algorithmic_bytes_per_launch": r["algorithmic_bytes"]}
    return res


SELFCOND_SHAPE = dict(batch=1, vocab=262144, d_model=2048, d_hidden=1920)


def measure_selfcond(reps=20):
    """The self-conditioning input (dg_self_condition) for one canvas: 256 positions,
    the 262144-token vocabulary, d=2048, MLP hidden width 1920 (7.86M parameters).
    Median per call (torch events on the launch stream) and per kernel (the
    library's events: the embedding product and the softmax pass).  The embedding
    product's algorithmic bytes are E and the softmax weights (bf16) once; its
    algorithmic FLOP 2*256*V*d.  The call's algorithmic bytes are the logits, E,
    W1, W2 and z once."""
    import torch
    import canvas_attention_amd.dg as dg
    from canvas_attention_amd import synth
    sh = SELFCOND_SHAPE
    B, V, d, h = sh["batch"], sh["vocab"], sh["d_model"], sh["d_hidden"]
    lg = dev(synth.sampler_logits(1006, B, vocab=V))
    E, w1, w2 = (dev(x) for x in synth.selfcond_weights(1400, V, d, h))
    z = torch.empty((B, 256, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(dg.selfcond_workspace_bytes(B, V, d, h), dtype=torch.uint8, device="cuda")

    def call():
        dg.self_condition(lg, E, w1, w2, out=z, workspace=ws)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ts = back_to_back(call, reps, stream)
    dg.kernel_timing_read()
    dg.kernel_timing_enable(True)
    for _ in range(reps):
        call()
    gemm_ms, soft_ms = dg.kernel_timing_samples(reps)
    dg.kernel_timing_enable(False)
    call_us = float(np.median(ts)) * 1e3
    gemm_us = float(np.median(gemm_ms)) * 1e3
    soft_us = float(np.median(soft_ms)) * 1e3
    M = B * 256
    nbytes = V * d * 2 + M * V * 2
    flop = 2.0 * M * V * d
    gbs = nbytes / (gemm_us * 1e-6) / 1e9
    tfl = flop / (gemm_us * 1e-6) / 1e12
    call_bytes = M * V * 2 + V * d * 2 + 2 * d * h * 2 + M * d * 2
    return {"batch": B, "vocab": V, "d_model": d, "d_hidden": h, "call_us_median": round(call_us, 2),
            "positions_per_s": round(M / (call_us * 1e-6), 1),
            "call_GBps": round(call_bytes / (call_us * 1e-6) / 1e9, 1),
            "call_hbm_frac": round(call_bytes / (call_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "kernels_us": {"embedding_product": round(gemm_us, 2), "softmax": round(soft_us, 2)},
            "softmax_GBps": round(2 * M * V * 2 / (soft_us * 1e-6) / 1e9, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic("selfcond"),
                         "kernel": "gemm_kernel<256> (embedding product, 256 x 262144 x 2048)",
                         "algorithmic_bytes_per_launch": nbytes,
                         "mfma_tflops": round(tfl, 1), "mfma_frac": round(tfl / PEAK_TFLOPS["bf16"], 4)},
            "timing": f"median of {reps} calls"}

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--dtype", choices=("bf16", "fp8"), default="bf16",
                    help="storage format of q, K and V (fp8: OCP e4m3, tensor scales 1)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sampler", action="store_true",
                    help="only time the canvas sampler (256 x 262144 bf16 logits per canvas)")
    ap.add_argument("--long-context", action="store_true",
                    help="only time the L=131072 canvas step")
    ap.add_argument("--selfcond", action="store_true",
                    help="only time the self-conditioning input (256 x 262144 logits, d=2048, h=1920)")
    ap.add_argument("--decode", nargs="?", const="all", default=None, metavar="WORKLOAD",
                    help="only time decode attention (all workloads, or the one named: "
                         + ", ".join(DECODE_WORKLOADS) + ")")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--profile-steps", action="store_true",
                    help="only run the timed cycles (for rocprofv3 runs)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device to device 5 times (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=5, metavar=("FETCH", "WRITE", "COPY_FETCH",
                                                              "COPY_WRITE", "COPY_MIB"),
                    help="write the traffic file from four rocprofv3 --pmc output folders")
    ap.add_argument("--summarize-mfma", nargs=3, metavar=("PASS1", "PASS2", "TRACE_TXT"),
                    help="write profiles/<tag>_mfma.txt from two rocprofv3 --pmc runs")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("STATS_CSV", "OUT_TXT"),
                    help="write a kernel summary from a rocprofv3 --stats kernel_stats.csv")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters,
                           dtype="sampler" if args.sampler else "decode" if args.decode
                           else "selfcond" if args.selfcond else "long" if args.long_context
                           else args.dtype)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, dtype=args.dtype, sampler=args.sampler,
                        decode=args.decode, selfcond=args.selfcond, long_context=args.long_context)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma, dtype=args.dtype)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the canvas "
              "attention path has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    torch.cuda.set_device(0)
    if args.sampler:
        print(json.dumps({"sampler": measure_sampler(max(args.steps, 10))}), flush=True)
        return
    if args.selfcond:
        print(json.dumps({"selfcond": measure_selfcond(max(args.steps, 5))}), flush=True)
        return
    if args.long_context:
        print(json.dumps({"long_context": long_context_summary(max(args.steps, 5))}), flush=True)
        return
    if args.decode:
        names = None if args.decode == "all" else [args.decode]
        print(json.dumps({"decode": measure_decode(max(args.steps, 10), names)}), flush=True)
        return
    m = measure(args.dtype, args.steps, args.warmup, args.profile_steps)
    if args.profile_steps:
        print(json.dumps(m), flush=True)
        return
    cfg = m.pop("_config")
    result = {
        "metric": METRIC,
        "value": m.pop("value"),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": "canvas denoising step at prefix L=8192 (timed inside block cycles of "
                               "12 canvas steps + commit; ms_per_step is one cycle)", **cfg},
        **m,
    }
    if args.dtype == "bf16":
        result["fp8"] = fp8_summary()
        result["long_context"] = long_context_summary()
        result["sampler"] = measure_sampler()
        result["decode"] = measure_decode()
        result["selfcond"] = measure_selfcond()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds, args.dtype)
    print(json.dumps(result), flush=True)


def cpu_baseline(budget_s, dtype="bf16"):
    """The CPU fp64 oracle (as it stands, untuned) on bounded samples of the canvas
    step at L=2048, L=8192 and L=131072 (B=1, 256 positions, Hq=16, Hkv=8, D=128):
    whole steps, each with its own seeded canvas Q/K/V, one after another until a
    share of the time budget is spent (at least one step), on all the threads the
    oracle's OpenMP runtime takes; then the L=2048 and L=8192 steps on one thread.
    value is the L=8192 figure on all threads (the metric's workload)."""
    import oracle
    from canvas_attention_amd import synth
    threads = oracle.num_threads()
    shares = {"step_l2k": 0.15, "cycle_l8k": 0.25, "long_l128k": 0.0}
    one_thread = {"step_l2k": 0.1, "cycle_l8k": 0.35}

    def run(name, budget, nthreads):
        w = synth.WORKLOADS[name]
        B, Hq, Hkv, D, seed = w["batch"], w["hq"], w["hkv"], w["d"], w["seed"]
        L = synth.prefix_lengths(name)
        Lv = int(L[0])
        kc, vc = synth.cache(seed, L, Lv + 256, Hkv, D, dtype)
        steps = [synth.canvas(seed, B, Hq, Hkv, D, dtype, step=s) for s in range(3)]
        oracle.set_num_threads(nthreads)
        done, t_start, elapsed = 0, time.perf_counter(), 0.0
        while done == 0 or elapsed < budget:
            q, kn, vn = steps[done % len(steps)]
            oracle.canvas_attn(q, kc, vc, L, kn, vn)
            done += 1
            elapsed = time.perf_counter() - t_start
        fl = done * step_flops(B, Hq, Lv, D)
        return {"prefix_len": Lv, "threads": nthreads, "steps": done, "seconds": round(elapsed, 2),
                "TFLOP/s": round(fl / elapsed / 1e12, 6),
                "canvas_positions_per_s": round(done * B * 256 / elapsed, 1)}

    figs = {f"{n}_all_threads": run(n, budget_s * f, threads) for n, f in shares.items()}
    figs.update({f"{n}_1_thread": run(n, budget_s * f, 1) for n, f in one_thread.items()})
    oracle.set_num_threads(threads)
    main = figs["cycle_l8k_all_threads"]
    return {"value": main["TFLOP/s"], "unit": "TFLOP/s", "cores": threads,
            "cpu_count": os.cpu_count(), "kind": "oracle",
            "sample": f"{main['steps']} whole canvas steps at L=8192 (B=1, 256 positions, Hq=16, Hkv=8, "
                      f"D=128) on {threads} threads in {main['seconds']} s: "
                      f"{main['canvas_positions_per_s']} canvas positions/s; baseline only",
            "configs": figs}


if __name__ == "__main__":
    main()
