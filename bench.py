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
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the canvas "
              "attention path has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch

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
        "kernels_us": {"canvas_attn": round(attn_us, 3), "canvas_merge": round(merge_us, 3),
                       "commit_attn": round(cattn_ms / max(n_cattn, 1) * 1e3, 3),
                       "commit_merge": round(cmerge_ms / max(n_cmerge, 1) * 1e3, 3)
                       if n_cmerge else 0.0},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "attn_bf16_kernel<128,false> (canvas step, L=8192)",
                     "algorithmic_flop_per_launch": fl_step,
                     "hbm_frac": round(step_bytes(B, Hq, Hkv, Lv, D) / (attn_us * 1e-6) / 1e9
                                       / PEAK_HBM_GBS, 4)},
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(name, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline(name, budget_s):
    """The CPU fp64 oracle on a bounded sample of the same canvas step: whole
    canvas rows (all heads) in chunks until the time budget is spent."""
    import oracle
    from canvas_attention_amd import synth
    w = synth.WORKLOADS[name]
    B, Hq, Hkv, D, seed = w["batch"], w["hq"], w["hkv"], w["d"], w["seed"]
    L = synth.prefix_lengths(name)
    Lv = int(L[0])
    kc, vc = synth.cache(seed, L, Lv + 256, Hkv, D, "bf16")
    q, kn, vn = synth.canvas(seed, B, Hq, Hkv, D, "bf16")
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    done_rows = 0
    t_start = time.perf_counter()
    elapsed = 0.0
    i0 = 0
    while elapsed < budget_s and i0 < 256:
        rows = np.array([(0, i, h) for i in range(i0, min(256, i0 + 16)) for h in range(Hq)],
                        np.int32)
        oracle.canvas_attn(q, kc, vc, L, kn, vn, rows=rows)
        done_rows += len(rows)
        i0 += 16
        elapsed = time.perf_counter() - t_start
    flops = done_rows * 4.0 * (Lv + 256) * D
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done_rows} of {B * 256 * Hq} query rows of one canvas step at L={Lv} "
                      f"({done_rows // Hq} canvas positions, all {Hq} heads), {elapsed:.1f} s; "
                      f"canvas positions/s {done_rows / Hq / elapsed:.2f}"}


if __name__ == "__main__":
    main()
