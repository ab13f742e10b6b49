"""Builds libdg.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

    python -m canvas_attention_amd.build        # or __graft_entry__.build()

Every HIP source is compiled for gfx950 only, with packed-fp32 VALU ops
disabled in the device pass, and linked into canvas_attention_amd/libdg.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdg.so")
SOURCES = ["dg_attn_mfma.hip", "dg_attn_f32.hip", "dg_merge.hip", "dg_sample.hip", "dg_selfcond.hip",
           "dg_api.cpp", "dg_plan.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdg.so)")


def compile_flags(extra=()):
    return ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", *extra]


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [cc, *compile_flags(extra), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
        if lines and (verbose or p.returncode):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    subprocess.check_call([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
