"""GPU parity: libdg (through its C ABI) against the CPU fp64 oracle.

Gates (per-row normalised max error, see helpers.row_err): 2e-2 for bf16
storage with fp32 accumulation, 1e-5 for the fp32 path.  Inputs come from the
seeded generator of canvas_attention_amd.synth; the oracle widens exactly the
bf16 values the GPU reads.
"""
import os

import numpy as np
import pytest

from canvas_attention_amd import synth
from helpers import TOL_BF16, TOL_F32, record, row_err, to_dev, to_host_bits, to_host_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU machines skip the module
    pytest.skip("needs a GPU", allow_module_level=True)

import canvas_attention_amd.dg as dg  # noqa: E402  (loads libdg.so; raises if missing)


@pytest.fixture
def split_keys():
    """Force keys per split through DG_SPLIT_KEYS for one test."""
    old = os.environ.get("DG_SPLIT_KEYS")

    def set_(v):
        if v is None:
            os.environ.pop("DG_SPLIT_KEYS", None)
        else:
            os.environ["DG_SPLIT_KEYS"] = str(v)

    yield set_
    set_(old)


def make(seed, B, L, Hq, Hkv, D, dtype, cap=None, block=0, step=0):
    L = np.asarray(L, np.int32)
    cap = cap or int(L.max()) + 256
    kc, vc = synth.cache(seed, L, cap, Hkv, D, dtype)
    q, kn, vn = synth.canvas(seed, B, Hq, Hkv, D, dtype, block=block, step=step)
    return dict(L=L, kc=kc, vc=vc, q=q, kn=kn, vn=vn)


def run_canvas(c, ws=None):
    out = dg.canvas_attn(to_dev(c["q"]), to_dev(c["kc"]), to_dev(c["vc"]), c["L"],
                         to_dev(c["kn"]), to_dev(c["vn"]), workspace=ws)
    torch.cuda.synchronize()
    return out


def check_canvas(c, tol, what="canvas step"):
    """Every output row of one canvas step against the oracle."""
    out = to_host_f64(run_canvas(c))
    err = record(what, row_err(out, oracle_canvas(c)), tol)
    assert err <= tol, f"per-row error {err:.3e} > {tol}"
    return err


def oracle_canvas(c):
    import oracle
    return oracle.canvas_attn(c["q"], c["kc"], c["vc"], c["L"], c["kn"], c["vn"])


def check_commit(oracle_lib, qb, kb, vb, kc, vc, L, out, what="commit"):
    """Every output row of one commit against the oracle (kc, vc: the cache
    before the append)."""
    ref = oracle_lib.commit_attn(qb, kc, vc, L, kb, vb)
    err = record(what, row_err(to_host_f64(out), ref), TOL_BF16)
    assert err <= TOL_BF16, f"{what}: per-row error {err:.3e} > {TOL_BF16}"
    return err


# --------------------------------------------------------------- fp32 workload

@pytest.mark.parametrize("forced", [None, 64, 96])
def test_tiny_fp32_step_and_commit(oracle_lib, split_keys, forced):
    """fp32, L=64, Nc=256, Hq=4, Hkv=2, D=64: canvas step, then the commit of a
    block and its append, checked against attention over all 320 positions."""
    split_keys(forced)
    w = synth.WORKLOADS["tiny_fp32_l64"]
    L = synth.prefix_lengths("tiny_fp32_l64")
    seed, Hq, Hkv, D = w["seed"], w["hq"], w["hkv"], w["d"]
    cap = 320
    c = make(seed, 1, L, Hq, Hkv, D, "f32", cap=cap)
    check_canvas(c, TOL_F32, f"fp32 canvas step, split {forced}")
    qb, kb, vb = synth.block(seed, 1, Hq, Hkv, D, "f32")
    kc_d, vc_d = to_dev(c["kc"]), to_dev(c["vc"])
    out = dg.commit_block(to_dev(qb), to_dev(kb), to_dev(vb), kc_d, vc_d, L)
    torch.cuda.synchronize()
    ref = oracle_lib.commit_attn(qb, c["kc"], c["vc"], L, kb, vb)
    err = record(f"fp32 commit, split {forced}", row_err(to_host_f64(out), ref), TOL_F32)
    assert err <= TOL_F32, err
    kc2, vc2 = c["kc"].copy(), c["vc"].copy()
    oracle_lib.append_block(kb, vb, kc2, vc2, L)
    np.testing.assert_array_equal(to_host_bits(kc_d), kc2)
    np.testing.assert_array_equal(to_host_bits(vc_d), vc2)


# --------------------------------------------------------------- bf16 canvas

def test_step_l2k_full(oracle_lib):
    """bf16 L=2048, Hq=16, Hkv=8, D=128; every output row against the oracle."""
    w = synth.WORKLOADS["step_l2k"]
    c = make(w["seed"], 1, synth.prefix_lengths("step_l2k"), w["hq"], w["hkv"], w["d"], "bf16",
             cap=2048)
    check_canvas(c, TOL_BF16, "L=2048 canvas step")


@pytest.mark.parametrize("B,L,Hq,Hkv,D,forced", [
    (1, [0], 16, 8, 128, None),          # empty prefix: plain bidirectional attention
    (1, [1], 16, 8, 128, None),
    (2, [1000, 77], 16, 8, 128, 96),     # ragged tails, many splits
    (2, [333, 0], 4, 4, 128, 160),       # G = 1
    (1, [515], 8, 2, 128, 64),           # G = 4
    (2, [700, 64], 4, 2, 64, 128),       # head_dim 64
    (3, [40, 1100, 257], 16, 8, 128, None),
])
def test_canvas_small_shapes(oracle_lib, split_keys, B, L, Hq, Hkv, D, forced):
    split_keys(forced)
    c = make(7, B, L, Hq, Hkv, D, "bf16")
    check_canvas(c, TOL_BF16, f"B={B} L={L} G={Hq // Hkv} D={D} split={forced}")


@pytest.mark.parametrize("forced", [128, 160, 192, 256, 288, 352, 416])
@pytest.mark.parametrize("L", [100, 190])
def test_canvas_ring_depths(oracle_lib, split_keys, forced, L):
    """Units of 2 .. 7 ring stages (64 keys each in the default shape), with the
    cache/canvas seam inside different stages: the first-chunk barrier and the tail
    of the ring protocol take their counted and their full waits."""
    split_keys(forced)
    c = make(31, 1, [L], 16, 8, 128, "bf16")
    check_canvas(c, TOL_BF16, f"L={L} split={forced}")


@pytest.mark.parametrize("forced", [128, 192, 288, 416])
def test_commit_ring_depths(oracle_lib, split_keys, forced):
    """The causal commit over units of 2 .. 7 stages, with the seam and the
    diagonal in the same units."""
    split_keys(forced)
    Ls = np.asarray([150], np.int32)
    cap = int(Ls.max()) + 256
    kc, vc = synth.cache(32, Ls, cap, 8, 128, "bf16")
    qb, kb, vb = synth.block(32, 1, 16, 8, 128, "bf16")
    kc_d, vc_d = to_dev(kc), to_dev(vc)
    out = dg.commit_block(to_dev(qb), to_dev(kb), to_dev(vb), kc_d, vc_d, Ls)
    torch.cuda.synchronize()
    check_commit(oracle_lib, qb, kb, vb, kc, vc, Ls, out, f"commit split={forced}")


def test_canvas_long_context_full(oracle_lib):
    """bf16 L=131072: split-key merge and cache streaming; every output row."""
    w = synth.WORKLOADS["long_l128k"]
    L = synth.prefix_lengths("long_l128k")
    c = make(w["seed"], 1, L, w["hq"], w["hkv"], w["d"], "bf16", cap=int(L[0]))
    check_canvas(c, TOL_BF16, "L=131072 canvas step")


def test_rising_scores_exercise_rescale(oracle_lib, split_keys):
    """Keys whose scores grow along the sequence force repeated max updates."""
    split_keys(None)
    c = make(11, 1, [3000], 16, 8, 128, "bf16")
    f = synth.bf16_to_f32(c["kc"])
    ramp = np.linspace(0.2, 12.0, f.shape[1], dtype=np.float32)[None, :, None, None]
    c["kc"] = synth.bf16_round(f * ramp)
    q = synth.bf16_to_f32(c["q"]) * 2.0
    c["q"] = synth.bf16_round(q)
    check_canvas(c, TOL_BF16, "rising scores")


def test_determinism(split_keys):
    split_keys(None)
    c = make(12, 2, [4000, 1500], 16, 8, 128, "bf16")
    a = to_host_bits(run_canvas(c))
    b = to_host_bits(run_canvas(c))
    np.testing.assert_array_equal(a, b)


# --------------------------------------------------------------- commit

@pytest.mark.parametrize("B,L,Hq,Hkv,D,forced", [
    (1, [0], 16, 8, 128, None),
    (2, [130, 999], 16, 8, 128, 96),
    (1, [64], 8, 2, 64, None),
    (1, [2000], 4, 4, 128, 224),
])
def test_commit_small(oracle_lib, split_keys, B, L, Hq, Hkv, D, forced):
    split_keys(forced)
    Ls = np.asarray(L, np.int32)
    cap = int(Ls.max()) + 256 + 32
    kc, vc = synth.cache(21, Ls, cap, Hkv, D, "bf16")
    qb, kb, vb = synth.block(21, B, Hq, Hkv, D, "bf16")
    kc_d, vc_d = to_dev(kc), to_dev(vc)
    out = dg.commit_block(to_dev(qb), to_dev(kb), to_dev(vb), kc_d, vc_d, Ls)
    torch.cuda.synchronize()
    check_commit(oracle_lib, qb, kb, vb, kc, vc, Ls, out, f"commit B={B} L={L} split={forced}")
    oracle_lib.append_block(kb, vb, kc, vc, Ls)
    np.testing.assert_array_equal(to_host_bits(kc_d), kc)
    np.testing.assert_array_equal(to_host_bits(vc_d), vc)


def test_block_cycle_l8k(oracle_lib):
    """12 canvas steps against a fixed L=8192 cache (loop == single calls, bit for
    bit), then the commit (L -> 8448), then a step on the grown cache; every
    output row of all 14 calls against the oracle."""
    w = synth.WORKLOADS["cycle_l8k"]
    seed, Hq, Hkv, D = w["seed"], w["hq"], w["hkv"], w["d"]
    L = synth.prefix_lengths("cycle_l8k")
    cap = int(L[0]) + 256
    kc, vc = synth.cache(seed, L, cap, Hkv, D, "bf16")
    kc_d, vc_d = to_dev(kc), to_dev(vc)
    steps = [synth.canvas(seed, 1, Hq, Hkv, D, "bf16", step=s) for s in range(12)]
    qs = torch.stack([to_dev(s[0]) for s in steps])
    ks = torch.stack([to_dev(s[1]) for s in steps])
    vs = torch.stack([to_dev(s[2]) for s in steps])
    loop_out = dg.canvas_step_loop(qs, ks, vs, kc_d, vc_d, L)
    singles = [dg.canvas_attn(qs[s], kc_d, vc_d, L, ks[s], vs[s]) for s in range(12)]
    torch.cuda.synchronize()
    for s in range(12):
        assert torch.equal(loop_out[s], singles[s]), f"step {s}: loop differs from single call"
    for s in range(12):
        ref = oracle_lib.canvas_attn(steps[s][0], kc, vc, L, steps[s][1], steps[s][2])
        err = record(f"L=8192 step {s}", row_err(to_host_f64(loop_out[s]), ref), TOL_BF16)
        assert err <= TOL_BF16, f"step {s}: {err:.3e}"
    qb, kb, vb = synth.block(seed, 1, Hq, Hkv, D, "bf16")
    out = dg.commit_block(to_dev(qb), to_dev(kb), to_dev(vb), kc_d, vc_d, L)
    torch.cuda.synchronize()
    check_commit(oracle_lib, qb, kb, vb, kc, vc, L, out, "L=8192 commit")
    oracle_lib.append_block(kb, vb, kc, vc, L)
    np.testing.assert_array_equal(to_host_bits(kc_d), kc)
    np.testing.assert_array_equal(to_host_bits(vc_d), vc)
    L2 = L + 256
    q2, k2, v2 = synth.canvas(seed, 1, Hq, Hkv, D, "bf16", block=1)
    out2 = dg.canvas_attn(to_dev(q2), kc_d, vc_d, L2, to_dev(k2), to_dev(v2))
    torch.cuda.synchronize()
    ref2 = oracle_lib.canvas_attn(q2, kc, vc, L2, k2, v2)
    err = record("L=8448 step after the commit", row_err(to_host_f64(out2), ref2), TOL_BF16)
    assert err <= TOL_BF16


def test_ragged_multi_block_generation(oracle_lib):
    """Batch of 8 sequences with seeded prefixes in [1024, 32768]; 4 blocks of
    (12 steps + commit).  Every output row of one seeded step per block and of
    every commit against the oracle; every step of the loop equals its single
    call bit for bit; the cache ends equal to the oracle's appends."""
    w = synth.WORKLOADS["ragged_b8"]
    seed, B, Hq, Hkv, D = w["seed"], w["batch"], w["hq"], w["hkv"], w["d"]
    L = synth.prefix_lengths("ragged_b8").copy()
    cap = int(L.max()) + 4 * 256
    kc, vc = synth.cache(seed, L, cap, Hkv, D, "bf16")
    kc_d, vc_d = to_dev(kc), to_dev(vc)
    ws = dg.alloc_workspace(to_dev(synth.canvas(seed, B, Hq, Hkv, D, "bf16")[0]), Hkv,
                            int(L.max()) + 3 * 256)
    rng = np.random.default_rng(2)
    for blk in range(4):
        steps = [synth.canvas(seed, B, Hq, Hkv, D, "bf16", block=blk, step=s) for s in range(12)]
        qs = torch.stack([to_dev(s[0]) for s in steps])
        ks = torch.stack([to_dev(s[1]) for s in steps])
        vs = torch.stack([to_dev(s[2]) for s in steps])
        out = dg.canvas_step_loop(qs, ks, vs, kc_d, vc_d, L, workspace=ws)
        s = int(rng.integers(12))
        single = dg.canvas_attn(qs[s], kc_d, vc_d, L, ks[s], vs[s], workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out[s], single), f"block {blk} step {s}: loop differs from single call"
        ref = oracle_lib.canvas_attn(steps[s][0], kc, vc, L, steps[s][1], steps[s][2])
        err = record(f"ragged block {blk} step {s}", row_err(to_host_f64(out[s]), ref), TOL_BF16)
        assert err <= TOL_BF16, f"block {blk} step {s}: {err:.3e}"
        qb, kb, vb = synth.block(seed, B, Hq, Hkv, D, "bf16", block=blk)
        outc = dg.commit_block(to_dev(qb), to_dev(kb), to_dev(vb), kc_d, vc_d, L, workspace=ws)
        torch.cuda.synchronize()
        check_commit(oracle_lib, qb, kb, vb, kc, vc, L, outc, f"ragged block {blk} commit")
        oracle_lib.append_block(kb, vb, kc, vc, L)
        L = L + 256
    np.testing.assert_array_equal(to_host_bits(kc_d), kc)
    np.testing.assert_array_equal(to_host_bits(vc_d), vc)
