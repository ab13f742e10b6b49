"""GPU parity of the fp8 path (OCP e4m3 q, K, V with per-tensor scales; bf16 out)
against the CPU fp64 oracle on the same bytes.

Gates (tests/helpers.py): an elementwise bound derived from rounding each softmax
weight to e4m3, a root-mean-square ratio and, for rows with at least 256 keys, the
per-row normalised error.  A construction with integer log2-domain scores makes
every e4m3 weight an exact power of two; there the only error left is bf16
rounding, and the bf16 gate applies, which pins the fp8 data path (key order,
operand layouts, masking, merges) far more tightly than the fp8 gates.
"""
import os

import numpy as np
import pytest

from canvas_attention_amd import synth
from helpers import TOL_BF16, fp8_check, row_err, sample_rows, to_dev, to_host_bits, to_host_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU machines skip the module
    pytest.skip("needs a GPU", allow_module_level=True)

import canvas_attention_amd.dg as dg  # noqa: E402  (loads libdg.so; raises if missing)

D = 128
LN2 = float(np.log(2.0))


@pytest.fixture
def split_keys():
    old = os.environ.get("DG_SPLIT_KEYS")

    def set_(v):
        if v is None:
            os.environ.pop("DG_SPLIT_KEYS", None)
        else:
            os.environ["DG_SPLIT_KEYS"] = str(v)

    yield set_
    set_(old)


def make(seed, B, L, Hq, Hkv, cap=None, block=0, step=0):
    L = np.asarray(L, np.int32)
    cap = cap or int(L.max()) + 256
    kc, vc = synth.cache(seed, L, cap, Hkv, D, "fp8")
    q, kn, vn = synth.canvas(seed, B, Hq, Hkv, D, "fp8", block=block, step=step)
    return dict(L=L, kc=kc, vc=vc, q=q, kn=kn, vn=vn)


def abs_bytes(v):
    """e4m3 bytes of |v| (sign bit cleared)."""
    return v & np.uint8(0x7F)


def gpu_canvas(c, scale=None, ts=None):
    out = dg.canvas_attn(to_dev(c["q"]), to_dev(c["kc"]), to_dev(c["vc"]), c["L"],
                         to_dev(c["kn"]), to_dev(c["vn"]), scale=scale, tensor_scales=ts)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    return to_host_f64(out)


def oracle_canvas(o, c, rows=None, scale=None, ts=None, absv=False):
    f = abs_bytes if absv else (lambda x: x)
    return o.canvas_attn(c["q"], c["kc"], f(c["vc"]), c["L"], c["kn"], f(c["vn"]), scale=scale,
                         rows=rows, tensor_scales=ts)


def check_canvas(o, c, rows=None, scale=None, ts=None):
    got = gpu_canvas(c, scale, ts)
    if rows is not None:
        got = got[rows[:, 0], rows[:, 1], rows[:, 2]]
    ref = oracle_canvas(o, c, rows, scale, ts)
    ref_abs = oracle_canvas(o, c, rows, scale, ts, absv=True)
    return fp8_check(got, ref, ref_abs)


# ------------------------------------------------------------ exact weights

def integer_score_inputs(seed, B, L, Hq, Hkv, cap=None):
    """q with two entries of +-1 and K with entries in {-2..2}: every q.k is an
    integer in [-4, 4].  With scale ln 2 the log2-domain scores are integers, so
    every exponential the kernel forms is a power of two that e4m3 holds exactly.
    V stays N(0,1)."""
    rng = np.random.default_rng(seed)
    L = np.asarray(L, np.int32)
    cap = cap or int(L.max()) + 256

    def ints(shape):
        x = rng.integers(-2, 3, size=shape).astype(np.float32)
        return synth.e4m3_round(x)

    def sparse_q(shape):
        x = np.zeros(shape, np.float32)
        flat = x.reshape(-1, shape[-1])
        for r in range(flat.shape[0]):
            idx = rng.choice(shape[-1], 2, replace=False)
            flat[r, idx] = rng.choice([-1.0, 1.0], 2)
        return synth.e4m3_round(x)

    kc = np.zeros((B, cap, Hkv, D), np.uint8)
    for b in range(B):
        kc[b, :L[b]] = ints((int(L[b]), Hkv, D))
    vc = synth.cache(seed, L, cap, Hkv, D, "fp8")[1]
    q = sparse_q((B, 256, Hq, D))
    kn = ints((B, 256, Hkv, D))
    vn = synth.canvas(seed, B, Hq, Hkv, D, "fp8")[2]
    return dict(L=L, kc=kc, vc=vc, q=q, kn=kn, vn=vn)


@pytest.mark.parametrize("B,L,Hq,Hkv,forced", [
    (1, [1000], 16, 8, None),
    (2, [1000, 77], 16, 8, 128),
    (1, [0], 16, 8, None),
    (1, [515], 8, 2, 192),
])
def test_fp8_exact_weights_canvas(oracle_lib, split_keys, B, L, Hq, Hkv, forced):
    split_keys(forced)
    c = integer_score_inputs(3, B, L, Hq, Hkv)
    got = gpu_canvas(c, scale=LN2)
    ref = oracle_canvas(oracle_lib, c, scale=LN2)
    err = row_err(got, ref)
    assert err <= TOL_BF16 / 2, err
    print(f"exact-weight canvas B={B} L={L} split={forced}: err {err:.2e}")


@pytest.mark.parametrize("L,forced", [([0], None), ([300], 128), ([2000], None)])
def test_fp8_exact_weights_commit(oracle_lib, split_keys, L, forced):
    split_keys(forced)
    c = integer_score_inputs(4, 1, L, 16, 8)
    kc_d, vc_d = to_dev(c["kc"]), to_dev(c["vc"])
    out = dg.commit_block(to_dev(c["q"]), to_dev(c["kn"]), to_dev(c["vn"]), kc_d, vc_d, c["L"],
                          scale=LN2)
    torch.cuda.synchronize()
    ref = oracle_lib.commit_attn(c["q"], c["kc"], c["vc"], c["L"], c["kn"], c["vn"], scale=LN2)
    err = row_err(to_host_f64(out), ref)
    assert err <= TOL_BF16 / 2, err
    kc2, vc2 = c["kc"].copy(), c["vc"].copy()
    oracle_lib.append_block(c["kn"], c["vn"], kc2, vc2, c["L"])
    np.testing.assert_array_equal(to_host_bits(kc_d), kc2)
    np.testing.assert_array_equal(to_host_bits(vc_d), vc2)
    print(f"exact-weight commit L={L} split={forced}: err {err:.2e}")


# ------------------------------------------------------------ N(0,1) data

def test_fp8_step_l2k_full(oracle_lib):
    """L=2048, Hq=16, Hkv=8: every output row."""
    c = make(1102, 1, [2048], 16, 8, cap=2048)
    rerr, rms = check_canvas(oracle_lib, c)
    print(f"fp8 L=2048 row err {rerr:.3e} rms {rms:.3e}")


@pytest.mark.parametrize("B,L,Hq,Hkv,forced", [
    (1, [0], 16, 8, None),
    (1, [1], 16, 8, None),
    (2, [1000, 77], 16, 8, 128),
    (2, [333, 0], 4, 4, 192),
    (1, [515], 8, 2, 64),
    (3, [40, 1100, 257], 16, 8, None),
])
def test_fp8_canvas_small_shapes(oracle_lib, split_keys, B, L, Hq, Hkv, forced):
    split_keys(forced)
    c = make(7, B, L, Hq, Hkv)
    rerr, rms = check_canvas(oracle_lib, c)
    print(f"fp8 B={B} L={L} split={forced}: row {rerr:.3e} rms {rms:.3e}")


@pytest.mark.parametrize("forced", [128, 256, 384, 512, 640, 768, 896])
@pytest.mark.parametrize("L", [700, 890])
def test_fp8_ring_depths(oracle_lib, split_keys, forced, L):
    """Units of 1 .. 7 ring stages (128 keys each: two key groups of 64) with the
    cache/canvas seam inside different stages: the first-chunk barrier and the
    tail of the ring protocol take their counted and their full waits."""
    split_keys(forced)
    c = make(31, 1, [L], 16, 8)
    rerr, rms = check_canvas(oracle_lib, c)
    print(f"fp8 L={L} split={forced}: row {rerr:.3e} rms {rms:.3e}")


def test_fp8_tensor_scales(oracle_lib, split_keys):
    """Per-tensor scales fold into the score scale (q, k) and the normalisation (v)."""
    split_keys(None)
    c = make(8, 1, [700], 16, 8)
    ts = (0.5, 1.75, 3.0)
    rerr, rms = check_canvas(oracle_lib, c, ts=ts)
    print(f"fp8 scales {ts}: row {rerr:.3e} rms {rms:.3e}")


def test_fp8_rising_scores_exercise_rescale(oracle_lib, split_keys):
    """Key magnitudes growing along the sequence: the reference max rises again and
    again, and every exponential must stay within e4m3 (a NaN would spread)."""
    split_keys(None)
    c = make(11, 1, [3000], 16, 8)
    rng = np.random.default_rng(5)
    f = rng.standard_normal(c["kc"].shape).astype(np.float32)
    ramp = np.linspace(0.2, 12.0, f.shape[1], dtype=np.float32)[None, :, None, None]
    c["kc"] = synth.e4m3_round(f * ramp)
    c["q"] = synth.e4m3_round(2.0 * rng.standard_normal(c["q"].shape).astype(np.float32))
    got = gpu_canvas(c)
    assert np.isfinite(got).all()
    ref = oracle_canvas(oracle_lib, c)
    ref_abs = oracle_canvas(oracle_lib, c, absv=True)
    # weights far below the running max become e4m3 subnormals, outside the
    # elementwise bound's relative model: the statistical gates apply
    err = np.abs(got - ref)
    rms = float(np.sqrt((err ** 2).sum() / (ref ** 2).sum()))
    assert rms <= 0.04, rms
    assert row_err(got, ref) <= 0.1
    assert (err <= 0.1 * ref_abs + 1e-3).all()
    print(f"fp8 rising scores rms {rms:.3e}")


def test_fp8_long_context_sampled(oracle_lib):
    """L=131072: split-key merge over a long fp8 cache; sampled rows."""
    c = make(1104, 1, [131072], 16, 8, cap=131072)
    rows = sample_rows(np.random.default_rng(0), 1, 256, 16, 48)
    rerr, rms = check_canvas(oracle_lib, c, rows)
    print(f"fp8 L=131072 sampled: row {rerr:.3e} rms {rms:.3e}")


def test_fp8_determinism(split_keys):
    split_keys(None)
    c = make(12, 2, [4000, 1500], 16, 8)
    a = gpu_canvas(c)
    b = gpu_canvas(c)
    np.testing.assert_array_equal(a, b)


# ------------------------------------------------------------ commit and cycle

@pytest.mark.parametrize("B,L,Hq,Hkv,forced", [
    (1, [0], 16, 8, None),
    (2, [130, 999], 16, 8, 128),
    (1, [2000], 4, 4, 192),
])
def test_fp8_commit(oracle_lib, split_keys, B, L, Hq, Hkv, forced):
    split_keys(forced)
    Ls = np.asarray(L, np.int32)
    cap = int(Ls.max()) + 256 + 64
    kc, vc = synth.cache(21, Ls, cap, Hkv, D, "fp8")
    qb, kb, vb = synth.block(21, B, Hq, Hkv, D, "fp8")
    kc_d, vc_d = to_dev(kc), to_dev(vc)
    out = dg.commit_block(to_dev(qb), to_dev(kb), to_dev(vb), kc_d, vc_d, Ls)
    torch.cuda.synchronize()
    ref = oracle_lib.commit_attn(qb, kc, vc, Ls, kb, vb)
    ref_abs = oracle_lib.commit_attn(qb, kc, abs_bytes(vc), Ls, kb, abs_bytes(vb))
    # early block rows see few keys: no per-row gate, the elementwise bound holds
    rerr, rms = fp8_check(to_host_f64(out), ref, ref_abs, per_row=False)
    oracle_lib.append_block(kb, vb, kc, vc, Ls)
    np.testing.assert_array_equal(to_host_bits(kc_d), kc)
    np.testing.assert_array_equal(to_host_bits(vc_d), vc)
    print(f"fp8 commit B={B} L={L}: row {rerr:.3e} rms {rms:.3e}")


def test_fp8_block_cycle_l8k(oracle_lib):
    """12 fp8 canvas steps against a fixed L=8192 cache (the loop equals single
    calls bit for bit), the commit (L -> 8448) with its append, then one step on
    the grown cache."""
    seed, Hq, Hkv = 1103, 16, 8
    L = np.asarray([8192], np.int32)
    cap = int(L[0]) + 256
    kc, vc = synth.cache(seed, L, cap, Hkv, D, "fp8")
    kc_d, vc_d = to_dev(kc), to_dev(vc)
    steps = [synth.canvas(seed, 1, Hq, Hkv, D, "fp8", step=s) for s in range(12)]
    qs = to_dev(np.stack([s[0] for s in steps]))
    ks = to_dev(np.stack([s[1] for s in steps]))
    vs = to_dev(np.stack([s[2] for s in steps]))
    loop_out = dg.canvas_step_loop(qs, ks, vs, kc_d, vc_d, L)
    singles = [dg.canvas_attn(qs[s], kc_d, vc_d, L, ks[s], vs[s]) for s in range(12)]
    torch.cuda.synchronize()
    for s in range(12):
        assert torch.equal(loop_out[s], singles[s]), f"step {s}: loop differs from single call"
    rng = np.random.default_rng(1)
    for s in (0, 11):
        rows = sample_rows(rng, 1, 256, Hq, 96)
        c = dict(L=L, kc=kc, vc=vc, q=steps[s][0], kn=steps[s][1], vn=steps[s][2])
        got = to_host_f64(loop_out[s])[rows[:, 0], rows[:, 1], rows[:, 2]]
        fp8_check(got, oracle_canvas(oracle_lib, c, rows), oracle_canvas(oracle_lib, c, rows, absv=True))
    qb, kb, vb = synth.block(seed, 1, Hq, Hkv, D, "fp8")
    out = dg.commit_block(to_dev(qb), to_dev(kb), to_dev(vb), kc_d, vc_d, L)
    torch.cuda.synchronize()
    rows = sample_rows(rng, 1, 256, Hq, 128)
    ref = oracle_lib.commit_attn(qb, kc, vc, L, kb, vb, rows=rows)
    ref_abs = oracle_lib.commit_attn(qb, kc, abs_bytes(vc), L, kb, abs_bytes(vb), rows=rows)
    got = to_host_f64(out)[rows[:, 0], rows[:, 1], rows[:, 2]]
    rerr, rms = fp8_check(got, ref, ref_abs)
    oracle_lib.append_block(kb, vb, kc, vc, L)
    np.testing.assert_array_equal(to_host_bits(kc_d), kc)
    np.testing.assert_array_equal(to_host_bits(vc_d), vc)
    L2 = L + 256
    q2, k2, v2 = synth.canvas(seed, 1, Hq, Hkv, D, "fp8", block=1)
    c2 = dict(L=L2, kc=kc, vc=vc, q=q2, kn=k2, vn=v2)
    out2 = dg.canvas_attn(to_dev(q2), kc_d, vc_d, L2, to_dev(k2), to_dev(v2))
    torch.cuda.synchronize()
    got2 = to_host_f64(out2)[rows[:, 0], rows[:, 1], rows[:, 2]]
    fp8_check(got2, oracle_canvas(oracle_lib, c2, rows), oracle_canvas(oracle_lib, c2, rows, absv=True))
    print(f"fp8 cycle ok, commit row {rerr:.3e} rms {rms:.3e}")


def test_fp8_ragged_batch(oracle_lib):
    """Eight sequences with the ragged workload's prefix lengths: two canvas steps
    and a commit, sampled rows."""
    Hq, Hkv = 16, 8
    L = synth.ragged_prefix_lengths(8)
    cap = int(L.max()) + 256
    kc, vc = synth.cache(1105, L, cap, Hkv, D, "fp8")
    kc_d, vc_d = to_dev(kc), to_dev(vc)
    rng = np.random.default_rng(2)
    for s in range(2):
        q, kn, vn = synth.canvas(1105, 8, Hq, Hkv, D, "fp8", step=s)
        c = dict(L=L, kc=kc, vc=vc, q=q, kn=kn, vn=vn)
        rows = sample_rows(rng, 8, 256, Hq, 64)
        got = gpu_canvas(c)[rows[:, 0], rows[:, 1], rows[:, 2]]
        fp8_check(got, oracle_canvas(oracle_lib, c, rows), oracle_canvas(oracle_lib, c, rows, absv=True))
    qb, kb, vb = synth.block(1105, 8, Hq, Hkv, D, "fp8")
    out = dg.commit_block(to_dev(qb), to_dev(kb), to_dev(vb), kc_d, vc_d, L)
    torch.cuda.synchronize()
    rows = sample_rows(rng, 8, 256, Hq, 64)
    ref = oracle_lib.commit_attn(qb, kc, vc, L, kb, vb, rows=rows)
    ref_abs = oracle_lib.commit_attn(qb, kc, abs_bytes(vc), L, kb, abs_bytes(vb), rows=rows)
    fp8_check(to_host_f64(out)[rows[:, 0], rows[:, 1], rows[:, 2]], ref, ref_abs)
    oracle_lib.append_block(kb, vb, kc, vc, L)
    np.testing.assert_array_equal(to_host_bits(kc_d), kc)
    np.testing.assert_array_equal(to_host_bits(vc_d), vc)
