"""GPU parity of decode attention (dg_decode_attn) against the CPU fp64 oracle.

AR mode ("DiffusionGemma Technical Report", paperfeed.app summary, section "The
numbers, honestly"): 1..16 new tokens per sequence attend causally to the cache
and to each other, and their K/V rows are appended to the cache.  Gates as for
the other entry points: per-row normalised max error 2e-2 for bf16 storage with
fp32 accumulation and 1e-5 for fp32; the fp8 gates of helpers.fp8_check; the
cache append bit for bit.
"""
import os

import numpy as np
import pytest

from canvas_attention_amd import synth
from helpers import TOL_BF16, TOL_F32, fp8_check, row_err, to_dev, to_host_bits, to_host_f64

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


def make(seed, B, L, k, Hq, Hkv, D, dtype, cap=None, step=0):
    L = np.asarray(L, np.int32)
    cap = cap or int(L.max()) + k
    kc, vc = synth.cache(seed, L, cap, Hkv, D, dtype)
    q, kn, vn = synth.decode(seed, B, k, Hq, Hkv, D, dtype, step=step)
    return dict(L=L, kc=kc, vc=vc, q=q, kn=kn, vn=vn)


def gpu_decode(c, ts=None, caches=None):
    kc_d, vc_d = caches if caches is not None else (to_dev(c["kc"]), to_dev(c["vc"]))
    out = dg.decode_attn(to_dev(c["q"]), to_dev(c["kn"]), to_dev(c["vn"]), kc_d, vc_d, c["L"],
                         tensor_scales=ts)
    torch.cuda.synchronize()
    return to_host_f64(out), kc_d, vc_d


def oracle_decode(o, c, ts=None, absv=False):
    f = (lambda x: x & np.uint8(0x7F)) if absv else (lambda x: x)
    return o.decode_attn(c["q"], c["kc"], f(c["vc"]), c["L"], c["kn"], f(c["vn"]),
                         tensor_scales=ts)


def check_append(o, c, kc_d, vc_d):
    kc, vc = c["kc"].copy(), c["vc"].copy()
    o.append_block(c["kn"], c["vn"], kc, vc, c["L"])
    assert np.array_equal(to_host_bits(kc_d), kc), "cache K after the append"
    assert np.array_equal(to_host_bits(vc_d), vc), "cache V after the append"


def check_bf16(o, c, tol=TOL_BF16):
    got, kc_d, vc_d = gpu_decode(c)
    err = row_err(got, oracle_decode(o, c))
    assert err <= tol, f"per-row error {err:.3e} > {tol}"
    check_append(o, c, kc_d, vc_d)
    return err


@pytest.mark.parametrize("B,L,k,Hq,Hkv,D,forced", [
    (1, [8192], 1, 16, 8, 128, None),    # AR decode at the block-cycle prefix
    (1, [8192], 16, 16, 8, 128, None),   # 16 drafted tokens
    (1, [2053], 7, 16, 8, 128, 96),      # ragged splits, cache/new seam inside a chunk
    (2, [0, 5], 1, 16, 8, 128, None),    # empty and tiny prefixes
    (1, [0], 16, 16, 8, 128, 32),        # splits inside the new rows
    (3, [1000, 4097, 31], 5, 32, 4, 64, None),  # G = 8, two row tiles, head_dim 64
    (1, [300], 16, 32, 4, 128, 96),      # four row tiles
    (2, [777, 64], 3, 4, 2, 64, 64),     # the tiny workload's heads
    (1, [1], 16, 64, 1, 128, None),      # one kv head for 64 query heads: 32 row tiles
])
def test_decode_bf16(oracle_lib, split_keys, B, L, k, Hq, Hkv, D, forced):
    split_keys(forced)
    err = check_bf16(oracle_lib, make(1200 + k, B, L, k, Hq, Hkv, D, "bf16"))
    print(f"decode bf16 B={B} L={L} k={k} Hq={Hq} Hkv={Hkv} D={D} forced={forced}: {err:.3e}")


def test_decode_ragged_batch(oracle_lib, split_keys):
    """Eight sequences with prefixes uniform in [1024, 32768], one token each."""
    split_keys(None)
    L = synth.ragged_prefix_lengths(8)
    err = check_bf16(oracle_lib, make(1210, 8, L, 1, 16, 8, 128, "bf16"))
    print(f"decode ragged b8: {err:.3e}")


def test_decode_concurrent_b32_l8k(oracle_lib, split_keys):
    """32 concurrent sequences at L=8192, one token each (every row checked)."""
    split_keys(None)
    err = check_bf16(oracle_lib, make(1211, 32, [8192] * 32, 1, 16, 8, 128, "bf16"))
    print(f"decode b32 L=8192: {err:.3e}")


@pytest.mark.parametrize("k", [1, 4])
def test_decode_long_context(oracle_lib, split_keys, k):
    split_keys(None)
    err = check_bf16(oracle_lib, make(1212, 1, [131072], k, 16, 8, 128, "bf16"))
    print(f"decode L=131072 k={k}: {err:.3e}")


def test_decode_hybrid_equals_token_by_token(oracle_lib, split_keys):
    """Eight drafted tokens in one call and eight single-token calls (prefix advanced
    by one after each) both match the oracle and leave the same cache."""
    split_keys(None)
    k = 8
    c = make(1213, 2, [3000, 515], k, 16, 8, 128, "bf16")
    ref = oracle_decode(oracle_lib, c)
    once, kc1, vc1 = gpu_decode(c)
    assert row_err(once, ref) <= TOL_BF16
    kc2, vc2 = to_dev(c["kc"]), to_dev(c["vc"])
    steps = np.zeros_like(once)
    for i in range(k):
        ci = dict(L=c["L"] + i, kc=None, vc=None, q=c["q"][:, i:i + 1].copy(),
                  kn=c["kn"][:, i:i + 1].copy(), vn=c["vn"][:, i:i + 1].copy())
        steps[:, i:i + 1] = gpu_decode(ci, caches=(kc2, vc2))[0]
    assert row_err(steps, ref) <= TOL_BF16
    assert torch.equal(kc1, kc2) and torch.equal(vc1, vc2)


def test_decode_rising_scores_exercise_rescale(oracle_lib, split_keys):
    """Key magnitudes growing along the cache: the lazy reference max is raised again
    and again inside every wave's stream."""
    split_keys(None)
    c = make(1214, 1, [6000], 4, 16, 8, 128, "bf16")
    rng = np.random.default_rng(6)
    f = rng.standard_normal(c["kc"].shape).astype(np.float32)
    ramp = np.linspace(0.2, 30.0, f.shape[1], dtype=np.float32)[None, :, None, None]
    c["kc"] = synth.bf16_round(f * ramp)
    err = check_bf16(oracle_lib, c)
    print(f"decode rising scores: {err:.3e}")


@pytest.mark.parametrize("k,forced", [(1, None), (3, 32), (16, 64), (16, None)])
def test_decode_fp32(oracle_lib, split_keys, k, forced):
    """fp32 storage and arithmetic at the tiny workload's heads (Hq=4, Hkv=2, D=64)."""
    split_keys(forced)
    c = make(1215, 1, [64], k, 4, 2, 64, "f32")
    got, kc_d, vc_d = gpu_decode(c)
    err = row_err(got, oracle_decode(oracle_lib, c))
    assert err <= TOL_F32, f"per-row error {err:.3e} > {TOL_F32}"
    check_append(oracle_lib, c, kc_d, vc_d)


@pytest.mark.parametrize("B,L,k,forced,ts", [
    (1, [8192], 1, None, None),
    (1, [2048], 16, 128, None),
    (2, [700, 300], 3, None, (0.5, 1.75, 3.0)),
    (1, [131072], 1, None, None),
])
def test_decode_fp8(oracle_lib, split_keys, B, L, k, forced, ts):
    split_keys(forced)
    c = make(1216 + k, B, L, k, 16, 8, 128, "fp8")
    got, kc_d, vc_d = gpu_decode(c, ts=ts)
    ref = oracle_decode(oracle_lib, c, ts=ts)
    ref_abs = oracle_decode(oracle_lib, c, ts=ts, absv=True)
    rerr, rms = fp8_check(got, ref, ref_abs)
    check_append(oracle_lib, c, kc_d, vc_d)
    print(f"decode fp8 B={B} L={L} k={k}: row {rerr:.3e} rms {rms:.3e}")


def test_decode_determinism(split_keys):
    split_keys(None)
    c = make(1217, 4, [9000, 100, 4096, 20000], 2, 16, 8, 128, "bf16")
    a = gpu_decode(c)[0]
    b = gpu_decode(c)[0]
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("Hq,Hkv,k,L,forced", [
    (32, 4, 16, [2500], 128),   # fp8, G = 8: four row tiles, splits of two chunks
    (16, 8, 9, [0, 300], None),
])
def test_decode_fp8_gqa(oracle_lib, split_keys, Hq, Hkv, k, L, forced):
    split_keys(forced)
    c = make(1230 + k, len(L), L, k, Hq, Hkv, 128, "fp8")
    got, kc_d, vc_d = gpu_decode(c)
    ref = oracle_decode(oracle_lib, c)
    ref_abs = oracle_decode(oracle_lib, c, absv=True)
    # rows with fewer than 256 visible keys are outside the per-row statistical gate
    fp8_check(got, ref, ref_abs, per_row=min(L) >= 256)
    check_append(oracle_lib, c, kc_d, vc_d)


def test_decode_bf16_d64_gqa4(oracle_lib, split_keys):
    split_keys(64)
    check_bf16(oracle_lib, make(1240, 2, [1500, 63], 16, 16, 4, 64, "bf16"))


def test_decode_shared_workspace(oracle_lib, split_keys):
    """One workspace, sized for the largest of the calls, serves a run of decode calls
    of different token counts, prefixes, split sizes and element types, each checked
    against the oracle (nothing of one call's partials leaks into the next)."""
    split_keys(None)
    Hq, Hkv, D = 16, 8, 128
    cases = [(1251, [8192], 1, "bf16", None), (1252, [8192], 16, "bf16", None),
             (1253, [40000], 1, "bf16", None), (1254, [8192], 1, "fp8", None),
             (1255, [3000], 2, "bf16", 64), (1256, [8192], 1, "bf16", None)]
    tdt = {"bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}
    n = 0
    for _, L, k, dt, forced in cases:  # the forced split size is part of the size query
        split_keys(forced)
        n = max(n, dg.decode_workspace_bytes(1, k, Hq, Hkv, D, L[0], tdt[dt]))
    ws = torch.full((n,), 0x7F, dtype=torch.uint8, device="cuda")
    for seed, L, k, dt, forced in cases:
        split_keys(forced)
        c = make(seed, 1, L, k, Hq, Hkv, D, dt)
        kc_d, vc_d = to_dev(c["kc"]), to_dev(c["vc"])
        out = dg.decode_attn(to_dev(c["q"]), to_dev(c["kn"]), to_dev(c["vn"]), kc_d, vc_d, c["L"],
                             workspace=ws)
        torch.cuda.synchronize()
        got, ref = to_host_f64(out), oracle_decode(oracle_lib, c)
        if dt == "bf16":
            err = row_err(got, ref)
            assert err <= TOL_BF16, f"seed {seed}: per-row error {err:.3e}"
        else:
            fp8_check(got, ref, oracle_decode(oracle_lib, c, absv=True), per_row=True)
        check_append(oracle_lib, c, kc_d, vc_d)
