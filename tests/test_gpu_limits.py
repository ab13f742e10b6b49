"""GPU parity at the library's largest batch (DG_MAX_BATCH sequences) and, for
decode, the largest token count (DG_MAX_DECODE), against the CPU fp64 oracle.

Prefix lengths are ragged and include the degenerate ones: an empty cache, a
single row, and lengths on and just off the 32-key chunk boundary.  Every output
row is checked (per-row normalised max error 2e-2, bf16 storage with fp32
accumulation; the fp8 step on the gates of helpers.fp8_check), and the cache
append of the commit and of decode bit for bit.
"""
import numpy as np
import pytest

from canvas_attention_amd import synth
from helpers import TOL_BF16, row_err, to_dev, to_host_bits, to_host_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU machines skip the module
    pytest.skip("needs a GPU", allow_module_level=True)

import canvas_attention_amd.dg as dg  # noqa: E402  (loads libdg.so; raises if missing)

MAX_BATCH = 64   # DG_MAX_BATCH in include/dg.h
MAX_DECODE = 16  # DG_MAX_DECODE


def ragged_lengths(seed, B, hi):
    """B prefix lengths: the degenerate ones first, the rest uniform in [0, hi]."""
    fixed = [0, 1, 31, 32, 33, 255, 256, 257]
    rng = np.random.default_rng(seed)
    return np.asarray(fixed + list(rng.integers(0, hi + 1, size=B - len(fixed))), np.int32)


def test_canvas_step_max_batch(oracle_lib):
    B, Hq, Hkv, D = MAX_BATCH, 4, 2, 64
    L = ragged_lengths(1301, B, 700)
    cap = int(L.max()) + 256
    kc, vc = synth.cache(1301, L, cap, Hkv, D, "bf16")
    q, kn, vn = synth.canvas(1301, B, Hq, Hkv, D, "bf16")
    out = dg.canvas_attn(to_dev(q), to_dev(kc), to_dev(vc), L, to_dev(kn), to_dev(vn))
    torch.cuda.synchronize()
    err = row_err(to_host_f64(out), oracle_lib.canvas_attn(q, kc, vc, L, kn, vn))
    assert err <= TOL_BF16, f"per-row error {err:.3e}"
    print(f"canvas step, {B} sequences: {err:.3e}")


def test_commit_max_batch(oracle_lib):
    B, Hq, Hkv, D = MAX_BATCH, 4, 2, 64
    L = ragged_lengths(1302, B, 700)
    cap = int(L.max()) + 256 + 32
    kc, vc = synth.cache(1302, L, cap, Hkv, D, "bf16")
    qb, kb, vb = synth.block(1302, B, Hq, Hkv, D, "bf16")
    kc_d, vc_d = to_dev(kc), to_dev(vc)
    out = dg.commit_block(to_dev(qb), to_dev(kb), to_dev(vb), kc_d, vc_d, L)
    torch.cuda.synchronize()
    err = row_err(to_host_f64(out), oracle_lib.commit_attn(qb, kc, vc, L, kb, vb))
    assert err <= TOL_BF16, f"per-row error {err:.3e}"
    oracle_lib.append_block(kb, vb, kc, vc, L)
    np.testing.assert_array_equal(to_host_bits(kc_d), kc)
    np.testing.assert_array_equal(to_host_bits(vc_d), vc)
    print(f"commit, {B} sequences: {err:.3e}")


def test_decode_max_batch_max_tokens(oracle_lib):
    B, k, Hq, Hkv, D = MAX_BATCH, MAX_DECODE, 4, 2, 128
    L = ragged_lengths(1303, B, 3000)
    cap = int(L.max()) + k
    kc, vc = synth.cache(1303, L, cap, Hkv, D, "bf16")
    q, kn, vn = synth.decode(1303, B, k, Hq, Hkv, D, "bf16")
    kc_d, vc_d = to_dev(kc), to_dev(vc)
    out = dg.decode_attn(to_dev(q), to_dev(kn), to_dev(vn), kc_d, vc_d, L)
    torch.cuda.synchronize()
    err = row_err(to_host_f64(out), oracle_lib.decode_attn(q, kc, vc, L, kn, vn))
    assert err <= TOL_BF16, f"per-row error {err:.3e}"
    oracle_lib.append_block(kn, vn, kc, vc, L)
    np.testing.assert_array_equal(to_host_bits(kc_d), kc)
    np.testing.assert_array_equal(to_host_bits(vc_d), vc)
    print(f"decode, {B} sequences x {k} tokens: {err:.3e}")


def test_step_loop_max_batch(oracle_lib):
    """Three steps of dg_canvas_step_loop over 64 sequences, each step against the
    oracle on its own inputs."""
    B, Hq, Hkv, D, N = MAX_BATCH, 4, 2, 64, 3
    L = ragged_lengths(1304, B, 500)
    kc, vc = synth.cache(1304, L, int(L.max()) + 256, Hkv, D, "bf16")
    steps = [synth.canvas(1304, B, Hq, Hkv, D, "bf16", step=s) for s in range(N)]
    qs, ks, vs = (torch.stack([to_dev(st[i]) for st in steps]) for i in range(3))
    out = dg.canvas_step_loop(qs, ks, vs, to_dev(kc), to_dev(vc), L)
    torch.cuda.synchronize()
    for s, (q, kn, vn) in enumerate(steps):
        err = row_err(to_host_f64(out[s]), oracle_lib.canvas_attn(q, kc, vc, L, kn, vn))
        assert err <= TOL_BF16, f"step {s}: per-row error {err:.3e}"


def test_fp8_canvas_step_max_batch(oracle_lib):
    """The e4m3 canvas step over 64 sequences, on the fp8 gates."""
    from helpers import fp8_check
    B, Hq, Hkv, D = MAX_BATCH, 4, 2, 128
    L = ragged_lengths(1305, B, 700)
    kc, vc = synth.cache(1305, L, int(L.max()) + 256, Hkv, D, "fp8")
    q, kn, vn = synth.canvas(1305, B, Hq, Hkv, D, "fp8")
    out = dg.canvas_attn(to_dev(q), to_dev(kc), to_dev(vc), L, to_dev(kn), to_dev(vn))
    torch.cuda.synchronize()
    ref = oracle_lib.canvas_attn(q, kc, vc, L, kn, vn)
    absv = (lambda x: x & np.uint8(0x7F))
    ref_abs = oracle_lib.canvas_attn(q, kc, absv(vc), L, kn, absv(vn))
    fp8_check(to_host_f64(out), ref, ref_abs, per_row=True)
