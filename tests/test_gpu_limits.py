"""GPU parity at the library's largest batch (DG_MAX_BATCH sequences) and, for
decode, the largest token count (DG_MAX_DECODE), and on caches whose addresses
pass 2^32 bytes, against the CPU fp64 oracle.

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


def test_cache_beyond_4gib(oracle_lib):
    """Caches of 2^21 rows (8 kv heads x 128 bf16): sequence 1 starts 4 GiB into each
    cache tensor, so its addresses lie past 2^32 bytes, in the canvas step, the commit
    with its append and a decode call after it.  Rows past the oracle's capacity are
    left uninitialised on the device: no kernel may read them."""
    B, Hq, Hkv, D, cap = 2, 16, 8, 128, 1 << 21
    L = np.array([700, 1234], np.int32)
    small = int(L.max()) + 256 + 16
    kc, vc = synth.cache(1306, L, small, Hkv, D, "bf16")
    big = []
    for a in (kc, vc):
        t = torch.empty((B, cap, Hkv, D), dtype=torch.bfloat16, device="cuda")
        t[:, :small] = to_dev(a)
        big.append(t)
    kc_d, vc_d = big

    def cached(t):
        return to_host_bits(t[:, :small].contiguous())

    q, kn, vn = synth.canvas(1306, B, Hq, Hkv, D, "bf16")
    out = dg.canvas_attn(to_dev(q), kc_d, vc_d, L, to_dev(kn), to_dev(vn))
    torch.cuda.synchronize()
    err = row_err(to_host_f64(out), oracle_lib.canvas_attn(q, kc, vc, L, kn, vn))
    assert err <= TOL_BF16, f"canvas step: per-row error {err:.3e}"

    qb, kb, vb = synth.block(1306, B, Hq, Hkv, D, "bf16")
    outc = dg.commit_block(to_dev(qb), to_dev(kb), to_dev(vb), kc_d, vc_d, L)
    torch.cuda.synchronize()
    err = row_err(to_host_f64(outc), oracle_lib.commit_attn(qb, kc, vc, L, kb, vb))
    assert err <= TOL_BF16, f"commit: per-row error {err:.3e}"
    oracle_lib.append_block(kb, vb, kc, vc, L)
    np.testing.assert_array_equal(cached(kc_d), kc)
    np.testing.assert_array_equal(cached(vc_d), vc)

    L2 = L + 256
    qd, knd, vnd = synth.decode(1306, B, 4, Hq, Hkv, D, "bf16")
    outd = dg.decode_attn(to_dev(qd), to_dev(knd), to_dev(vnd), kc_d, vc_d, L2)
    torch.cuda.synchronize()
    err = row_err(to_host_f64(outd), oracle_lib.decode_attn(qd, kc, vc, L2, knd, vnd))
    assert err <= TOL_BF16, f"decode: per-row error {err:.3e}"
    oracle_lib.append_block(knd, vnd, kc, vc, L2)
    np.testing.assert_array_equal(cached(kc_d), kc)
    np.testing.assert_array_equal(cached(vc_d), vc)
    del kc_d, vc_d, big
    torch.cuda.empty_cache()
