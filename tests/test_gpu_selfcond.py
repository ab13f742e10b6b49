"""GPU parity of the self-conditioning input (dg_self_condition) against the CPU
oracle (oracle/selfcond.py).

"DiffusionGemma Technical Report" (paperfeed.app summary), section "The
mechanism: an AR model turned inside out", self-conditioning paragraph:
z = FFW(p0_hat E), p0_hat = softmax(logits), FFW(y) = gelu(y W1) W2.

Gate: per-row normalised max error (helpers.row_err) 2e-2, the bf16 gate.  The
kernel rounds p0_hat, y and gelu(y W1) to bf16 before the product that consumes
each (relative 2^-9 per element, independent between elements) and accumulates
in fp32; a row of z carries a few such roundings, about 1e-3 relative to its
largest element.
"""
import numpy as np
import pytest

from canvas_attention_amd import synth
from helpers import TOL_BF16, row_err, to_dev, to_host_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU machines skip the module
    pytest.skip("needs a GPU", allow_module_level=True)

import canvas_attention_amd.dg as dg  # noqa: E402  (loads libdg.so; raises if missing)
from oracle import selfcond  # noqa: E402


def make(seed, B, V, d, h):
    lg = synth.sampler_logits(seed, B, vocab=V)
    E, w1, w2 = synth.selfcond_weights(seed, V, d, h)
    return lg, E, w1, w2


def gpu(lg, E, w1, w2):
    z = dg.self_condition(to_dev(lg), to_dev(E), to_dev(w1), to_dev(w2))
    torch.cuda.synchronize()
    return to_host_f64(z)


def check(lg, E, w1, w2, rows=None):
    B, nc, V = lg.shape
    flat = lg.reshape(B * nc, V)
    got = gpu(lg, E, w1, w2).reshape(B * nc, -1)
    if rows is not None:
        got = got[rows]
    ref = selfcond.self_condition(flat, E, w1, w2, rows=rows)
    err = row_err(got, ref)
    assert err <= TOL_BF16, f"per-row error {err:.3e} > {TOL_BF16}"
    return err


@pytest.mark.parametrize("B,V,d,h", [
    (1, 4096, 256, 128),          # one partial vocabulary split, 256-wide tiles
    (2, 16384 + 96, 512, 384),    # ragged last split, two row tiles
    (1, 8192, 256, 640),
])
def test_selfcond_small(oracle_lib, B, V, d, h):
    err = check(*make(1400 + d, B, V, d, h))
    print(f"selfcond B={B} V={V} d={d} h={h}: {err:.3e}")


def test_selfcond_full_vocab_sampled(oracle_lib):
    """The 262144-token vocabulary, d=2048, h=1920 (the bench shape); 24 rows."""
    lg, E, w1, w2 = make(1410, 1, synth.VOCAB, 2048, 1920)
    rows = np.array(sorted({0, 255, *np.random.default_rng(3).integers(0, 256, 22).tolist()}))
    err = check(lg, E, w1, w2, rows=rows)
    print(f"selfcond V=262144 d=2048 h=1920 sampled: {err:.3e}")


def test_selfcond_masked_logits(oracle_lib):
    """-inf logits: scattered, and a whole vocabulary split of one row."""
    V = 8192 * 3
    lg, E, w1, w2 = make(1411, 1, V, 256, 256)
    x = synth.bf16_to_f32(lg)
    rng = np.random.default_rng(4)
    x[rng.random(x.shape) < 0.2] = -np.inf
    x[0, 7, 8192:16384] = -np.inf
    x[0, 9, :8192] = -np.inf
    lg = synth.bf16_round(x)
    check(lg, E, w1, w2)


def test_selfcond_determinism():
    lg, E, w1, w2 = make(1412, 1, 16384, 256, 256)
    a = gpu(lg, E, w1, w2)
    b = gpu(lg, E, w1, w2)
    np.testing.assert_array_equal(a, b)


def test_selfcond_largest_vocabulary(oracle_lib):
    """V = 524288, the largest vocabulary the library takes: 64 vocabulary splits,
    every one merged by the weighted split sum."""
    V = 524288
    lg, E, w1, w2 = make(1413, 1, V, 256, 128)
    rows = np.array([0, 1, 77, 128, 200, 255])
    err = check(lg, E, w1, w2, rows=rows)
    print(f"selfcond V=524288: {err:.3e}")


def test_selfcond_batch4(oracle_lib):
    """Four canvases (1024 rows, four row tiles of the products)."""
    err = check(*make(1414, 4, 8192, 256, 256))
    print(f"selfcond B=4: {err:.3e}")
