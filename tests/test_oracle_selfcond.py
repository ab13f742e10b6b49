"""Pins of the self-conditioning oracle (oracle/selfcond.py; CPU only).

"DiffusionGemma Technical Report" (paperfeed.app summary), section "The
mechanism: an AR model turned inside out", self-conditioning paragraph:
z_t = FFW(p0_hat E).  Pinned by brute force on tiny inputs, closed forms (a
one-hot distribution selects one embedding row; a uniform one averages them), a
library special case (scipy's softmax), an independent definition of GELU (the
erf form, which the tanh form approximates to about 1e-3) and invariances of
the softmax (a shift of a logits row; a joint permutation of vocabulary and
embedding rows).
"""
import math

import numpy as np
import pytest

from canvas_attention_amd import synth
from oracle import selfcond

scipy_special = pytest.importorskip("scipy.special")


def bits(x):
    return synth.bf16_round(np.asarray(x, np.float32))


def test_softmax_matches_scipy():
    rng = np.random.default_rng(1)
    x = synth.bf16_to_f64(bits(3 * rng.standard_normal((5, 300))))
    np.testing.assert_allclose(selfcond.softmax_rows(x), scipy_special.softmax(x, axis=-1),
                               rtol=1e-13, atol=1e-16)


def test_one_hot_distribution_selects_one_embedding_row():
    V, d = 64, 16
    E, _, _ = synth.selfcond_weights(3, V, d, 8)
    logits = np.zeros((3, V), np.float32)
    for r, v in enumerate((0, 17, 63)):
        logits[r, v] = 1000.0   # every other weight is exp(-1000) = 0 in fp64
    y = selfcond.expected_embedding(bits(logits), E)
    np.testing.assert_array_equal(y, synth.bf16_to_f64(E[[0, 17, 63]]))


def test_uniform_distribution_averages_the_embedding_rows():
    V, d = 96, 8
    E, _, _ = synth.selfcond_weights(4, V, d, 8)
    y = selfcond.expected_embedding(bits(np.full((2, V), 1.5)), E, chunk=40)
    np.testing.assert_allclose(y, np.tile(synth.bf16_to_f64(E).mean(0), (2, 1)), rtol=0, atol=1e-14)


def test_gelu_tanh_against_the_erf_form():
    x = np.linspace(-6, 6, 2001)
    erf_form = 0.5 * x * (1 + scipy_special.erf(x / math.sqrt(2)))
    assert np.abs(selfcond.gelu_tanh(x) - erf_form).max() < 1e-3
    assert selfcond.gelu_tanh(np.array([0.0]))[0] == 0.0
    big = np.array([30.0, -30.0])
    np.testing.assert_allclose(selfcond.gelu_tanh(big), [30.0, 0.0], atol=1e-12)


def test_gelu_tanh_against_torch_tanh_gelu():
    """The tanh form against torch's own tanh-approximated GELU in float64 on the
    CPU: an independent implementation of the same formula, so a wrong constant
    (a digit swap in 0.044715 moves values by about 1e-5) fails at 1e-14."""
    torch = pytest.importorskip("torch")
    x = np.linspace(-8, 8, 4001)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    np.testing.assert_allclose(selfcond.gelu_tanh(x), ref, rtol=0, atol=1e-14)


def test_brute_force_tiny():
    """Every step written out with Python loops and math.exp / math.tanh."""
    M, V, d, h = 3, 7, 4, 5
    rng = np.random.default_rng(5)
    logits = bits(2 * rng.standard_normal((M, V)))
    E, w1, w2 = synth.selfcond_weights(6, V, d, h)
    x, Ef, W1, W2 = (synth.bf16_to_f64(a) for a in (logits, E, w1, w2))
    want = np.zeros((M, d))
    for r in range(M):
        ex = [math.exp(x[r, v]) for v in range(V)]
        p = [e / sum(ex) for e in ex]
        y = [sum(p[v] * Ef[v, j] for v in range(V)) for j in range(d)]
        a = [sum(y[j] * W1[j, k] for j in range(d)) for k in range(h)]
        g = [0.5 * t * (1 + math.tanh(math.sqrt(2 / math.pi) * (t + 0.044715 * t ** 3))) for t in a]
        for j in range(d):
            want[r, j] = sum(g[k] * W2[k, j] for k in range(h))
    np.testing.assert_allclose(selfcond.self_condition(logits, E, w1, w2), want, rtol=1e-12, atol=1e-14)


def test_shift_and_vocabulary_permutation_invariance():
    M, V, d, h = 4, 200, 16, 12
    rng = np.random.default_rng(7)
    x = np.round(4 * rng.standard_normal((M, V))).astype(np.float32)  # integers: exact in bf16
    E, w1, w2 = synth.selfcond_weights(8, V, d, h)
    z = selfcond.self_condition(bits(x), E, w1, w2)
    np.testing.assert_allclose(selfcond.self_condition(bits(x + 16.0), E, w1, w2), z,
                               rtol=1e-12, atol=1e-13)
    perm = rng.permutation(V)
    np.testing.assert_allclose(selfcond.self_condition(bits(x[:, perm]), E[perm], w1, w2), z,
                               rtol=1e-12, atol=1e-13)


def test_row_subset_matches_full():
    M, V, d, h = 6, 300, 8, 8
    rng = np.random.default_rng(9)
    logits = bits(rng.standard_normal((M, V)))
    E, w1, w2 = synth.selfcond_weights(10, V, d, h)
    full = selfcond.self_condition(logits, E, w1, w2)
    np.testing.assert_allclose(selfcond.self_condition(logits, E, w1, w2, rows=[4, 1]), full[[4, 1]],
                               rtol=1e-13, atol=1e-15)
