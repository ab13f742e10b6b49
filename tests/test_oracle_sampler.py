"""Pins of the canvas sampler oracle (oracle/sampler.py) against things other than
itself (CPU only): closed forms of the entropy, scipy's entropy routine, argmax
tie order, and hand-derived selection cases in tests/golden/sampler_cases.json.

The sampler follows "DiffusionGemma Technical Report" (paperfeed.app summary),
section "The mechanism: an AR model turned inside out", sampler paragraph."""
import json
import math
import os

import numpy as np
import pytest

from canvas_attention_amd import synth
from oracle import sampler

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sampler_cases.json")


def bf16(x):
    return synth.bf16_round(np.asarray(x, np.float32))


@pytest.mark.parametrize("V", [8, 1000, 262144])
def test_uniform_row_entropy_is_log_v(V):
    row = bf16(np.full((1, V), 1.5))
    H, am = sampler.row_stats(row, 0.7)
    assert abs(H[0] - math.log(V)) < 1e-12
    assert am[0] == 0


@pytest.mark.parametrize("k,a,b,tau", [(1, 4.0, 0.0, 0.8), (3, 2.5, -1.0, 0.4), (7, 0.5, 0.25, 1.0)])
def test_two_level_closed_form(k, a, b, tau):
    """k tokens at logit a, V-k at b: q_a = e^(a/tau) / (k e^(a/tau) + (V-k) e^(b/tau))."""
    V = 4096
    x = np.full(V, b, np.float32)
    x[np.random.default_rng(k).choice(V, k, replace=False)] = a
    H, _ = sampler.row_stats(bf16(x)[None], tau)
    ea, eb = math.exp(a / tau), math.exp(b / tau)
    zz = k * ea + (V - k) * eb
    qa, qb = ea / zz, eb / zz
    want = -(k * qa * math.log(qa) + (V - k) * qb * math.log(qb))
    assert abs(H[0] - want) < 1e-10 * max(1.0, want)


def test_matches_scipy_entropy():
    scipy_stats = pytest.importorskip("scipy.stats")
    rng = np.random.default_rng(1)
    rows = bf16(rng.standard_normal((6, 5000)) * np.array([0.1, 1, 3, 10, 30, 100])[:, None])
    for tau in (0.4, 0.8):
        H, am = sampler.row_stats(rows, tau)
        x = sampler.widen_bf16(rows) / tau
        p = np.exp(x - x.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        want = scipy_stats.entropy(p, axis=1)
        np.testing.assert_allclose(H, want, rtol=1e-10, atol=1e-13)
        np.testing.assert_array_equal(am, np.argmax(sampler.widen_bf16(rows), axis=1))


def test_argmax_ties_and_permutation():
    x = np.zeros(64, np.float32)
    x[[9, 40, 17]] = 3.0
    H, am = sampler.row_stats(bf16(x)[None], 0.5)
    assert am[0] == 9
    perm = np.random.default_rng(2).permutation(64)
    H2, _ = sampler.row_stats(bf16(x[perm])[None], 0.5)
    assert abs(H[0] - H2[0]) < 1e-14


def test_temperature_lowers_entropy():
    rng = np.random.default_rng(3)
    row = bf16(rng.standard_normal((1, 2048)) * 2)
    hs = [sampler.row_stats(row, t)[0][0] for t in (1.0, 0.8, 0.6, 0.4)]
    assert all(a > b for a, b in zip(hs, hs[1:]))
    assert hs[0] < math.log(2048)


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_selection_hand_cases(case):
    tokens, acc, stop = sampler.select(case["entropy"], case["argmax"], case["noise"],
                                       case["prev_argmax"], case["budget"], case["stop_entropy"])
    np.testing.assert_array_equal(tokens, case["tokens"])
    np.testing.assert_array_equal(acc, case["accepted"])
    np.testing.assert_array_equal(stop, case["stop"])


def test_selection_is_the_longest_prefix():
    """On random entropies: the accepted set is a prefix of the (entropy, index)
    order, within the budget, and the next position would not fit."""
    rng = np.random.default_rng(4)
    H = (rng.exponential(0.02, (3, 256))).astype(np.float32)
    am = rng.integers(0, 1000, (3, 256))
    noise = rng.integers(0, 1000, (3, 256))
    tokens, acc, stop = sampler.select(H, am, noise, None, 0.1, 0.005)
    for b in range(3):
        order = sorted(range(256), key=lambda i: (float(H[b, i]), i))
        n = int(acc[b].sum())
        assert all(acc[b, i] == 1 for i in order[:n]) and all(acc[b, i] == 0 for i in order[n:])
        assert float(np.sum(H[b, order[:n]], dtype=np.float64)) <= 0.1 + 1e-6
        if n < 256:
            assert float(np.sum(H[b, order[:n + 1]], dtype=np.float64)) > 0.1 - 1e-6
        np.testing.assert_array_equal(tokens[b], np.where(acc[b] == 1, am[b], noise[b]))
    assert not stop.any()


def test_masked_tokens_drop_out():
    """-inf logits (masked tokens) carry q = 0: the entropy and argmax equal those
    of the row without them."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(3000) * 2).astype(np.float32)
    keep = rng.random(3000) < 0.7
    masked = np.where(keep, x, -np.inf).astype(np.float32)
    H1, am1 = sampler.row_stats(bf16(masked)[None], 0.6)
    H2, am2 = sampler.row_stats(bf16(x[keep])[None], 0.6)
    assert abs(H1[0] - H2[0]) < 1e-12
    assert np.flatnonzero(keep)[am2[0]] == am1[0]
