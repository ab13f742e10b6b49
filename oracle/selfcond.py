"""CPU oracle of the self-conditioning input -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py`` may import this
module.  It shares no code with the GPU library.

What it computes follows "DiffusionGemma Technical Report" (paperfeed.app
summary), section "The mechanism: an AR model turned inside out", paragraph on
self-conditioning: besides the noisy canvas, the decoder receives
z_t = FFW(p0_hat E), the previous step's predicted token distribution p0_hat
multiplied by the embedding matrix E and passed through a small MLP of about
7.8M parameters.  Readings of what the page leaves open:

  * p0_hat is the model's predicted distribution, softmax of the previous step's
    logits at temperature 1 (the annealed temperature belongs to the sampler);
  * E is the [V, d] embedding table, so p0_hat E is the expected embedding;
  * FFW is a two-layer perceptron without biases, d -> h -> d, with the tanh form
    of GELU between the layers: FFW(y) = gelu(y W1) W2, W1 [d, h], W2 [h, d].

Everything here is float64: the logits are widened exactly from their bf16
bits; E, W1 and W2 are taken as given (their bf16 values widened exactly).
Nothing is rounded between the steps.
"""
from __future__ import annotations

import math

import numpy as np


def widen_bf16(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exact."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def softmax_rows(x: np.ndarray) -> np.ndarray:
    """Softmax over the last axis of float64 rows (max-shifted)."""
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """GELU in its tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def expected_embedding(logits, embed, rows=None, chunk=16384):
    """y = softmax(logits) E for logits [M, V] (bf16 bits) and E [V, d] (bf16 bits
    or float), optionally only for the row indices in `rows`.  The product runs
    over the vocabulary in chunks of `chunk` rows of E (a library matmul per
    chunk; only memory, not the arithmetic, is split)."""
    x = widen_bf16(logits)
    if rows is not None:
        x = x[np.asarray(rows)]
    p = softmax_rows(x)
    V = x.shape[-1]
    y = np.zeros((x.shape[0], embed.shape[1]))
    for v0 in range(0, V, chunk):
        e = embed[v0:v0 + chunk]
        e = widen_bf16(e) if e.dtype == np.uint16 else e.astype(np.float64)
        y += p[:, v0:v0 + chunk] @ e
    return y


def ffw(y, w1, w2):
    """The MLP: gelu(y W1) W2 (weights as bf16 bits or floats)."""
    w1 = widen_bf16(w1) if w1.dtype == np.uint16 else np.asarray(w1, np.float64)
    w2 = widen_bf16(w2) if w2.dtype == np.uint16 else np.asarray(w2, np.float64)
    return gelu_tanh(y @ w1) @ w2


def self_condition(logits, embed, w1, w2, rows=None):
    """z = FFW(softmax(logits) E) for logits [M, V]; returns float64 [M or len(rows), d]."""
    return ffw(expected_embedding(logits, embed, rows), w1, w2)
