"""CPU oracle of the canvas sampler -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the GPU library.

What it computes follows "DiffusionGemma Technical Report" (paperfeed.app
summary), section "The mechanism: an AR model turned inside out", paragraph on
the sampler: at each denoising step the logits, divided by an annealed
temperature tau, give a per-position entropy; positions are accepted from the
lowest entropy upwards until a cumulative entropy budget b is used up; every
other position is re-noised to a uniformly random token; generation stops once
the mean canvas entropy is below a threshold and the argmax prediction is the
same as in the previous step.  Readings of the points the page leaves open:

  * entropy in nats of softmax(logits / tau): H = -sum_v q_v ln q_v;
  * the argmax is that of the logits (tau > 0 keeps the order); ties go to the
    lowest vocabulary index; an accepted position takes its argmax token;
  * positions are ordered by entropy, ties by position index, and the accepted
    set is the longest prefix of that order whose cumulative entropy is <= b
    (it may be empty);
  * the random tokens of re-noised positions are an input (drawn by the caller);
  * "stable across two steps": the argmax of every position equals the previous
    step's; without a previous step the canvas is not stable.

row_stats is fp64 (the definition, two passes per row).  select takes the
entropies it is given (float32, as the GPU computes them) and makes its
decisions in the GPU's precision: each entropy and the budget and threshold
count as integers q(x) = rint(x * 2^32) (2^-32 nats), so every cumulative sum
is exact and its order does not matter; the stop test compares the exact sum
with Nc * q(threshold).
"""
from __future__ import annotations

import numpy as np


def widen_bf16(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exact."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def row_entropy(logits_row: np.ndarray, tau: float) -> float:
    """Entropy (nats) of softmax(logits_row / tau) for one row of fp64 logits."""
    x = logits_row / float(tau)
    m = x.max()
    e = np.exp(x - m)
    z = e.sum()
    q = e / z
    lq = (x - m) - np.log(z)          # ln q, exact form (no log of a rounded q)
    # 0 ln 0 = 0: tokens with -inf logits (masked) have q = 0 and add nothing
    pos = q > 0
    return float(-(q[pos] * lq[pos]).sum())


def row_stats(logits: np.ndarray, tau: float):
    """Entropy (fp64, nats) and argmax (lowest index among equal maxima) of every
    row of bf16 logits [..., V] (uint16 bit patterns).  Returns (H, argmax) with
    the leading shape of logits."""
    lead = logits.shape[:-1]
    flat = logits.reshape(-1, logits.shape[-1])
    H = np.empty(flat.shape[0])
    am = np.empty(flat.shape[0], np.int64)
    for r in range(flat.shape[0]):
        x = widen_bf16(flat[r])
        H[r] = row_entropy(x, tau)
        am[r] = int(np.argmax(x))     # first occurrence of the maximum
    return H.reshape(lead), am.reshape(lead)


def q32(x) -> int:
    """A float32 value in integer units of 2^-32 (round to nearest even)."""
    return int(np.rint(np.float64(np.float32(x)) * 2.0 ** 32))


def select(entropy, argmax, noise_tokens, prev_argmax, budget, stop_entropy):
    """Acceptance, re-noising and the stop rule for one canvas per row of the
    inputs ([B, Nc] each; prev_argmax may be None).  Returns (tokens, accepted,
    stop) as int arrays [B, Nc], [B, Nc] (0/1) and [B] (0/1)."""
    H = np.asarray(entropy, np.float32)
    am = np.asarray(argmax, np.int64)
    noise = np.asarray(noise_tokens, np.int64)
    B, Nc = H.shape
    tokens = np.empty((B, Nc), np.int64)
    accepted = np.zeros((B, Nc), np.int64)
    stop = np.zeros(B, np.int64)
    qb, qt = q32(budget), q32(stop_entropy)
    for b in range(B):
        q = [q32(H[b, i]) for i in range(Nc)]
        order = sorted(range(Nc), key=lambda i: (float(H[b, i]), i))
        cum = 0
        for i in order:
            if cum + q[i] > qb:
                break
            cum += q[i]
            accepted[b, i] = 1
        tokens[b] = np.where(accepted[b] == 1, am[b], noise[b])
        stable = prev_argmax is not None and bool(np.all(am[b] == np.asarray(prev_argmax)[b]))
        stop[b] = int(sum(q) < Nc * qt and stable)
    return tokens, accepted, stop
