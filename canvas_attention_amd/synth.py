"""Seeded synthetic inputs for canvas denoising attention.

This module only draws numbers and stores them; it holds none of the
attention arithmetic.  Both the GPU path (through the benchmark and the tests)
and the CPU oracle consume exactly the arrays produced here.

Recipe (the same for every workload):
  * generator: ``numpy.random.default_rng([seed, tensor_id, seq, block, step])``
    with one seed per workload and tensor ids 0/1 cache K/V, 2/3/4 canvas Q/K/V,
    5/6/7 commit (block) Q/K/V, 11/12/13 decode Q/K/V, 14/15/16 the
    self-conditioning embedding table and MLP weights;
  * values: ``standard_normal`` drawn in float32, stored as bf16 by rounding to
    nearest-even (fp32 workloads keep the float32 values; fp8 workloads store
    OCP e4m3 bytes, rounded to nearest-even, with tensor scales of 1);
  * layout: row-major [B, rows, heads, head_dim]; each sequence is drawn with its
    own ``seq`` index, so a sequence's data does not depend on the batch size.

The workloads mirror the shapes of the method's decode loop ("DiffusionGemma
Technical Report", paperfeed.app summary, sections "The mechanism: an AR model
turned inside out" and "The numbers, honestly"): a 256-position canvas, a
causal cache of prompt plus committed text, ~12 refinement passes per block,
then a causal commit that appends the block.
"""
from __future__ import annotations

import numpy as np

N_CANVAS = 256

T_CACHE_K, T_CACHE_V, T_Q, T_K, T_V, T_QB, T_KB, T_VB = range(8)
T_LOGITS, T_NOISE, T_PEAK = 8, 9, 10   # canvas sampler inputs
T_QD, T_KD, T_VD = 11, 12, 13          # decode Q/K/V of the new tokens
T_EMB, T_W1, T_W2 = 14, 15, 16          # self-conditioning weights (embedding table, MLP)

VOCAB = 262144  # vocabulary of the sampled model family ("262k vocabulary")

# Workloads, named by what they are.  "steps": canvas steps per block,
# "blocks": consecutive blocks (each = steps + one commit).
WORKLOADS = {
    "tiny_fp32_l64": dict(dtype="f32", batch=1, prefix=[64], hq=4, hkv=2, d=64, seed=1001,
                          steps=1, blocks=1, commit=True),
    "step_l2k": dict(dtype="bf16", batch=1, prefix=[2048], hq=16, hkv=8, d=128, seed=1002,
                     steps=1, blocks=1, commit=False),
    "cycle_l8k": dict(dtype="bf16", batch=1, prefix=[8192], hq=16, hkv=8, d=128, seed=1003,
                      steps=12, blocks=1, commit=True),
    "long_l128k": dict(dtype="bf16", batch=1, prefix=[131072], hq=16, hkv=8, d=128, seed=1004,
                       steps=1, blocks=1, commit=False),
    "ragged_b8": dict(dtype="bf16", batch=8, prefix=None, hq=16, hkv=8, d=128, seed=1005,
                      steps=12, blocks=4, commit=True),
}


def ragged_prefix_lengths(batch: int = 8) -> np.ndarray:
    """Prefix lengths of the ragged batch: uniform integers in [1024, 32768]."""
    return np.random.default_rng([1005, 99]).integers(1024, 32768, endpoint=True,
                                                      size=batch).astype(np.int32)


def prefix_lengths(name: str) -> np.ndarray:
    w = WORKLOADS[name]
    if w["prefix"] is None:
        return ragged_prefix_lengths(w["batch"])
    return np.asarray(w["prefix"], dtype=np.int32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP e4m3 bytes (uint8): round to nearest, ties to even; finite
    magnitudes beyond the largest value 448 (and infinities) saturate to it, NaN
    becomes 0x7f.

    Within binade [2^e, 2^(e+1)), e >= -6, the representable magnitudes are
    q * 2^(e-3) with q = 8..16, and their byte is 8 * (e + 6) + q (below 2^-6 the
    subnormals m * 2^-9 follow the same rule with e = -6, q = m), so rounding
    a / 2^(e-3) to the nearest even integer rounds the byte the same way."""
    x = np.ascontiguousarray(x, dtype=np.float32).astype(np.float64)
    nan = np.isnan(x)
    a = np.minimum(np.abs(np.where(nan, 0.0, x)), 448.0)
    _, ex = np.frexp(np.maximum(a, 2.0 ** -6))  # a = f * 2^ex, f in [0.5, 1)
    e = np.minimum(ex - 1, 8)
    q = np.rint(a / np.exp2(e - 3))             # exact division; rint ties to even
    code = (8 * (e + 6) + q).astype(np.uint8)
    code |= np.signbit(x).astype(np.uint8) << 7
    code[nan] = 0x7F
    return code


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact."""
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_to_f64(u: np.ndarray) -> np.ndarray:
    return bf16_to_f32(u).astype(np.float64)


def draw(seed: int, tensor_id: int, shape, dtype: str, seq: int = 0, block: int = 0,
         step: int = 0) -> np.ndarray:
    """One tensor of N(0,1) values: uint16 bf16 bits for "bf16", uint8 e4m3 bits
    for "fp8", float32 for "f32"."""
    rng = np.random.default_rng([seed, tensor_id, seq, block, step])
    x = rng.standard_normal(size=tuple(shape), dtype=np.float32)
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "fp8":
        return e4m3_round(x)
    return x


def _storage(dtype: str):
    return {"bf16": np.uint16, "fp8": np.uint8}.get(dtype, np.float32)


def batched(seed: int, tensor_id: int, batch: int, rows: int, heads: int, d: int, dtype: str,
            block: int = 0, step: int = 0) -> np.ndarray:
    """[batch, rows, heads, d], sequence b drawn with seq = b."""
    out = np.empty((batch, rows, heads, d), _storage(dtype))
    for b in range(batch):
        out[b] = draw(seed, tensor_id, (rows, heads, d), dtype, seq=b, block=block, step=step)
    return out


def cache(seed: int, prefix: np.ndarray, capacity: int, hkv: int, d: int, dtype: str):
    """Cache K and V [B, capacity, Hkv, D]: rows < prefix[b] drawn, the rest zero."""
    batch = len(prefix)
    k = np.zeros((batch, capacity, hkv, d), _storage(dtype))
    v = np.zeros((batch, capacity, hkv, d), _storage(dtype))
    for b in range(batch):
        L = int(prefix[b])
        k[b, :L] = draw(seed, T_CACHE_K, (L, hkv, d), dtype, seq=b)
        v[b, :L] = draw(seed, T_CACHE_V, (L, hkv, d), dtype, seq=b)
    return k, v


def canvas(seed: int, batch: int, hq: int, hkv: int, d: int, dtype: str, block: int = 0,
           step: int = 0):
    """Canvas Q [B,256,Hq,D] and K, V [B,256,Hkv,D] for one step of one block."""
    q = batched(seed, T_Q, batch, N_CANVAS, hq, d, dtype, block, step)
    k = batched(seed, T_K, batch, N_CANVAS, hkv, d, dtype, block, step)
    v = batched(seed, T_V, batch, N_CANVAS, hkv, d, dtype, block, step)
    return q, k, v


def block(seed: int, batch: int, hq: int, hkv: int, d: int, dtype: str, block: int = 0):
    """Commit inputs: block Q [B,256,Hq,D] and K, V [B,256,Hkv,D]."""
    q = batched(seed, T_QB, batch, N_CANVAS, hq, d, dtype, block)
    k = batched(seed, T_KB, batch, N_CANVAS, hkv, d, dtype, block)
    v = batched(seed, T_VB, batch, N_CANVAS, hkv, d, dtype, block)
    return q, k, v


def decode(seed: int, batch: int, n_new: int, hq: int, hkv: int, d: int, dtype: str,
           step: int = 0):
    """Decode inputs of n_new tokens per sequence: Q [B,n_new,Hq,D] and K, V
    [B,n_new,Hkv,D]; `step` numbers successive decode calls."""
    q = batched(seed, T_QD, batch, n_new, hq, d, dtype, 0, step)
    k = batched(seed, T_KD, batch, n_new, hkv, d, dtype, 0, step)
    v = batched(seed, T_VD, batch, n_new, hkv, d, dtype, 0, step)
    return q, k, v


def selfcond_weights(seed: int, vocab: int, d: int, h: int):
    """Synthetic self-conditioning weights as bf16 bits: the embedding table E
    [V, d] ~ N(0, 1), and the MLP's W1 [d, h] ~ N(0, 1/d) and W2 [h, d] ~ N(0, 1/h)
    (unit-variance activations through both layers).  E is drawn in slabs of 8192
    rows so that memory stays bounded at large vocabularies."""
    E = np.empty((vocab, d), np.uint16)
    for v0 in range(0, vocab, 8192):
        rng = np.random.default_rng([seed, T_EMB, v0 // 8192])
        n = min(8192, vocab - v0)
        E[v0:v0 + n] = bf16_round(rng.standard_normal((n, d), dtype=np.float32))
    w1 = bf16_round(np.random.default_rng([seed, T_W1]).standard_normal((d, h), dtype=np.float32)
                    / np.float32(np.sqrt(d)))
    w2 = bf16_round(np.random.default_rng([seed, T_W2]).standard_normal((h, d), dtype=np.float32)
                    / np.float32(np.sqrt(h)))
    return E, w1, w2


def sampler_logits(seed: int, batch: int, vocab: int = VOCAB, step: int = 0) -> np.ndarray:
    """bf16 logits [B, 256, V] of one denoising step, for the canvas sampler.

    Every position gets N(0,1) logits plus, at one uniformly drawn token, a peak
    whose height is uniform in [0, 24]: from near-uniform positions (entropy
    close to ln V) to near-certain ones (entropy near 0), as in a canvas that is
    partly resolved."""
    out = np.empty((batch, N_CANVAS, vocab), np.uint16)
    for b in range(batch):
        rng = np.random.default_rng([seed, T_LOGITS, b, 0, step])
        x = rng.standard_normal(size=(N_CANVAS, vocab), dtype=np.float32)
        pk = np.random.default_rng([seed, T_PEAK, b, 0, step])
        tok = pk.integers(0, vocab, N_CANVAS)
        x[np.arange(N_CANVAS), tok] += pk.uniform(0.0, 24.0, N_CANVAS).astype(np.float32)
        out[b] = bf16_round(x)
    return out


def noise_tokens(seed: int, batch: int, vocab: int = VOCAB, step: int = 0) -> np.ndarray:
    """Uniformly random tokens [B, 256] (int32) for the re-noised positions."""
    out = np.empty((batch, N_CANVAS), np.int32)
    for b in range(batch):
        rng = np.random.default_rng([seed, T_NOISE, b, 0, step])
        out[b] = rng.integers(0, vocab, N_CANVAS, dtype=np.int64).astype(np.int32)
    return out
