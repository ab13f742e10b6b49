"""Pins of the oracle's fp8 (OCP e4m3) inputs and of the seeded e4m3 encoder (CPU only).

The oracle reads e4m3 bytes with its own decoder (written from the OCP 8-bit
floating point specification) and multiplies each element by its tensor's scale.
torch's float8_e4m3fn type implements the same format; it serves here as the
library reference for decoding and for round-to-nearest-even encoding.
"""
import math

import numpy as np
import pytest

from canvas_attention_amd import synth

torch = pytest.importorskip("torch")

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def torch_decode(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def test_decoder_every_finite_code(oracle_lib):
    """All value rows equal: the output is that row, one head_dim column per e4m3
    byte, times the value scale."""
    D = len(FINITE)
    rng = np.random.default_rng(0)
    q = synth.e4m3_round(rng.standard_normal((1, 4, 1, D)).astype(np.float32))
    kc = synth.e4m3_round(rng.standard_normal((1, 3, 1, D)).astype(np.float32))
    kn = synth.e4m3_round(rng.standard_normal((1, 4, 1, D)).astype(np.float32))
    vc = np.broadcast_to(FINITE, (1, 3, 1, D)).copy()
    vn = np.broadcast_to(FINITE, (1, 4, 1, D)).copy()
    for vs in (1.0, 0.375):
        out = oracle_lib.canvas_attn(q, kc, vc, [3], kn, vn, scale=0.1,
                                     tensor_scales=(1.0, 1.0, vs))
        want = vs * torch_decode(FINITE)
        np.testing.assert_allclose(out[0, :, 0], np.broadcast_to(want, (4, D)), rtol=1e-14,
                                   atol=0)
    # spot values of the format: smallest subnormal, smallest normal, one, largest
    for code, val in ((0x01, 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0), (0x7E, 448.0),
                      (0x80, -0.0), (0xFE, -448.0)):
        assert torch_decode(np.uint8([code]))[0] == val
        col = int(np.nonzero(FINITE == code)[0][0])
        assert out[0, 0, 0, col] == pytest.approx(0.375 * val, rel=1e-14, abs=0)


def test_nan_bytes_propagate(oracle_lib):
    """0x7f and 0xff are NaN in e4m3 (the format has no infinities)."""
    q = np.full((1, 2, 1, 2), 0x38, np.uint8)
    kn = np.full((1, 2, 1, 2), 0x38, np.uint8)
    vn = np.array([[[[0x38, 0x7F]], [[0x38, 0xFF]]]], np.uint8)
    out = oracle_lib.canvas_attn(q, np.zeros((1, 0, 1, 2), np.uint8),
                                 np.zeros((1, 0, 1, 2), np.uint8), [0], kn, vn, scale=1.0)
    assert np.all(out[..., 0] == 1.0) and np.all(np.isnan(out[..., 1]))


def brute(q, keys, vals, scale, mask=None):
    s = scale * (q @ keys.T)
    e = np.exp(s)
    if mask is not None:
        e = np.where(mask, e, 0.0)
    return (e @ vals) / e.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("ts", [(1.0, 1.0, 1.0), (0.5, 2.5, 0.75), (3.0, 0.125, 8.0)])
def test_scaled_fp8_matches_brute_force(oracle_lib, causal, ts):
    """Tiny e4m3 inputs: decoded by torch, scaled, and attended by a materialised
    softmax; each tensor scale lands on its own operand."""
    rng = np.random.default_rng(7)
    B, Nc, Hq, Hkv, D, L = 2, 5, 4, 2, 6, [3, 0]
    cap = 4

    def codes(*shape):
        return synth.e4m3_round(rng.standard_normal(shape).astype(np.float32) * 1.5)

    q, kn, vn = codes(B, Nc, Hq, D), codes(B, Nc, Hkv, D), codes(B, Nc, Hkv, D)
    kc, vc = codes(B, cap, Hkv, D), codes(B, cap, Hkv, D)
    scale = 1.0 / math.sqrt(D)
    fn = oracle_lib.commit_attn if causal else oracle_lib.canvas_attn
    got = fn(q, kc, vc, L, kn, vn, scale=scale, tensor_scales=ts)
    qf, kcf, vcf = ts[0] * torch_decode(q), ts[1] * torch_decode(kc), ts[2] * torch_decode(vc)
    knf, vnf = ts[1] * torch_decode(kn), ts[2] * torch_decode(vn)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            g = h // G
            keys = np.concatenate([kcf[b, :L[b], g], knf[b, :, g]])
            vals = np.concatenate([vcf[b, :L[b], g], vnf[b, :, g]])
            mask = None
            if causal:
                mask = np.ones((Nc, L[b] + Nc), bool)
                mask[:, L[b]:] = np.tril(np.ones((Nc, Nc), bool))
            want = brute(qf[b, :, h], keys, vals, scale, mask)
            np.testing.assert_allclose(got[b, :, h], want, rtol=0, atol=1e-12)


def test_scale_one_equals_unscaled(oracle_lib):
    rng = np.random.default_rng(3)
    q = synth.e4m3_round(rng.standard_normal((1, 8, 2, 16)).astype(np.float32))
    k = synth.e4m3_round(rng.standard_normal((1, 8, 1, 16)).astype(np.float32))
    v = synth.e4m3_round(rng.standard_normal((1, 8, 1, 16)).astype(np.float32))
    e = np.zeros((1, 0, 1, 16), np.uint8)
    a = oracle_lib.canvas_attn(q, e, e, [0], k, v)
    b = oracle_lib.canvas_attn(q, e, e, [0], k, v, tensor_scales=(1.0, 1.0, 1.0))
    np.testing.assert_array_equal(a, b)
    with pytest.raises(ValueError):
        oracle_lib.canvas_attn(q, e, e, [0], k, v, tensor_scales=(1.0, 0.0, 1.0))


def test_encoder_matches_torch_rounding():
    """synth.e4m3_round rounds to nearest even like torch's conversion, across the
    subnormal and normal binades and on every midpoint between neighbours; beyond
    448 it saturates (torch's conversion gives NaN from 464 up)."""
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp2(rng.integers(-12, 9, 100000))).astype(np.float32)
    x = x[np.abs(x) <= 448]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(synth.e4m3_round(x), want)
    pos = torch_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = np.concatenate([(pos[:-1] + pos[1:]) / 2, -(pos[:-1] + pos[1:]) / 2]).astype(np.float32)
    want = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(synth.e4m3_round(mids), want)
    np.testing.assert_array_equal(synth.e4m3_round(np.float32([500.0, -1e9, np.inf, np.nan])),
                                  np.uint8([0x7E, 0xFE, 0x7E, 0x7F]))
