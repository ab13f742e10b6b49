"""Pins of the CPU fp64 oracle against things other than itself (CPU only).

The method's definition ("DiffusionGemma Technical Report", paperfeed.app
summary, section "The mechanism: an AR model turned inside out"): a canvas
step is full bidirectional attention within the canvas plus cross-attention to
the cache; a commit encodes the frozen block causally and appends it.  The
pages print no worked numeric example for attention, so the oracle is pinned
by brute force on tiny inputs, closed forms, invariants, a library special
case (torch SDPA on CPU float64) and hand-derived cases in tests/golden/.
"""
import json
import math
import os

import numpy as np
import pytest

from canvas_attention_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(rng, *shape):
    return rng.standard_normal(shape)


def brute(q, keys, vals, scale, mask=None):
    """Materialised softmax without max subtraction (tiny inputs only).
    q [n,D], keys/vals [m,D], mask [n,m] bool (True = visible)."""
    s = scale * (q @ keys.T)
    e = np.exp(s)
    if mask is not None:
        e = np.where(mask, e, 0.0)
    return (e @ vals) / e.sum(axis=1, keepdims=True)


def brute_canvas(q, kc, vc, L, kn, vn, scale, causal=False):
    B, Nc, Hq, D = q.shape
    Hkv = kc.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Nc, Hq, D))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            keys = np.concatenate([kc[b, :L[b], g], kn[b, :, g]])
            vals = np.concatenate([vc[b, :L[b], g], vn[b, :, g]])
            mask = None
            if causal:
                mask = np.ones((Nc, L[b] + Nc), bool)
                mask[:, L[b]:] = np.tril(np.ones((Nc, Nc), bool))
            out[b, :, h] = brute(q[b, :, h], keys, vals, scale, mask)
    return out


def make_case(seed, B, Nc, Hq, Hkv, D, L, cap=None):
    rng = np.random.default_rng(seed)
    cap = cap or (max(L) + Nc)
    q = rnd(rng, B, Nc, Hq, D)
    kc = np.zeros((B, cap, Hkv, D))
    vc = np.zeros((B, cap, Hkv, D))
    for b in range(B):
        kc[b, :L[b]] = rnd(rng, L[b], Hkv, D)
        vc[b, :L[b]] = rnd(rng, L[b], Hkv, D)
    kn = rnd(rng, B, Nc, Hkv, D)
    vn = rnd(rng, B, Nc, Hkv, D)
    return q, kc, vc, np.asarray(L, np.int32), kn, vn


@pytest.mark.parametrize("B,Nc,Hq,Hkv,D,L", [
    (1, 5, 2, 2, 8, [3]),
    (2, 4, 4, 2, 8, [6, 0]),
    (3, 7, 6, 2, 4, [1, 8, 2]),
    (1, 1, 1, 1, 1, [0]),
])
def test_canvas_matches_brute_force(oracle_lib, B, Nc, Hq, Hkv, D, L):
    q, kc, vc, L, kn, vn = make_case(1, B, Nc, Hq, Hkv, D, L)
    scale = 1.0 / math.sqrt(D)
    got = oracle_lib.canvas_attn(q, kc, vc, L, kn, vn, scale)
    want = brute_canvas(q, kc, vc, L, kn, vn, scale)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("B,Nc,Hq,Hkv,D,L", [(1, 5, 2, 1, 8, [3]), (2, 6, 4, 2, 4, [4, 0])])
def test_commit_matches_brute_force(oracle_lib, B, Nc, Hq, Hkv, D, L):
    q, kc, vc, L, kn, vn = make_case(2, B, Nc, Hq, Hkv, D, L)
    scale = 0.3
    got = oracle_lib.commit_attn(q, kc, vc, L, kn, vn, scale)
    want = brute_canvas(q, kc, vc, L, kn, vn, scale, causal=True)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_bf16_and_f32_inputs_widen_exactly(oracle_lib):
    rng = np.random.default_rng(3)
    B, Nc, Hq, Hkv, D, L = 1, 6, 2, 1, 8, np.array([5], np.int32)
    f = {n: rng.standard_normal(s).astype(np.float32) for n, s in
         dict(q=(B, Nc, Hq, D), kc=(B, 8, Hkv, D), vc=(B, 8, Hkv, D), kn=(B, Nc, Hkv, D),
              vn=(B, Nc, Hkv, D)).items()}
    bits = {n: synth.bf16_round(a) for n, a in f.items()}
    wide = {n: synth.bf16_to_f64(a) for n, a in bits.items()}
    got_bf16 = oracle_lib.canvas_attn(bits["q"], bits["kc"], bits["vc"], L, bits["kn"],
                                      bits["vn"])
    want = brute_canvas(wide["q"], wide["kc"], wide["vc"], L, wide["kn"], wide["vn"],
                        1 / math.sqrt(D))
    np.testing.assert_allclose(got_bf16, want, rtol=0, atol=1e-12)
    got_f32 = oracle_lib.canvas_attn(f["q"], f["kc"], f["vc"], L, f["kn"], f["vn"])
    want32 = brute_canvas(*(f[n].astype(np.float64) for n in ("q", "kc", "vc")), L,
                          f["kn"].astype(np.float64), f["vn"].astype(np.float64),
                          1 / math.sqrt(D))
    np.testing.assert_allclose(got_f32, want32, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms

def test_constant_values_give_that_value(oracle_lib):
    q, kc, vc, L, kn, vn = make_case(4, 2, 9, 4, 2, 16, [7, 3])
    c = np.random.default_rng(5).standard_normal((2, 16))  # one vector per kv head
    vc[:] = c[None, None]
    vn[:] = c[None, None]
    got = oracle_lib.canvas_attn(q, kc, vc, L, kn, vn)
    want = np.broadcast_to(np.repeat(c, 2, axis=0)[None, None], got.shape)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


def test_zero_queries_give_mean_of_all_values(oracle_lib):
    q, kc, vc, L, kn, vn = make_case(6, 1, 8, 2, 1, 8, [11])
    q[:] = 0
    got = oracle_lib.canvas_attn(q, kc, vc, L, kn, vn)
    mean = np.concatenate([vc[0, :11, 0], vn[0, :, 0]]).mean(axis=0)
    np.testing.assert_allclose(got[0, 3, 1], mean, rtol=0, atol=1e-14)
    # commit with zero queries: row i averages L + i + 1 values
    got_c = oracle_lib.commit_attn(q, kc, vc, L, kn, vn)
    for i in (0, 4, 7):
        m = np.concatenate([vc[0, :11, 0], vn[0, :i + 1, 0]]).mean(axis=0)
        np.testing.assert_allclose(got_c[0, i, 0], m, rtol=0, atol=1e-14)


def test_single_key_returns_its_value(oracle_lib):
    q, kc, vc, L, kn, vn = make_case(7, 1, 1, 1, 1, 8, [0])
    got = oracle_lib.canvas_attn(q, kc, vc, L, kn, vn)
    np.testing.assert_array_equal(got[0, 0, 0], vn[0, 0, 0])
    # commit: block row 0 with an empty prefix sees only itself
    q, kc, vc, L, kn, vn = make_case(8, 1, 5, 2, 2, 4, [0])
    got = oracle_lib.commit_attn(q, kc, vc, L, kn, vn)
    np.testing.assert_array_equal(got[0, 0], vn[0, 0])


def test_dominant_key_wins(oracle_lib):
    D = 8
    q, kc, vc, L, kn, vn = make_case(9, 1, 4, 1, 1, D, [6])
    q[0, 2, 0] = 0
    q[0, 2, 0, 0] = 1.0
    kc[0, :6, 0, 0] = 0
    kn[0, :, 0, 0] = 0
    kc[0, 4, 0, 0] = 60.0  # score of key 4 is 60 above every other key (scale 1)
    got = oracle_lib.canvas_attn(q, kc, vc, L, kn, vn, scale=1.0)
    np.testing.assert_allclose(got[0, 2, 0], vc[0, 4, 0], rtol=0, atol=1e-20)


# ------------------------------------------------------------------ invariants

def test_canvas_permutation_equivariance(oracle_lib):
    q, kc, vc, L, kn, vn = make_case(10, 1, 12, 4, 2, 8, [9])
    base = oracle_lib.canvas_attn(q, kc, vc, L, kn, vn)
    perm = np.random.default_rng(11).permutation(12)
    # permuting canvas positions (queries and their K/V jointly) permutes outputs
    got = oracle_lib.canvas_attn(q[:, perm], kc, vc, L, kn[:, perm], vn[:, perm])
    np.testing.assert_allclose(got, base[:, perm], rtol=0, atol=1e-13)
    # permuting only the canvas K/V leaves every output unchanged
    got2 = oracle_lib.canvas_attn(q, kc, vc, L, kn[:, perm], vn[:, perm])
    np.testing.assert_allclose(got2, base, rtol=0, atol=1e-13)


def test_key_shift_invariance(oracle_lib):
    q, kc, vc, L, kn, vn = make_case(12, 1, 6, 2, 1, 8, [5])
    base = oracle_lib.canvas_attn(q, kc, vc, L, kn, vn)
    k0 = np.random.default_rng(13).standard_normal(8)
    got = oracle_lib.canvas_attn(q, kc + k0, vc, L, kn + k0, vn)
    np.testing.assert_allclose(got, base, rtol=0, atol=1e-12)


def test_linearity_in_values(oracle_lib):
    q, kc, vc, L, kn, vn = make_case(14, 1, 6, 2, 2, 8, [4])
    _, _, vc2, _, _, vn2 = make_case(15, 1, 6, 2, 2, 8, [4])
    a, b = 0.7, -2.5
    o1 = oracle_lib.canvas_attn(q, kc, vc, L, kn, vn)
    o2 = oracle_lib.canvas_attn(q, kc, vc2, L, kn, vn2)
    o = oracle_lib.canvas_attn(q, kc, a * vc + b * vc2, L, kn, a * vn + b * vn2)
    np.testing.assert_allclose(o, a * o1 + b * o2, rtol=0, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv(oracle_lib):
    q, kc, vc, L, kn, vn = make_case(16, 2, 5, 6, 3, 8, [4, 2])
    gqa = oracle_lib.canvas_attn(q, kc, vc, L, kn, vn)
    rep = lambda x: np.repeat(x, 2, axis=2)  # kv head g serves query heads 2g, 2g+1
    mha = oracle_lib.canvas_attn(q, rep(kc), rep(vc), L, rep(kn), rep(vn))
    np.testing.assert_array_equal(gqa, mha)
    gqa_c = oracle_lib.commit_attn(q, kc, vc, L, kn, vn)
    mha_c = oracle_lib.commit_attn(q, rep(kc), rep(vc), L, rep(kn), rep(vn))
    np.testing.assert_array_equal(gqa_c, mha_c)


def test_split_merge_equals_concatenated_attention(oracle_lib):
    rng = np.random.default_rng(17)
    D, n_q, L, Nc = 8, 5, 23, 6
    q = rng.standard_normal((n_q, D))
    keys = rng.standard_normal((L + Nc, D))
    vals = rng.standard_normal((L + Nc, D))
    scale = 0.4
    full = brute(q, keys, vals, scale)
    # prefix split into uneven pieces (one empty), then the canvas tile
    bounds = [0, 7, 7, 16, L, L + Nc]
    parts = [oracle_lib.partial(q, keys[a:b], vals[a:b], scale)
             for a, b in zip(bounds[:-1], bounds[1:])]
    assert parts[1][0][0] == -np.inf and parts[1][1][0] == 0.0
    ms = np.stack([p[0] for p in parts])
    ls = np.stack([p[1] for p in parts])
    os_ = np.stack([p[2] for p in parts])
    np.testing.assert_allclose(oracle_lib.merge(ms, ls, os_), full, rtol=0, atol=1e-12)


def test_split_merge_canvas_rows(oracle_lib):
    rng = np.random.default_rng(18)
    D, Nc, L = 8, 6, 19
    q, kc, vc, Ls, kn, vn = make_case(18, 1, Nc, 1, 1, D, [L])
    scale = 1 / math.sqrt(D)
    want = oracle_lib.canvas_attn(q, kc, vc, Ls, kn, vn)[0, :, 0]
    keys = np.concatenate([kc[0, :L, 0], kn[0, :, 0]])
    vals = np.concatenate([vc[0, :L, 0], vn[0, :, 0]])
    cut = sorted(rng.choice(np.arange(1, L + Nc), 3, replace=False))
    bounds = [0, *cut, L + Nc]
    parts = [oracle_lib.partial(q[0, :, 0], keys[a:b], vals[a:b], scale)
             for a, b in zip(bounds[:-1], bounds[1:])]
    got = oracle_lib.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]),
                           np.stack([p[2] for p in parts]))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# ------------------------------------------------------------- commit identity

def test_commit_is_tail_of_full_causal_attention(oracle_lib):
    B, Nc, Hq, Hkv, D, L = 1, 6, 2, 1, 8, 9
    rng = np.random.default_rng(19)
    T = L + Nc
    # a whole causal sequence; its first L positions form the cache
    qs, ks, vs = (rng.standard_normal((T, Hq if n == "q" else Hkv, D)) for n in "qkv")
    scale = 1 / math.sqrt(D)
    full = np.zeros((T, Hq, D))
    for h in range(Hq):
        mask = np.tril(np.ones((T, T), bool))
        full[:, h] = brute(qs[:, h], ks[:, h // (Hq // Hkv)], vs[:, h // (Hq // Hkv)], scale,
                           mask)
    cap = T + 4
    kc = np.zeros((B, cap, Hkv, D))
    vc = np.zeros((B, cap, Hkv, D))
    kc[0, :L], vc[0, :L] = ks[:L], vs[:L]
    kb, vb = ks[None, L:].copy(), vs[None, L:].copy()
    got = oracle_lib.commit_attn(qs[None, L:], kc, vc, [L], kb, vb, scale)
    np.testing.assert_allclose(got[0], full[L:], rtol=0, atol=1e-12)
    # append: the cache becomes old cache ++ block, bit for bit; nothing else moves
    before = kc.copy(), vc.copy()
    oracle_lib.append_block(kb, vb, kc, vc, [L])
    np.testing.assert_array_equal(kc[0, :L], before[0][0, :L])
    np.testing.assert_array_equal(kc[0, L:T], ks[L:])
    np.testing.assert_array_equal(vc[0, L:T], vs[L:])
    np.testing.assert_array_equal(kc[0, T:], 0)
    # a canvas step on the grown cache equals attention over the whole history
    qn, kn, vn = (rng.standard_normal((1, Nc, Hq if n == "q" else Hkv, D)) for n in "qkv")
    step = oracle_lib.canvas_attn(qn, kc, vc, [T], kn, vn, scale)
    keys = np.concatenate([ks, kn[0]])
    vals = np.concatenate([vs, vn[0]])
    for h in range(Hq):
        np.testing.assert_allclose(step[0, :, h], brute(qn[0, :, h], keys[:, 0], vals[:, 0],
                                                        scale), rtol=0, atol=1e-12)


def test_append_rejects_overflow(oracle_lib):
    kb = np.zeros((1, 4, 1, 2))
    kc = np.zeros((1, 6, 1, 2))
    with pytest.raises(ValueError):
        oracle_lib.append_block(kb, kb, kc, kc.copy(), [3])


# ---------------------------------------------------- library special case: SDPA

def test_empty_prefix_is_plain_attention_sdpa(oracle_lib):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    B, Nc, Hq, Hkv, D = 2, 16, 4, 2, 8
    q, kc, vc, L, kn, vn = make_case(20, B, Nc, Hq, Hkv, D, [0, 0], cap=4)
    got = oracle_lib.canvas_attn(q, kc, vc, L, kn, vn)
    got_c = oracle_lib.commit_attn(q, kc, vc, L, kn, vn)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)                       # [B,Hq,Nc,D]
    tk = torch.from_numpy(np.repeat(kn, 2, axis=2)).permute(0, 2, 1, 3)
    tv = torch.from_numpy(np.repeat(vn, 2, axis=2)).permute(0, 2, 1, 3)
    ref = F.scaled_dot_product_attention(tq, tk, tv).permute(0, 2, 1, 3).numpy()
    ref_c = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got_c, ref_c, rtol=0, atol=1e-12)


def test_commit_with_prefix_matches_sdpa_bottom_right_mask(oracle_lib):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    B, Nc, Hq, Hkv, D, L = 1, 8, 2, 2, 8, 5
    q, kc, vc, Ls, kn, vn = make_case(21, B, Nc, Hq, Hkv, D, [L])
    got = oracle_lib.commit_attn(q, kc, vc, Ls, kn, vn)
    keys = np.concatenate([kc[:, :L], kn], axis=1)
    vals = np.concatenate([vc[:, :L], vn], axis=1)
    mask = torch.ones(Nc, L + Nc, dtype=torch.bool)
    mask[:, L:] = torch.tril(torch.ones(Nc, Nc, dtype=torch.bool))
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q).permute(0, 2, 1, 3), torch.from_numpy(keys).permute(0, 2, 1, 3),
        torch.from_numpy(vals).permute(0, 2, 1, 3), attn_mask=mask).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_row_subset_matches_full_output(oracle_lib):
    q, kc, vc, L, kn, vn = make_case(22, 2, 6, 4, 2, 8, [3, 5])
    full = oracle_lib.canvas_attn(q, kc, vc, L, kn, vn)
    rows = [(1, 5, 3), (0, 0, 0), (1, 2, 1)]
    got = oracle_lib.canvas_attn(q, kc, vc, L, kn, vn, rows=rows)
    for r, (b, i, h) in enumerate(rows):
        np.testing.assert_array_equal(got[r], full[b, i, h])
    fullc = oracle_lib.commit_attn(q, kc, vc, L, kn, vn)
    gotc = oracle_lib.commit_attn(q, kc, vc, L, kn, vn, rows=rows)
    for r, (b, i, h) in enumerate(rows):
        np.testing.assert_array_equal(gotc[r], fullc[b, i, h])


# ------------------------------------------------------- hand-derived cases

def _load_golden():
    with open(os.path.join(GOLDEN, "hand_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _load_golden(), ids=lambda c: c["name"])
def test_hand_derived_cases(oracle_lib, case):
    a = {k: np.asarray(case[k], np.float64) for k in ("q", "k_cache", "v_cache", "k_new",
                                                      "v_new")}
    fn = oracle_lib.commit_attn if case["op"] == "commit" else oracle_lib.canvas_attn
    got = fn(a["q"], a["k_cache"], a["v_cache"], case["prefix_len"], a["k_new"], a["v_new"],
             case["scale"])
    env = {"e": math.e, "exp": math.exp, "sqrt": math.sqrt}
    want = np.array([[[[eval(x, {"__builtins__": {}}, env) for x in head] for head in row]
                      for row in seq] for seq in case["expected"]], np.float64)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)
