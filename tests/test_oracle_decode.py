"""Pins of the oracle's decode attention (CPU only).

AR mode ("DiffusionGemma Technical Report", paperfeed.app summary, section "The
numbers, honestly"): the same weights decode causally over the same cache, one
token at a time, or several drafted tokens in one pass (hybrid decoding).  New
token i attends to cache rows 0..L-1 and new rows 0..i, and the new K/V rows then
join the cache.  oracle.decode_attn is pinned here by brute force on tiny inputs,
closed forms, a library special case (torch SDPA on CPU float64 with an explicit
mask) and two relations that tie it to other calls: decoding k tokens at once
equals decoding them one by one with an append after each, and equals the last k
rows of a block commit.
"""
import numpy as np
import pytest


def case(seed, B, k, Hq, Hkv, D, L, cap=None):
    rng = np.random.default_rng(seed)
    cap = cap or (max(L) + k)
    q = rng.standard_normal((B, k, Hq, D))
    kc = np.zeros((B, cap, Hkv, D))
    vc = np.zeros((B, cap, Hkv, D))
    for b in range(B):
        kc[b, :L[b]] = rng.standard_normal((L[b], Hkv, D))
        vc[b, :L[b]] = rng.standard_normal((L[b], Hkv, D))
    kn = rng.standard_normal((B, k, Hkv, D))
    vn = rng.standard_normal((B, k, Hkv, D))
    return q, kc, vc, np.asarray(L, np.int32), kn, vn


def brute_decode(q, kc, vc, L, kn, vn, scale):
    """Softmax written out per row, without max subtraction (tiny inputs only)."""
    B, k, Hq, D = q.shape
    G = Hq // kc.shape[2]
    out = np.zeros(q.shape)
    for b in range(B):
        for i in range(k):
            for h in range(Hq):
                g = h // G
                keys = [kc[b, j, g] for j in range(L[b])] + [kn[b, j, g] for j in range(i + 1)]
                vals = [vc[b, j, g] for j in range(L[b])] + [vn[b, j, g] for j in range(i + 1)]
                w = [np.exp(scale * float(np.dot(q[b, i, h], kk))) for kk in keys]
                out[b, i, h] = sum(wj * vj for wj, vj in zip(w, vals)) / sum(w)
    return out


@pytest.mark.parametrize("B,k,Hq,Hkv,D,L", [
    (1, 1, 2, 1, 8, [5]),
    (2, 3, 4, 2, 8, [6, 0]),
    (3, 16, 4, 2, 4, [1, 9, 0]),
    (1, 1, 1, 1, 1, [0]),
])
def test_decode_matches_brute_force(oracle_lib, B, k, Hq, Hkv, D, L):
    q, kc, vc, Ls, kn, vn = case(30, B, k, Hq, Hkv, D, L)
    scale = 0.7 / np.sqrt(D)
    got = oracle_lib.decode_attn(q, kc, vc, Ls, kn, vn, scale=scale)
    np.testing.assert_allclose(got, brute_decode(q, kc, vc, Ls, kn, vn, scale), rtol=0, atol=1e-12)


def test_first_token_of_an_empty_cache_returns_its_value(oracle_lib):
    # one visible key: its softmax weight is exactly 1
    q, kc, vc, L, kn, vn = case(31, 2, 1, 4, 2, 8, [0, 0], cap=1)
    got = oracle_lib.decode_attn(q, kc, vc, L, kn, vn)
    np.testing.assert_array_equal(got, np.repeat(vn, 2, axis=2))


def test_zero_keys_give_the_mean_of_the_visible_values(oracle_lib):
    # equal scores: token i averages the L cache values and new values 0..i
    B, k, Hq, Hkv, D, L = 1, 5, 2, 1, 4, 7
    q, kc, vc, Ls, kn, vn = case(32, B, k, Hq, Hkv, D, [L])
    kc[:] = 0.0
    kn[:] = 0.0
    got = oracle_lib.decode_attn(q, kc, vc, Ls, kn, vn)
    for i in range(k):
        ref = (vc[0, :L, 0].sum(0) + vn[0, :i + 1, 0].sum(0)) / (L + i + 1)
        for h in range(Hq):
            np.testing.assert_allclose(got[0, i, h], ref, rtol=0, atol=1e-14)


def test_decode_matches_sdpa_with_bottom_right_mask(oracle_lib):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    B, k, Hq, Hkv, D, L = 1, 6, 4, 2, 8, 9
    q, kc, vc, Ls, kn, vn = case(33, B, k, Hq, Hkv, D, [L])
    got = oracle_lib.decode_attn(q, kc, vc, Ls, kn, vn)
    keys = np.repeat(np.concatenate([kc[:, :L], kn], axis=1), Hq // Hkv, axis=2)
    vals = np.repeat(np.concatenate([vc[:, :L], vn], axis=1), Hq // Hkv, axis=2)
    mask = torch.ones(k, L + k, dtype=torch.bool)
    mask[:, L:] = torch.tril(torch.ones(k, k, dtype=torch.bool))
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q).permute(0, 2, 1, 3), torch.from_numpy(keys).permute(0, 2, 1, 3),
        torch.from_numpy(vals).permute(0, 2, 1, 3), attn_mask=mask).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_hybrid_equals_token_by_token(oracle_lib):
    """k drafted tokens in one pass equal k single-token AR steps, each followed by
    the append of its K/V (the cache ends the same either way)."""
    B, k, Hq, Hkv, D = 2, 5, 4, 2, 8
    q, kc, vc, L, kn, vn = case(34, B, k, Hq, Hkv, D, [4, 11], cap=11 + k)
    kc1, vc1 = kc.copy(), vc.copy()
    once = oracle_lib.decode_attn(q, kc1, vc1, L, kn, vn)
    oracle_lib.append_block(kn, vn, kc1, vc1, L)
    kc2, vc2 = kc.copy(), vc.copy()
    steps = np.zeros_like(once)
    Lt = L.copy()
    for i in range(k):
        sl = slice(i, i + 1)
        steps[:, sl] = oracle_lib.decode_attn(q[:, sl], kc2, vc2, Lt, kn[:, sl], vn[:, sl])
        oracle_lib.append_block(kn[:, sl].copy(), vn[:, sl].copy(), kc2, vc2, Lt)
        Lt = Lt + 1
    np.testing.assert_allclose(once, steps, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(kc1, kc2)
    np.testing.assert_array_equal(vc1, vc2)


def test_decode_is_the_tail_of_a_block_commit(oracle_lib):
    """The last k rows of a commit of Nc rows equal a decode of those k rows over the
    cache extended by the block's first Nc - k rows."""
    B, Nc, k, Hq, Hkv, D, L = 1, 12, 4, 4, 2, 8, 6
    q, kc, vc, Ls, kb, vb = case(35, B, Nc, Hq, Hkv, D, [L], cap=L + Nc)
    full = oracle_lib.commit_attn(q, kc, vc, Ls, kb, vb)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, L:L + Nc - k] = kb[:, :Nc - k]
    vc2[:, L:L + Nc - k] = vb[:, :Nc - k]
    tail = oracle_lib.decode_attn(q[:, Nc - k:].copy(), kc2, vc2, Ls + (Nc - k),
                                  kb[:, Nc - k:].copy(), vb[:, Nc - k:].copy())
    np.testing.assert_allclose(tail, full[:, Nc - k:], rtol=0, atol=1e-13)
