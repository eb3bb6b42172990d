"""Pins for the oracle's window scores (CPU only).

Each test checks the float64 oracle against something other than itself:
pure-Python brute force, a library routine (scipy softmax / logsumexp), a
closed form, or an invariant that a dropped term, wrong sign, wrong index or
transposed operand would break.
"""
import math

import numpy as np
import pytest
import scipy.special

from oracle import brute
from oracle import oracle as orc



def _rand(seed, B, Hq, Hkv, W, N, d):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, W, d))
    k = rng.standard_normal((B, Hkv, N, d))
    return q, k


@pytest.mark.parametrize("G,causal,ctx", [(1, False, None), (2, False, None),
                                          (2, True, None), (1, True, [9, 13]),
                                          (2, False, [7, 13])])
def test_score_matches_brute_force(G, causal, ctx):
    B, Hkv, W, N, d = 2, 2, 3, 13, 5
    q, k = _rand(1 + G, B, Hkv * G, Hkv, W, N, d)
    scale = 1.0 / math.sqrt(d)
    s, lse = orc.window_scores(q, k, ctx, causal=causal)
    ctx_arr = [N] * B if ctx is None else ctx
    for b in range(B):
        n = ctx_arr[b]
        for h in range(Hkv):
            qs = [[list(q[b, h * G + j, w]) for w in range(W)] for j in range(G)]
            ks = [list(k[b, h, t]) for t in range(n)]
            s_ref, lse_ref = brute.score(qs, ks, n, G, scale, causal)
            np.testing.assert_allclose(s[b, h, :n], s_ref, rtol=1e-12, atol=1e-15)
            assert np.all(s[b, h, n:] == 0.0)
            for j in range(G):
                np.testing.assert_allclose(lse[b, h * G + j], lse_ref[j], rtol=1e-12)


def test_single_row_is_scipy_softmax():
    # W = G = 1: the score of token t is softmax(scale * K q)_t and the row
    # normaliser is scipy's logsumexp.
    q, k = _rand(7, 1, 3, 3, 1, 40, 16)
    s, lse = orc.window_scores(q, k)
    for h in range(3):
        logits = (k[0, h] @ q[0, h, 0]) / math.sqrt(16)
        np.testing.assert_allclose(s[0, h], scipy.special.softmax(logits), rtol=1e-12)
        np.testing.assert_allclose(lse[0, h, 0], scipy.special.logsumexp(logits), rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_scores_sum_to_rows_per_head(causal):
    # Each window row is a probability distribution, so a KV head's scores
    # total W * G (W per query head), whatever the mask.
    q, k = _rand(3, 3, 8, 2, 6, 50, 8)
    ctx = [50, 17, 6]
    s, _ = orc.window_scores(q, k, ctx, causal=causal)
    np.testing.assert_allclose(s.sum(axis=2), np.full((3, 2), 6 * 4.0), rtol=1e-13)


def test_identical_keys_closed_forms():
    # All keys equal: every visible token gets the same logit, so a row
    # spreads probability uniformly over what it sees.
    B, Hq, Hkv, W, N, d = 1, 4, 2, 4, 10, 8
    rng = np.random.default_rng(5)
    q = rng.standard_normal((B, Hq, W, d))
    k = np.tile(rng.standard_normal(d), (B, Hkv, N, 1))
    G = Hq // Hkv
    s, _ = orc.window_scores(q, k)
    np.testing.assert_allclose(s, np.full((B, Hkv, N), W * G / N), rtol=1e-13)
    s_c, _ = orc.window_scores(q, k, causal=True)
    for t in range(N):
        expect = G * sum(1.0 / (N - W + w + 1) for w in range(W) if t <= N - W + w)
        np.testing.assert_allclose(s_c[0, :, t], expect, rtol=1e-13)


def test_zero_query_is_uniform():
    q, k = _rand(11, 1, 2, 1, 5, 30, 8)
    q[:] = 0.0
    s, lse = orc.window_scores(q, k, [30])
    np.testing.assert_allclose(s[0, 0], np.full(30, 10 / 30), rtol=1e-13)
    np.testing.assert_allclose(lse, math.log(30), rtol=1e-14)


def test_dominant_key_takes_all_mass():
    # One key strongly aligned with every window query: it should collect
    # nearly all W * G; a flipped sign would send its score to ~0.
    rng = np.random.default_rng(2)
    d, N, W = 8, 20, 3
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = np.tile(4.0 * u, (1, 2, W, 1)) + 0.01 * rng.standard_normal((1, 2, W, d))
    k = 0.1 * rng.standard_normal((1, 1, N, d))
    k[0, 0, 7] = 40.0 * u
    s, _ = orc.window_scores(q, k)
    assert s[0, 0, 7] > 2 * W * (1 - 1e-10)
    assert np.all(np.delete(s[0, 0], 7) < 1e-10)


def test_gqa_groups_are_contiguous():
    # Query heads 0,1 look along e0 and 2,3 along e1.  KV head 0 hides an e0
    # key at token 2, KV head 1 an e1 key at token 4.  With contiguous groups
    # (h = j // G) each head's planted key takes all of its group's mass; a
    # strided mapping (h = j % Hkv) would split it.
    d, N, W = 4, 6, 2
    e = np.eye(d)
    q = np.zeros((1, 4, W, d))
    q[0, 0:2] = 10 * e[0]
    q[0, 2:4] = 10 * e[1]
    k = np.full((1, 2, N, d), 0.01)
    k[0, 0, 2] = 10 * e[0]
    k[0, 1, 4] = 10 * e[1]
    s, _ = orc.window_scores(q, k)
    assert s[0, 0, 2] > 2 * W - 1e-9
    assert s[0, 1, 4] > 2 * W - 1e-9


def test_permuting_tokens_permutes_scores():
    q, k = _rand(21, 1, 4, 2, 3, 25, 8)
    perm = np.random.default_rng(0).permutation(25)
    s, lse = orc.window_scores(q, k)
    s_p, lse_p = orc.window_scores(q, k[:, :, perm])
    np.testing.assert_allclose(s_p, s[:, :, perm], rtol=1e-12)
    np.testing.assert_allclose(lse_p, lse, rtol=1e-13)


def test_scale_argument_scales_logits():
    q, k = _rand(4, 1, 2, 2, 3, 20, 16)
    s2, lse2 = orc.window_scores(q, k, scale=0.5)
    s_ref, lse_ref = orc.window_scores(2.0 * q, k)      # 2/sqrt(16) = 0.5
    np.testing.assert_allclose(s2, s_ref, rtol=1e-12)
    np.testing.assert_allclose(lse2, lse_ref, rtol=1e-12)


def test_causal_single_row_equals_noncausal():
    # W = 1: the only window row sits at the last token and sees everything.
    q, k = _rand(9, 2, 4, 2, 1, 33, 8)
    a, la = orc.window_scores(q, k, [33, 20], causal=True)
    b, lb = orc.window_scores(q, k, [33, 20], causal=False)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


# ---- one-pass scores from given row LSEs -----------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_from_lse_with_own_lse_is_two_pass(causal):
    # Handing the oracle's own row LSE back must reproduce the two-pass scores.
    q, k = _rand(21, 2, 6, 2, 5, 40, 8)
    ctx = [40, 23]
    s, lse = orc.window_scores(q, k, ctx, causal=causal)
    s1 = orc.window_scores_from_lse(q, k, lse, ctx, causal=causal)
    np.testing.assert_allclose(s1, s, rtol=1e-12, atol=1e-300)


def test_from_lse_shift_scales_scores():
    # Raising every normaliser by log 2 halves every score (closed form).
    q, k = _rand(22, 1, 4, 2, 3, 30, 8)
    s, lse = orc.window_scores(q, k)
    s2 = orc.window_scores_from_lse(q, k, lse + math.log(2.0))
    np.testing.assert_allclose(s2, s / 2.0, rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_from_lse_matches_brute_force(causal):
    rng = np.random.default_rng(23)
    B, Hkv, G, W, N, d = 1, 2, 2, 3, 11, 5
    q, k = _rand(24, B, Hkv * G, Hkv, W, N, d)
    lse = rng.standard_normal((B, Hkv * G, W)) + 3.0
    lse[0, 1, 2] = np.inf                      # a row that adds nothing
    s = orc.window_scores_from_lse(q, k, lse, causal=causal)
    scale = 1.0 / math.sqrt(d)
    for h in range(Hkv):
        qs = [[list(q[0, h * G + j, w]) for w in range(W)] for j in range(G)]
        ks = [list(k[0, h, t]) for t in range(N)]
        ls = [[float(lse[0, h * G + j, w]) for w in range(W)] for j in range(G)]
        ref = brute.score_from_lse(qs, ks, N, G, scale, ls, causal)
        np.testing.assert_allclose(s[0, h], ref, rtol=1e-12, atol=1e-300)
