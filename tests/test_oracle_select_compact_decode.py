"""Pins for the oracle's budget, selection, compaction and decode (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import oracle as orc


def _scores_with_ties(seed, n, levels=6):
    rng = np.random.default_rng(seed)
    return rng.integers(0, levels, size=n).astype(np.float64) / levels


@pytest.mark.parametrize("seed", range(6))
def test_selection_matches_pairwise_rank(seed):
    # Heavy ties: the kept set must be the tokens with fewer than k
    # predecessors in the (score desc, index asc) order.
    n = 23
    s = _scores_with_ties(seed, n)
    for k in (1, 5, 11, 23):
        kept, cnt = orc.select(s.reshape(1, 1, n), None, orc.BUDGET_K, k=k)
        assert cnt[0] == k
        assert list(kept[0, 0, :k]) == brute.top_k(list(s), k)


def test_selection_with_distinct_scores_maximises_mass():
    s = np.random.default_rng(3).random(10)
    for k in (1, 3, 6):
        kept, _ = orc.select(s.reshape(1, 1, 10), None, orc.BUDGET_K, k=k)
        assert list(kept[0, 0, :k]) == brute.top_k_by_subsets(list(s), k)


def test_all_equal_scores_keep_lowest_indices():
    s = np.full((1, 1, 40), 0.25)
    kept, cnt = orc.select(s, None, orc.BUDGET_K, k=7)
    assert list(kept[0, 0, :7]) == list(range(7)) and cnt[0] == 7
    # signed zero: -0.0 ties with +0.0 and the lower index wins
    z = np.array([[[0.0, -0.0, 0.0, -0.0, 1.0]]])
    kept, _ = orc.select(z, None, orc.BUDGET_K, k=3)
    assert list(kept[0, 0, :3]) == [0, 1, 4]


def test_k_equal_one_is_lowest_index_argmax():
    s = np.array([[[0.1, 0.7, 0.3, 0.7, 0.7]]])
    kept, _ = orc.select(s, None, orc.BUDGET_K, k=1)
    assert kept[0, 0, 0] == 1


@pytest.mark.parametrize("n,r,expect", [(1024, 0.25, 256), (8192, 0.20, 1638),
                                        (32768, 0.10, 3277), (131072, 0.10, 13107),
                                        (10, 0.0, 1), (10, 1.0, 10), (3, 0.5, 2)])
def test_ratio_counts(n, r, expect):
    # round half up of r*n with r the fp32 value, clamped to [1, n]
    assert orc.budget_count(np.zeros(n), orc.BUDGET_RATIO, ratio=r) == expect


def test_threshold_keeps_scores_at_or_above_tau():
    s = np.array([0.5, 0.25, 0.125, 0.25, 0.75, 0.0625])
    kept, cnt = orc.select(s.reshape(1, 1, -1), None, orc.BUDGET_THRESHOLD, tau=0.25)
    assert cnt[0] == 4 and list(kept[0, 0, :4]) == [0, 1, 3, 4]
    # nothing above tau still keeps one token (the lowest-index maximum)
    kept, cnt = orc.select(s.reshape(1, 1, -1), None, orc.BUDGET_THRESHOLD, tau=2.0)
    assert cnt[0] == 1 and kept[0, 0, 0] == 4
    # clamps: at most 50%, at least 50%
    _, cnt = orc.select(s.reshape(1, 1, -1), None, orc.BUDGET_THRESHOLD, tau=0.0,
                        max_ratio=0.5)
    assert cnt[0] == 3
    _, cnt = orc.select(s.reshape(1, 1, -1), None, orc.BUDGET_THRESHOLD, tau=1.0,
                        min_ratio=0.5)
    assert cnt[0] == 3


@pytest.mark.parametrize("seed", range(5))
def test_mass_budget_bracket_and_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = 30
    s = rng.random(n) ** 4
    s[rng.integers(0, n, 5)] = s[0]            # some exact ties
    for f in (0.3, 0.5, 0.95):
        k = orc.budget_count(s, orc.BUDGET_MASS, mass=f)
        ff = float(np.float32(f))
        assert k == brute.mass_count(list(s), ff)
        top = np.sort(s)[::-1]
        total = math.fsum(s)
        assert math.fsum(top[:k]) >= ff * total - 1e-12
        assert math.fsum(top[:k - 1]) < ff * total + 1e-12


def test_exact_prefix_sums_match_correctly_rounded_sums():
    # each exact prefix, rounded once, is the correctly rounded sum (fsum)
    from fractions import Fraction
    rng = np.random.default_rng(3)
    s = np.exp(rng.standard_normal(200) * 20)           # magnitudes over ~17 decades
    c = orc.exact_prefix_sums(s)
    for k in (1, 2, 17, 100, 200):
        assert float(Fraction(c[k - 1], 2 ** 1074)) == math.fsum(s[:k])
    assert orc.exact_prefix_sums([5e-324, 5e-324]) == [1, 2]   # the smallest subnormal is one unit


def test_mass_budget_counts_a_flat_tail_exactly():
    # f = 1 needs every positive score: closed form k = #positive.  The tail
    # scores sit far below one ulp of the running sum, where a float64
    # cumulative sum stops growing (it would return k = 1).
    s = np.concatenate([[1.0], np.full(50, 1e-20), np.zeros(10)])
    assert orc.budget_count(s, orc.BUDGET_MASS, mass=1.0) == 51
    assert np.cumsum(s)[0] == np.cumsum(s)[-1]           # the float64 cumsum is saturated
    # any fraction below 1 is reached by the head token alone
    assert orc.budget_count(s, orc.BUDGET_MASS, mass=float(np.float32(1.0 - 1e-7))) == 1


def test_per_head_ctx_and_arrays():
    s = np.random.default_rng(0).random((2, 2, 12))
    kept, cnt = orc.select(s, [12, 5], orc.BUDGET_RATIO, ratio=[0.5, 0.25, 1.0, 0.5])
    assert list(cnt) == [6, 3, 5, 3]
    assert np.all(kept[1, 0, :5] < 5)


def _case(seed, B=2, Hkv=2, N=16, d=8, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn(B, Hkv, N, d, generator=g).to(dtype)
    v = torch.randn(B, Hkv, N, d, generator=g).to(dtype)
    return k, v


def test_compact_is_a_bitwise_ordered_gather():
    k, v = _case(1)
    s = np.random.default_rng(1).random((2, 2, 16))
    kept, cnt = orc.select(s, None, orc.BUDGET_K, k=5)
    kc, vc, pos, off = orc.compact(k, v, kept, cnt)
    assert list(off) == [0, 5, 10, 15, 20]
    kb = k.view(torch.int16).numpy()
    vb = v.view(torch.int16).numpy()
    for i, (b, h) in enumerate([(0, 0), (0, 1), (1, 0), (1, 1)]):
        rows = pos[off[i]:off[i + 1]]
        assert np.all(np.diff(rows) > 0)
        assert np.array_equal(kc[off[i]:off[i + 1]], kb[b, h, rows])
        assert np.array_equal(vc[off[i]:off[i + 1]], vb[b, h, rows])


def test_full_keep_compaction_is_identity():
    k, v = _case(2)
    s = np.random.default_rng(2).random((2, 2, 16))
    kept, cnt = orc.select(s, None, orc.BUDGET_RATIO, ratio=1.0)
    kc, vc, pos, off = orc.compact(k, v, kept, cnt)
    assert np.array_equal(kc.reshape(2, 2, 16, 8), k.view(torch.int16).numpy())
    assert np.array_equal(pos, np.tile(np.arange(16), 4))


def test_decode_matches_torch_sdpa():
    # library routine: scaled_dot_product_attention in float64 on the CPU
    rng = np.random.default_rng(4)
    B, Hq, Hkv, d = 2, 4, 2, 16
    counts = np.array([5, 9, 1, 7])
    off = np.concatenate([[0], np.cumsum(counts)])
    kc = rng.standard_normal((off[-1], d))
    vc = rng.standard_normal((off[-1], d))
    q = rng.standard_normal((B, Hq, d))
    out, lse = orc.decode(q, kc, vc, off, Hkv)
    G = Hq // Hkv
    for b in range(B):
        for j in range(Hq):
            i = b * Hkv + j // G
            K = torch.from_numpy(kc[off[i]:off[i + 1]])[None, None]
            V = torch.from_numpy(vc[off[i]:off[i + 1]])[None, None]
            Q = torch.from_numpy(q[b, j])[None, None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V)
            np.testing.assert_allclose(out[b, j], ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-14)
            o_b, l_b = brute.attend(list(q[b, j]), kc[off[i]:off[i + 1]].tolist(),
                                    vc[off[i]:off[i + 1]].tolist(), 1 / math.sqrt(d))
            np.testing.assert_allclose(out[b, j], o_b, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(lse[b, j], l_b, rtol=1e-13)


def test_decode_special_cases():
    rng = np.random.default_rng(6)
    kc = rng.standard_normal((7, 8))
    vc = rng.standard_normal((7, 8))
    off = np.array([0, 6, 7])
    q = np.zeros((1, 2, 8))
    out, lse = orc.decode(q, kc, vc, off, 2)
    np.testing.assert_allclose(out[0, 0], vc[:6].mean(axis=0), rtol=1e-13)
    np.testing.assert_allclose(lse[0, 0], math.log(6), rtol=1e-14)
    q = rng.standard_normal((1, 2, 8))
    out, lse = orc.decode(q, kc, vc, off, 2)
    assert np.array_equal(out[0, 1], vc[6])                  # one row: that row
    np.testing.assert_allclose(lse[0, 1], kc[6] @ q[0, 1] / math.sqrt(8), rtol=1e-14)


def test_full_keep_reproduces_full_attention_exactly():
    k, v = _case(3, N=24)
    q = torch.randn(2, 4, 8, generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    s = np.random.default_rng(3).random((2, 2, 24))
    kept, cnt = orc.select(s, [24, 19], orc.BUDGET_RATIO, ratio=1.0)
    kc, vc, pos, off = orc.compact(k, v, kept, cnt)
    kc_t = torch.from_numpy(kc).view(torch.bfloat16)
    vc_t = torch.from_numpy(vc).view(torch.bfloat16)
    out, lse = orc.decode(q, kc_t, vc_t, off, 2)
    out_f, lse_f = orc.attend_full(q, k, v, [24, 19])
    assert np.array_equal(out, out_f) and np.array_equal(lse, lse_f)


# ---- protected sinks and recent window ------------------------------------

PROT_CASES = [(0, 0), (2, 0), (0, 3), (2, 3), (4, 9), (20, 0), (1, 30)]


def _tied_scores(rng, n):
    # few distinct values so that ties are common
    return rng.integers(0, 5, size=n).astype(np.float64) / 4.0


@pytest.mark.parametrize("n_sink,n_recent", PROT_CASES)
def test_protected_topk_matches_brute_force(n_sink, n_recent):
    rng = np.random.default_rng(40 + n_sink + 7 * n_recent)
    n = 17
    for trial in range(6):
        s = _tied_scores(rng, n)
        prot = orc.protected_mask(n, n_sink, n_recent)
        for k in (1, 3, 8, 17):
            idx, cnt = orc.select(s[None, None, :], None, orc.BUDGET_K, k=k,
                                  n_sink=n_sink, n_recent=n_recent)
            expect = brute.top_k_protected(list(s), list(prot), k)
            assert idx[0, 0, :cnt[0]].tolist() == expect
            # protected tokens are always kept
            assert set(np.flatnonzero(prot)) <= set(expect)


def test_protected_mask_union_and_overlap():
    assert orc.protected_mask(10, 2, 3).tolist() == [1, 1, 0, 0, 0, 0, 0, 1, 1, 1]
    assert orc.protected_mask(5, 4, 4).all()          # overlap covers everything
    assert not orc.protected_mask(6, 0, 0).any()
    assert orc.protected_mask(4, 9, 0).all()          # longer than the head


@pytest.mark.parametrize("n_sink,n_recent", PROT_CASES)
def test_protected_threshold_is_union(n_sink, n_recent):
    # Without clamps the kept set is the protected tokens plus every token at
    # or above tau (a set definition, no counting).
    rng = np.random.default_rng(3 + n_sink)
    n = 23
    s = rng.random(n)
    for tau in (0.2, 0.5, 0.9, 2.0):
        idx, cnt = orc.select(s[None, None, :], None, orc.BUDGET_THRESHOLD, tau=tau,
                              n_sink=n_sink, n_recent=n_recent)
        prot = orc.protected_mask(n, n_sink, n_recent)
        want = sorted(set(np.flatnonzero(prot)) | set(np.flatnonzero(s >= np.float32(tau))))
        if not want:      # nothing qualifies: one token, the lowest-index maximum
            want = [int(np.argmax(s))]
        assert idx[0, 0, :cnt[0]].tolist() == want


@pytest.mark.parametrize("n_sink,n_recent", PROT_CASES)
def test_protected_mass_matches_brute_force(n_sink, n_recent):
    rng = np.random.default_rng(11 + n_recent)
    n = 15
    for trial in range(5):
        s = list(rng.random(n) ** 3)
        prot = list(orc.protected_mask(n, n_sink, n_recent))
        for f in (0.3, 0.6, 0.95):
            idx, cnt = orc.select(np.array(s)[None, None, :], None, orc.BUDGET_MASS,
                                  mass=f, n_sink=n_sink, n_recent=n_recent)
            k = max(brute.mass_count_protected(s, prot, float(np.float32(f))), sum(prot))
            assert cnt[0] == min(k, n)
            assert idx[0, 0, :cnt[0]].tolist() == brute.top_k_protected(s, prot, k)


def test_protected_zero_is_plain_selection():
    rng = np.random.default_rng(5)
    s = rng.random((2, 3, 50))
    for mode, p in ((orc.BUDGET_RATIO, {"ratio": 0.2}), (orc.BUDGET_MASS, {"mass": 0.7})):
        a = orc.select(s, None, mode, **p)
        b = orc.select(s, None, mode, n_sink=0, n_recent=0, **p)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---- fidelity of a compacted cache (output and log-sum-exp terms) ----------

def test_fidelity_full_keep_is_zero():
    rng = np.random.default_rng(31)
    B, Hkv, G, N, d = 2, 2, 2, 30, 8
    k = rng.standard_normal((B, Hkv, N, d)); v = rng.standard_normal((B, Hkv, N, d))
    q = rng.standard_normal((B, Hkv * G, d))
    ctx = [30, 17]
    idx = np.tile(np.arange(N, dtype=np.int32), (B, Hkv, 1))
    cnt = np.repeat(np.array(ctx, np.int32), Hkv)
    f = orc.fidelity(q, k, v, idx, cnt, ctx)
    assert np.abs(f["out_err2"]).max() < 1e-24 and np.abs(f["lse_diff"]).max() < 1e-12


def test_fidelity_matches_brute_force():
    # exp(l^ - l) is the full softmax mass on the kept rows (so l^ <= l), and
    # Y^ is attention over the kept rows alone: both from pure-Python loops.
    rng = np.random.default_rng(32)
    B, Hkv, G, N, d = 1, 2, 2, 12, 4
    k = rng.standard_normal((B, Hkv, N, d)); v = rng.standard_normal((B, Hkv, N, d))
    q = rng.standard_normal((B, Hkv * G, d))
    s = rng.random((B, Hkv, N))
    idx, cnt = orc.select(s, None, orc.BUDGET_K, k=5)
    f = orc.fidelity(q, k, v, idx, cnt)
    scale = 1.0 / math.sqrt(d)
    for h in range(Hkv):
        kept = idx[0, h, :5].tolist()
        for g in range(G):
            j = h * G + g
            y, l = brute.attend(list(q[0, j]), [list(r) for r in k[0, h]], [list(r) for r in v[0, h]], scale)
            yh, lh = brute.attend(list(q[0, j]), [list(k[0, h, t]) for t in kept],
                                  [list(v[0, h, t]) for t in kept], scale)
            u = [scale * math.fsum(a * b for a, b in zip(q[0, j], k[0, h, t])) for t in range(N)]
            mass = math.fsum(math.exp(u[t] - l) for t in kept)
            assert f["lse_diff"][0, j] <= 0.0
            assert math.isclose(math.exp(f["lse_diff"][0, j]), mass, rel_tol=1e-12)
            assert math.isclose(f["lse_diff"][0, j], lh - l, abs_tol=1e-12)
            assert math.isclose(f["out_err2"][0, j], math.fsum((a - b) ** 2 for a, b in zip(yh, y)),
                                rel_tol=1e-10, abs_tol=1e-24)


def test_decode_empty_head():
    # A head with no kept rows: the empty sum gives lse = log 0 = -inf and a
    # zero output; the other heads are the same as without it.
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 4, 8))
    k_c = rng.standard_normal((6, 8))
    v_c = rng.standard_normal((6, 8))
    out, lse = orc.decode(q, k_c, v_c, np.array([0, 0, 6]), 2)   # head 0 empty, G = 2
    assert np.all(out[0, :2] == 0.0) and np.all(np.isneginf(lse[0, :2]))
    out1, lse1 = orc.decode(q[:, 2:], k_c, v_c, np.array([0, 6]), 1)
    np.testing.assert_allclose(out[0, 2:], out1[0], rtol=1e-15, atol=0)
    np.testing.assert_allclose(lse[0, 2:], lse1[0], rtol=1e-15, atol=0)
