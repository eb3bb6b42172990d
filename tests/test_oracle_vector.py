"""Pins for the VECTOR three-way routing oracle (CPU only)."""
import math

import numpy as np
import pytest

from oracle import brute
from oracle import oracle as orc


def test_rope_inverse_undoes_forward_rotation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 8))
    pos = [0, 1, 7, 100, 4096]
    fwd = np.array([brute.rope_rotate(list(x[m]), pos[m], 10000.0, +1.0) for m in range(5)])
    back = orc.rope_inverse(fwd, pos, 10000.0)
    np.testing.assert_allclose(back, x, atol=1e-12)
    # rotations keep norms, position 0 and base 0 are the identity
    np.testing.assert_allclose(np.linalg.norm(fwd, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    np.testing.assert_allclose(orc.rope_inverse(x, [0] * 5, 500.0), x, atol=0)
    np.testing.assert_allclose(orc.rope_inverse(x, pos, 0.0), x, atol=0)


def test_rope_inverse_single_pair_closed_form():
    # d = 2: the only frequency is base^0 = 1, so position 1 turns by one radian
    y = orc.rope_inverse(np.array([[1.0, 0.0]]), [1], 10000.0)
    np.testing.assert_allclose(y[0], [math.cos(1.0), -math.sin(1.0)], atol=1e-15)


@pytest.mark.parametrize("n,p_c,p_a,pool,apx", [(1000, 0.9, 0.05, 150, 100), (1000, 0.5, 0.0, 500, 0),
                                                (10, 0.75, 0.125, 4, 3), (7, 0.99, 0.2, 1, 1),
                                                (32768, 0.9, 0.05, 4915, 3277)])
def test_vector_counts(n, p_c, p_a, pool, apx):
    assert orc.vector_counts(n, p_c, p_a) == (pool, apx)


def _case(seed, B=1, Hkv=2, N=14, d=6, noise=0.3):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, Hkv, N, d))
    w = rng.standard_normal((Hkv, d, d)) / math.sqrt(d)
    v = np.empty_like(k)
    for b in range(B):
        for h in range(Hkv):
            kt = orc.rope_inverse(k[b, h], np.arange(N), 50.0)
            v[b, h] = kt @ w[h].T + noise * rng.standard_normal((N, d))
    s = rng.random((B, Hkv, N))
    return k, v, w, s


@pytest.mark.parametrize("p_c,p_a", [(0.5, 0.15), (0.3, 0.2), (0.7, 0.1)])
def test_vector_route_matches_brute_force(p_c, p_a):
    k, v, w, s = _case(3)
    pool_idx, pool_count, eps, apx = orc.vector_route(s, k, v, w, None, p_c, p_a, 50.0)
    N = k.shape[2]
    kp, ka = orc.vector_counts(N, p_c, p_a)
    for h in range(2):
        pool = brute.top_k(list(s[0, h]), kp)
        assert pool_idx[0, h, :kp].tolist() == pool and pool_count[h] == kp
        e = [brute.residual(list(v[0, h, t]), list(k[0, h, t]), [list(r) for r in w[h]], t, 50.0)
             for t in pool]
        np.testing.assert_allclose(eps[0, h, :kp], e, rtol=1e-10)
        # the ka lowest residuals (pairwise rank on -eps, lower entry on ties)
        want = brute.top_k([-x for x in e], ka) if ka else []
        assert np.flatnonzero(apx[0, h, :kp]).tolist() == want
        assert not apx[0, h, kp:].any()


def test_vector_without_approximation_is_plain_decode():
    k, v, w, s = _case(4)
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 4, 6))
    pool_idx, pool_count, eps, apx = orc.vector_route(s, k, v, w, None, 0.5, 0.0, 50.0)
    assert not apx.any()
    out, lse = orc.vector_decode(q, k, v, w, pool_idx, pool_count, apx, 2, 50.0)
    idx, cnt = orc.select(s, None, orc.BUDGET_RATIO, ratio=0.5)
    k_c, v_c, _, off = orc.compact(k, v, idx, cnt)
    out2, lse2 = orc.decode(q, k_c, v_c, off, 2)
    np.testing.assert_allclose(out, out2, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, atol=1e-12)


def test_vector_exact_map_reconstructs_values():
    # V = W RoPE^-1(K) exactly: every residual is 0 and the routed decode
    # equals decode over the whole pool with its true values.
    k, v, w, s = _case(5, noise=0.0)
    rng = np.random.default_rng(10)
    q = rng.standard_normal((1, 4, 6))
    pool_idx, pool_count, eps, apx = orc.vector_route(s, k, v, w, None, 0.4, 0.2, 50.0)
    assert np.abs(eps[np.isfinite(eps)]).max() < 1e-24
    assert apx.sum() == 2 * orc.vector_counts(14, 0.4, 0.2)[1]
    out, lse = orc.vector_decode(q, k, v, w, pool_idx, pool_count, apx, 2, 50.0)
    k_c, v_c, _, off = orc.compact(k, v, pool_idx, pool_count)
    out2, lse2 = orc.decode(q, k_c, v_c, off, 2)
    np.testing.assert_allclose(out, out2, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, atol=1e-15)
