"""VECTOR three-way routing on the GPU vs the float64 oracle.

Inputs: seeded keys and queries from the shared generator, a random linear
map W per KV head, and values V = W RoPE^-1(K) + noise (so residuals vary
and some rows are well reconstructed).  Stage parity: the pool is compared
exactly with the oracle's selection on the same fp32 scores, the residuals
within 1e-3 relative, and the approximated subset exactly with the oracle's
selection on the GPU's own fp32 residuals (both sides decide in fp32).
"""
import math

import numpy as np
import pytest
import torch

from kv_cache_compression_score_amd import api
from kv_cache_compression_score_amd import workloads as wl
from oracle import oracle as orc

from gpu_helpers import bits, dev, log

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, N, d, dtype, ctx, rope_base, p_c, p_a
    (2, 8, 2, 3000, 128, torch.bfloat16, [3000, 1700], 10000.0, 0.9, 0.05),
    (1, 4, 4, 1024, 64, torch.float32, None, 0.0, 0.75, 0.125),
    (1, 4, 1, 40000, 128, torch.bfloat16, None, 500000.0, 0.9, 0.05),
    (2, 4, 2, 500, 64, torch.bfloat16, [500, 37], 10000.0, 0.5, 0.0),
    (1, 2, 1, 300, 128, torch.bfloat16, None, 10000.0, 0.2, 0.4),
]


def make_case(c, seed=5):
    B, Hq, Hkv, N, d, dt, ctx, base, p_c, p_a = c
    lay = wl.random_case(seed, B=B, Hq=Hq, Hkv=Hkv, d=d, N_max=N, W=8, dtype=dt, ctx=ctx)
    rng = np.random.default_rng(seed + 1)
    w = (rng.standard_normal((Hkv, d, d)) / math.sqrt(d)).astype(np.float32)
    k64 = lay.k.double().numpy()
    v = np.zeros((B, Hkv, N, d))
    n_b = lay.ctx_len.numpy()
    for b in range(B):
        for h in range(Hkv):
            n = int(n_b[b])
            kt = orc.rope_inverse(k64[b, h, :n], np.arange(n), base)
            noise = rng.standard_normal((n, d)) * rng.choice([0.02, 0.3, 1.0], size=(n, 1))
            v[b, h, :n] = kt @ w[h].astype(np.float64).T + noise
    v_t = torch.from_numpy(v.astype(np.float32)).to(dt)
    s = rng.random((B, Hkv, N)).astype(np.float32) ** 4
    return lay, torch.from_numpy(w), v_t, s


@pytest.mark.parametrize("c", CASES, ids=lambda c: f"B{c[0]}Hkv{c[2]}N{c[3]}d{c[4]}"
                         f"{'f32' if c[5] == torch.float32 else 'bf16'}b{int(c[7])}pa{c[9]}")
def test_vector_route_compact_decode(c):
    B, Hq, Hkv, N, d, dt, ctx, base, p_c, p_a = c
    log(f"vector case {c}")
    lay, w, v, s = make_case(c)
    k_d, v_d, w_d, c_d = dev(lay.k), dev(v), dev(w), dev(lay.ctx_len)
    s_d = torch.from_numpy(s).cuda()
    pool_idx, pool_count, neg_eps, apx_pos, apx_count = api.kv_vector_route(
        s_d, c_d, k_d, v_d, w_d, p_c=p_c, p_a=p_a, rope_base=base)
    torch.cuda.synchronize()
    pi, pc = pool_idx.cpu().numpy(), pool_count.cpu().numpy()
    ne, ap, ac = neg_eps.cpu().numpy(), apx_pos.cpu().numpy(), apx_count.cpu().numpy()
    n_b = lay.ctx_len.numpy()

    # pool: exact against the oracle's selection on the same scores
    kp = np.array([orc.vector_counts(int(n_b[b]), p_c, p_a)[0] for b in range(B) for _ in range(Hkv)])
    ri, rc = orc.select(s, lay.ctx_len, orc.BUDGET_K, k=kp)
    assert np.array_equal(pc, rc)
    for b in range(B):
        for h in range(Hkv):
            i = b * Hkv + h
            assert np.array_equal(pi[b, h, :pc[i]], ri[b, h, :rc[i]])
    # residuals within 1e-3 relative of the float64 oracle
    eps_ref = orc.vector_residuals(lay.k, v, w, pi, pc, base)
    for b in range(B):
        for h in range(Hkv):
            cnt = int(pc[b * Hkv + h])
            np.testing.assert_allclose(-ne[b, h, :cnt], eps_ref[b, h, :cnt], rtol=1e-3,
                                       atol=1e-4 * d)
            assert np.all(np.isneginf(ne[b, h, cnt:]))
    # approximated subset: exact against a float selection on the GPU's residuals
    for b in range(B):
        ka = orc.vector_counts(int(n_b[b]), p_c, p_a)[1]
        for h in range(Hkv):
            i = b * Hkv + h
            cnt = int(pc[i])
            order = np.lexsort((np.arange(cnt), -ne[b, h, :cnt].astype(np.float64)))
            assert ac[i] == ka
            assert np.array_equal(ap[b, h, :ka], np.sort(order[:ka]))

    # compaction: key rows for the pool, value rows for the exact entries
    cap = int(pc.sum())
    vcap = int(cap - ac.sum())
    k_c, v_c, pos, vmap, off, voff = api.kv_vector_compact(k_d, v_d, pool_idx, pool_count,
                                                           apx_pos, apx_count, cap, vcap)
    torch.cuda.synchronize()
    kb, vb = bits(lay.k), bits(v)
    k_cb, v_cb = bits(k_c.cpu()), bits(v_c.cpu())
    vm, ps, of, vo = vmap.cpu().numpy(), pos.cpu().numpy(), off.cpu().numpy(), voff.cpu().numpy()
    apx_mask = np.zeros((B, Hkv, N), dtype=bool)
    for b in range(B):
        for h in range(Hkv):
            i = b * Hkv + h
            cnt = int(pc[i])
            toks = pi[b, h, :cnt]
            assert of[i + 1] - of[i] == cnt
            assert np.array_equal(ps[of[i]:of[i + 1]], toks)
            assert np.array_equal(k_cb[of[i]:of[i + 1]], kb[b, h, toks])
            a_m = np.zeros(cnt, dtype=bool)
            a_m[ap[b, h, :ac[i]]] = True
            apx_mask[b, h, :cnt] = a_m
            vm_h = vm[of[i]:of[i + 1]]
            assert np.all(vm_h[a_m] == -1)
            assert np.array_equal(vm_h[~a_m], np.arange(vo[i], vo[i + 1]))
            assert np.array_equal(v_cb[vo[i]:vo[i + 1]], vb[b, h, toks[~a_m]])
    assert vo[-1] == vcap and of[-1] == cap

    # decode over the routed cache vs the oracle's routed decode
    out, lse = api.kv_vector_decode(dev(lay.q_dec[0]), k_c, v_c, vmap, pos, off, w_d, Hkv,
                                    v_capacity_rows=vcap, rope_base=base)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.vector_decode(lay.q_dec[0], lay.k, v, w, pi, pc, apx_mask, Hkv, base)
    np.testing.assert_allclose(out.cpu().numpy(), o_ref, atol=1e-2, rtol=0)
    np.testing.assert_allclose(lse.cpu().numpy(), l_ref, atol=1e-3, rtol=0)
    log(f"  pool {cap} rows, exact values {vcap}, max |out err| "
        f"{np.abs(out.cpu().numpy() - o_ref).max():.2e}")


def test_vector_without_approximation_matches_plain_decode():
    c = (1, 8, 2, 2048, 128, torch.bfloat16, None, 10000.0, 0.8, 0.0)
    lay, w, v, s = make_case(c, seed=9)
    k_d, v_d, w_d = dev(lay.k), dev(v), dev(w)
    s_d = torch.from_numpy(s).cuda()
    pool_idx, pool_count, _, apx_pos, apx_count = api.kv_vector_route(
        s_d, None, k_d, v_d, w_d, p_c=0.8, p_a=0.0, rope_base=10000.0)
    cap = int(pool_count.sum().item())
    k_c, v_c, pos, vmap, off, voff = api.kv_vector_compact(k_d, v_d, pool_idx, pool_count,
                                                           apx_pos, apx_count, cap, cap)
    qd = dev(lay.q_dec[0])
    out, lse = api.kv_vector_decode(qd, k_c, v_c, vmap, pos, off, w_d, 2, v_capacity_rows=cap,
                                    rope_base=10000.0)
    kc2, vc2, _, off2 = api.kv_compact(k_d, v_d, pool_idx, pool_count, cap)
    out2, lse2 = api.kv_decode_attn(qd, kc2, vc2, off2, 2)
    torch.cuda.synchronize()
    assert int(apx_count.sum().item()) == 0
    np.testing.assert_allclose(out.cpu().numpy(), out2.cpu().numpy(), atol=1e-5, rtol=0)
    np.testing.assert_allclose(lse.cpu().numpy(), lse2.cpu().numpy(), atol=1e-5, rtol=0)
