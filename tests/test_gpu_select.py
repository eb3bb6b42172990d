"""kv_select on the GPU vs the oracle's selection on the same fp32 scores."""
import math

import numpy as np
import pytest
import torch

from kv_cache_compression_score_amd import api
from kv_cache_compression_score_amd import workloads as wl
from oracle import oracle as orc

from gpu_helpers import MASS_BAND, dev, log, mass_between, mass_count_ok

pytestmark = pytest.mark.gpu


def synth_scores(seed, B, Hkv, N, ctx, kind):
    rng = np.random.default_rng(seed)
    if kind == "ties":        # few distinct values: long runs of equal keys
        s = rng.integers(0, 7, size=(B, Hkv, N)).astype(np.float32) / 8
    elif kind == "zeros":     # mostly zeros, half of them -0.0
        s = np.where(rng.random((B, Hkv, N)) < 0.9, 0.0, rng.random((B, Hkv, N)))
        s = s.astype(np.float32)
        s[(s == 0) & (rng.random((B, Hkv, N)) < 0.5)] = np.float32(-0.0)
    elif kind == "twobins":   # 60% and 35% of the keys in two top-digit bins, 5% spread
        u = rng.random((B, Hkv, N))
        j = 1 + rng.random((B, Hkv, N)) * 2.0 ** -8      # leaves the top digit alone
        s = np.where(u < 0.6, 0.5 * j, np.where(u < 0.95, 0.25 * j, rng.random((B, Hkv, N))))
        s = s.astype(np.float32)
    elif kind == "heavy":     # softmax-like heavy tail over many decades
        s = np.exp(rng.standard_normal((B, Hkv, N)) * 6).astype(np.float32)
    else:                     # plain uniform
        s = rng.random((B, Hkv, N)).astype(np.float32)
    for b in range(B):
        s[b, :, ctx[b]:] = np.float32(rng.random())     # garbage beyond n_b
    return s


def run_select(s_np, ctx, budget):
    s = torch.from_numpy(s_np).cuda()
    c = torch.tensor(ctx, dtype=torch.int32).cuda()
    idx, cnt = api.kv_select(s, c, budget)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


def compare_sets(idx_g, cnt_g, idx_r, cnt_r):
    assert np.array_equal(cnt_g, cnt_r), (cnt_g, cnt_r)
    B, Hkv = idx_r.shape[:2]
    for b in range(B):
        for h in range(Hkv):
            k = int(cnt_r[b * Hkv + h])
            assert np.array_equal(idx_g[b, h, :k], idx_r[b, h, :k]), (b, h)


KINDS = ["ties", "zeros", "heavy", "uniform"]
# 12001: a ragged batch whose row length is not a multiple of 4 (the
# scalar staging path), with a head of 4097 tokens and one of a single token.
SHAPES = [(2, 3, 1000, [1000, 517]), (1, 2, 32768, [32768]), (1, 2, 40000, [40000]),
          (3, 1, 64, [64, 1, 63]), (3, 2, 12001, [12001, 4097, 1])]


@pytest.mark.parametrize("kind", ["ties", "zeros", "heavy", "uniform"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}H{s[1]}N{s[2]}")
def test_select_ratio_and_k(kind, shape):
    B, Hkv, N, ctx = shape
    log(f"select ratio/k {kind} {shape}")
    s = synth_scores(KINDS.index(kind) * 100003 + N, B, Hkv, N, ctx, kind)
    for r in (0.1, 0.5, 1.0, 0.0):
        idx_g, cnt_g = run_select(s, ctx, api.Budget(api.BUDGET_RATIO, ratio_scalar=r))
        idx_r, cnt_r = orc.select(s, ctx, orc.BUDGET_RATIO, ratio=r)
        compare_sets(idx_g, cnt_g, idx_r, cnt_r)
    idx_g, cnt_g = run_select(s, ctx, api.Budget(api.BUDGET_K, k_scalar=37))
    idx_r, cnt_r = orc.select(s, ctx, orc.BUDGET_K, k=37)
    compare_sets(idx_g, cnt_g, idx_r, cnt_r)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}H{s[1]}N{s[2]}")
def test_select_per_head_arrays(shape):
    B, Hkv, N, ctx = shape
    s = synth_scores(4, B, Hkv, N, ctx, "heavy")
    rng = np.random.default_rng(1)
    ratios = rng.random(B * Hkv).astype(np.float32)
    ks = rng.integers(-3, N + 5, size=B * Hkv).astype(np.int32)
    idx_g, cnt_g = run_select(s, ctx, api.Budget(api.BUDGET_RATIO,
                                                 ratio=torch.from_numpy(ratios).cuda()))
    idx_r, cnt_r = orc.select(s, ctx, orc.BUDGET_RATIO, ratio=ratios)
    compare_sets(idx_g, cnt_g, idx_r, cnt_r)
    idx_g, cnt_g = run_select(s, ctx, api.Budget(api.BUDGET_K, k=torch.from_numpy(ks).cuda()))
    idx_r, cnt_r = orc.select(s, ctx, orc.BUDGET_K, k=ks)
    compare_sets(idx_g, cnt_g, idx_r, cnt_r)


@pytest.mark.parametrize("kind", ["ties", "heavy", "uniform"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}H{s[1]}N{s[2]}")
def test_select_threshold(kind, shape):
    B, Hkv, N, ctx = shape
    s = synth_scores(7, B, Hkv, N, ctx, kind)
    for tau, lo, hi in [(0.5, 0.0, 1.0), (0.25, 0.0, 1.0), (10.0, 0.0, 1.0),
                        (0.0, 0.0, 0.3), (0.9, 0.2, 0.5)]:
        b = api.Budget(api.BUDGET_THRESHOLD, tau=tau, min_ratio=lo, max_ratio=hi)
        idx_g, cnt_g = run_select(s, ctx, b)
        idx_r, cnt_r = orc.select(s, ctx, orc.BUDGET_THRESHOLD, tau=tau, min_ratio=lo,
                                  max_ratio=hi)
        compare_sets(idx_g, cnt_g, idx_r, cnt_r)


# twobins: the mass descent's crowded-key sums hold a second bin in registers,
# and its first digit's counts serve the count descent of a clamped head
@pytest.mark.parametrize("kind", ["ties", "heavy", "uniform", "twobins"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}H{s[1]}N{s[2]}")
def test_select_mass(kind, shape):
    B, Hkv, N, ctx = shape
    s = synth_scores(9, B, Hkv, N, ctx, kind)
    for f, lo, hi in [(0.95, 0.02, 0.5), (0.5, 0.0, 1.0), (1.0, 0.0, 1.0), (0.0, 0.0, 1.0)]:
        b = api.Budget(api.BUDGET_MASS, mass=f, min_ratio=lo, max_ratio=hi)
        idx_g, cnt_g = run_select(s, ctx, b)
        idx_r, cnt_r = orc.select(s, ctx, orc.BUDGET_MASS, mass=f, min_ratio=lo, max_ratio=hi)
        worst_dk, worst_mass = 0, 0.0
        for bb in range(B):
            for h in range(Hkv):
                i = bb * Hkv + h
                kg, kr = int(cnt_g[i]), int(cnt_r[i])
                sh = s[bb, h, :ctx[bb]].astype(np.float64)
                if kg != kr:
                    # the counts may differ only where the exact prefix sums
                    # stay within the fixed-point band of f * C(n)
                    assert mass_count_ok(sh, kg, f, lo, hi), (bb, h, kg, kr)
                    worst_dk = max(worst_dk, abs(kg - kr))
                    worst_mass = max(worst_mass, mass_between(sh, kg, kr))
                    assert worst_mass <= 2 * MASS_BAND, (bb, h, kg, kr, worst_mass)
                ref = np.sort(orc.total_order(sh)[:kg])
                assert np.array_equal(idx_g[bb, h, :kg], ref), (bb, h)
        log(f"mass {kind} {shape[:3]} f={f}: max |k_gpu - k_oracle| {worst_dk}, "
            f"mass between them {worst_mass:.1e} of the total")


def test_select_on_real_scores_and_determinism():
    cfg = wl.CONFIGS["needle32k"]
    lay = wl.make_layer(cfg, B=1, with_v=False)
    s, _ = api.kv_score(dev(lay.q_win), dev(lay.k), dev(lay.ctx_len))
    c = dev(lay.ctx_len)
    b = api.Budget(api.BUDGET_RATIO, ratio_scalar=cfg.ratio)
    i1, n1 = api.kv_select(s, c, b)
    i2, n2 = api.kv_select(s, c, b)
    torch.cuda.synchronize()
    assert torch.equal(n1, n2)
    for h in range(cfg.Hkv):
        k = int(n1[h])
        assert k == 3277
        assert torch.equal(i1[0, h, :k], i2[0, h, :k])
    idx_r, cnt_r = orc.select(s.cpu().numpy(), lay.ctx_len, orc.BUDGET_RATIO, ratio=cfg.ratio)
    compare_sets(i1.cpu().numpy(), n1.cpu().numpy(), idx_r, cnt_r)


PROT = [(4, 64), (0, 128), (3000, 0), (10, 100000), (1, 1)]


@pytest.mark.parametrize("kind", ["ties", "heavy"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}H{s[1]}N{s[2]}")
def test_select_protected(kind, shape):
    # Sinks and recent window: stage parity on the same fp32 scores in every
    # budget mode (mass counts within the fixed-point bracket), and every
    # protected token is kept.
    B, Hkv, N, ctx = shape
    log(f"select protected {kind} {shape}")
    s = synth_scores(13 + N, B, Hkv, N, ctx, kind)
    for n_sink, n_recent in PROT:
        pr = dict(n_sink=n_sink, n_recent=n_recent)
        cases = [
            (api.Budget(api.BUDGET_RATIO, ratio_scalar=0.05, **pr), dict(mode=orc.BUDGET_RATIO, ratio=0.05)),
            (api.Budget(api.BUDGET_K, k_scalar=3, **pr), dict(mode=orc.BUDGET_K, k=3)),
            (api.Budget(api.BUDGET_THRESHOLD, tau=0.5, min_ratio=0.0, max_ratio=0.3, **pr),
             dict(mode=orc.BUDGET_THRESHOLD, tau=0.5, min_ratio=0.0, max_ratio=0.3)),
        ]
        for bud, ref in cases:
            idx_g, cnt_g = run_select(s, ctx, bud)
            idx_r, cnt_r = orc.select(s, ctx, **ref, **pr)
            compare_sets(idx_g, cnt_g, idx_r, cnt_r)
        for f, lo, hi in [(0.9, 0.02, 0.5), (0.3, 0.0, 1.0)]:
            idx_g, cnt_g = run_select(s, ctx, api.Budget(api.BUDGET_MASS, mass=f, min_ratio=lo,
                                                         max_ratio=hi, **pr))
            idx_r, cnt_r = orc.select(s, ctx, orc.BUDGET_MASS, mass=f, min_ratio=lo,
                                      max_ratio=hi, **pr)
            for bb in range(B):
                n = ctx[bb]
                prot = orc.protected_mask(n, n_sink, n_recent)
                for h in range(Hkv):
                    i = bb * Hkv + h
                    kg, kr = int(cnt_g[i]), int(cnt_r[i])
                    sh = s[bb, h, :n].astype(np.float64)
                    if kg != kr:
                        assert mass_count_ok(sh, kg, f, lo, hi, prot=prot), (bb, h, kg, kr)
                        assert mass_between(sh, kg, kr, prot) <= 2 * MASS_BAND, (bb, h)
                    ref = np.sort(orc.total_order(sh, prot)[:kg])
                    assert np.array_equal(idx_g[bb, h, :kg], ref), (bb, h)
                    assert set(np.flatnonzero(prot)) <= set(idx_g[bb, h, :kg].tolist())



@pytest.mark.parametrize("shape", [(2, 2, 70001, [70001, 40000]), (1, 2, 300001, [300001])],
                         ids=["N70001", "N300001"])
@pytest.mark.parametrize("kind", KINDS)
def test_select_long_heads_parts_equal_one_workgroup(kind, shape):
    # Heads above 32768 tokens under a count budget are split over several
    # workgroups when the workspace is given; without it one workgroup per
    # head selects.  Both must give the same kept indices, bit for bit, and
    # match the oracle.  300001 tokens make 19 parts: the last launch places
    # each part after the earlier ones sixteen parts at a time, so it takes
    # two rounds there.
    from kv_cache_compression_score_amd import _lib
    import ctypes
    B, Hkv, N, ctx = shape
    log(f"select parts {kind} {shape[:3]}")
    s_np = synth_scores(KINDS.index(kind) * 7919 + 5, B, Hkv, N, ctx, kind)
    s = torch.from_numpy(s_np).cuda()
    c = torch.tensor(ctx, dtype=torch.int32).cuda()
    L = _lib.lib()
    need = int(L.kv_select_workspace_size(B, Hkv, N))
    assert need > 0
    ws = torch.empty(need, device="cuda", dtype=torch.uint8)
    buds = [(api.Budget(api.BUDGET_RATIO, ratio_scalar=0.1), dict(mode=orc.BUDGET_RATIO, ratio=0.1)),
            (api.Budget(api.BUDGET_K, k_scalar=5000), dict(mode=orc.BUDGET_K, k=5000)),
            (api.Budget(api.BUDGET_THRESHOLD, tau=float(np.median(s_np[0, 0, :40000])),
                        min_ratio=0.02, max_ratio=0.5),
             dict(mode=orc.BUDGET_THRESHOLD, tau=float(np.median(s_np[0, 0, :40000])),
                  min_ratio=0.02, max_ratio=0.5)),
            (api.Budget(api.BUDGET_RATIO, ratio_scalar=0.05, n_sink=4, n_recent=300),
             dict(mode=orc.BUDGET_RATIO, ratio=0.05, n_sink=4, n_recent=300))]
    for bud, ref in buds:
        out = []
        for w, nb in ((ws, need), (None, 0)):
            idx = torch.full((B, Hkv, N), -1, device="cuda", dtype=torch.int32)
            cnt = torch.zeros(B * Hkv, device="cuda", dtype=torch.int32)
            cb = bud.to_c()
            st = L.kv_select(api._ptr(s), api._ptr(c), B, Hkv, N, ctypes.byref(cb), api._ptr(idx),
                             api._ptr(cnt), api._ptr(w), nb, api._stream())
            assert st == 0, st
            torch.cuda.synchronize()
            out.append((idx.cpu().numpy(), cnt.cpu().numpy()))
        (i_p, c_p), (i_1, c_1) = out
        assert np.array_equal(c_p, c_1)
        for h in range(B * Hkv):
            k = int(c_p[h])
            assert np.array_equal(i_p.reshape(B * Hkv, N)[h, :k], i_1.reshape(B * Hkv, N)[h, :k]), h
        mode = ref.pop("mode")
        idx_r, cnt_r = orc.select(s_np, ctx, mode, **ref)
        compare_sets(i_p, c_p, idx_r, cnt_r)
