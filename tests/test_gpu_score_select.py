"""kv_score_select (the score sweep also histograms the top key bits, and
the selection starts from that histogram) against kv_score followed by
kv_select: scores, row LSEs, kept counts and kept indices equal bit for bit,
under the budgets that take the histogram path and under those that fall
back to the plain selection."""
import numpy as np
import pytest
import torch

from kv_cache_compression_score_amd import api
from kv_cache_compression_score_amd import workloads as wl
from oracle import oracle as orc

from gpu_helpers import check_band, check_scores, dev, log

pytestmark = pytest.mark.gpu


def both(lay, budget, causal=False):
    q, k, c = dev(lay.q_win), dev(lay.k), dev(lay.ctx_len)
    s1, l1 = api.kv_score(q, k, c, causal=causal, with_row_lse=True)
    i1, n1 = api.kv_select(s1, c, budget)
    s2, l2, i2, n2 = api.kv_score_select(q, k, c, budget, causal=causal, with_row_lse=True)
    torch.cuda.synchronize()
    B, Hkv = lay.k.shape[:2]
    for bb, n in enumerate(lay.ctx_len.tolist()):   # entries t >= n_b are not written
        assert torch.equal(s1[bb, :, :n].view(torch.int32), s2[bb, :, :n].view(torch.int32))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    assert torch.equal(n1, n2)
    cnt = n1.cpu().numpy()
    a, b = i1.cpu().numpy(), i2.cpu().numpy()
    for bb in range(B):
        for h in range(Hkv):
            kk = int(cnt[bb * Hkv + h])
            assert np.array_equal(a[bb, h, :kk], b[bb, h, :kk]), (bb, h)
    return s2.cpu().numpy(), b, cnt


RATIO = lambda r: api.Budget(api.BUDGET_RATIO, ratio_scalar=r)

CASES = [
    # seed, B, Hq, Hkv, d, N_max, W, dtype, ctx, causal
    (1, 2, 8, 2, 128, 3000, 16, torch.bfloat16, [3000, 1777], False),
    (2, 3, 4, 4, 64, 1001, 8, torch.bfloat16, [1001, 1, 517], False),    # N_max not a multiple of 4
    (3, 1, 4, 4, 64, 1024, 32, torch.float32, None, False),
    (4, 2, 8, 2, 128, 2048, 24, torch.bfloat16, [2048, 900], True),
    (5, 1, 32, 8, 128, 32768, 64, torch.bfloat16, None, False),          # one full 32K head per KV head
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}N{c[5]}d{c[4]}{'c' if c[9] else ''}")
def test_histogram_path_equals_score_then_select(case):
    seed, B, Hq, Hkv, d, N, W, dt, ctx, causal = case
    log(f"score_select {case}")
    lay = wl.random_case(seed, B=B, Hq=Hq, Hkv=Hkv, d=d, N_max=N, W=W, dtype=dt, ctx=ctx)
    for r in (0.1, 0.5, 1.0, 0.0):
        both(lay, RATIO(r), causal)
    both(lay, api.Budget(api.BUDGET_K, k_scalar=37), causal)
    ks = np.random.default_rng(seed).integers(-2, N + 3, size=B * Hkv).astype(np.int32)
    both(lay, api.Budget(api.BUDGET_K, k=dev(torch.from_numpy(ks))), causal)
    ratios = np.random.default_rng(seed + 1).random(B * Hkv).astype(np.float32)
    both(lay, api.Budget(api.BUDGET_RATIO, ratio=dev(torch.from_numpy(ratios))), causal)


def test_all_scores_tied():
    # identical key rows: every token of a head gets the same score, so the
    # k-th key's top-digit bin holds the whole head (ties to the lowest index)
    lay = wl.random_case(9, B=2, Hq=4, Hkv=2, d=128, N_max=4096, W=16, ctx=[4096, 3001])
    lay.k[:] = lay.k[:, :, :1, :]
    for b, n in enumerate([4096, 3001]):
        lay.k[b, :, n:] = 0
    s, idx, cnt = both(lay, RATIO(0.3))
    for b, n in enumerate([4096, 3001]):
        for h in range(2):
            k = int(cnt[b * 2 + h])
            assert np.array_equal(idx[b, h, :k], np.arange(k))


def test_half_the_tokens_tied():
    # every other key row is one repeated row: half of a head's scores are
    # equal (one crowded bin at every digit) and the rest spread; the k-th
    # key falls inside the tied block at some ratios and outside at others
    lay = wl.random_case(10, B=2, Hq=8, Hkv=2, d=128, N_max=6000, W=16, ctx=[6000, 4099])
    lay.k[:, :, 1::2] = lay.k[:, :, :1]
    for b, n in enumerate([6000, 4099]):
        lay.k[b, :, n:] = 0
    for r in (0.05, 0.3, 0.5, 0.7, 0.95):
        both(lay, RATIO(r))


@pytest.mark.parametrize("budget", [
    api.Budget(api.BUDGET_THRESHOLD, tau=0.01, min_ratio=0.02, max_ratio=0.5),
    api.Budget(api.BUDGET_MASS, mass=0.9, min_ratio=0.02, max_ratio=0.5),
    api.Budget(api.BUDGET_RATIO, ratio_scalar=0.1, n_sink=4, n_recent=32),
], ids=["threshold", "mass", "protected"])
def test_fallback_budgets(budget):
    lay = wl.random_case(11, B=2, Hq=8, Hkv=2, d=128, N_max=3000, W=16, ctx=[3000, 1500])
    both(lay, budget)


def test_heads_above_32k_take_the_part_path_from_the_histogram():
    # above 32768 tokens the part path starts from the score pass's
    # histogram (its first launch skipped) under k and kept-fraction budgets
    lay = wl.random_case(12, B=1, Hq=8, Hkv=2, d=128, N_max=40000, W=16)
    both(lay, RATIO(0.1))
    # ragged lengths (one head below 32K, one not a multiple of 4), N_max
    # odd (scalar loads), half of every head tied, per-head k and fractions
    log("score_select: part path, ragged, tied")
    lay = wl.random_case(13, B=2, Hq=8, Hkv=2, d=128, N_max=70001, W=16, ctx=[70001, 20003])
    lay.k[:, :, 1::2] = lay.k[:, :, :1]
    for b, n in enumerate([70001, 20003]):
        lay.k[b, :, n:] = 0
    for r in (0.02, 0.3, 0.5, 0.95, 1.0):
        both(lay, RATIO(r))
    ks = np.array([1, 35001, 70001, 0], dtype=np.int32)
    both(lay, api.Budget(api.BUDGET_K, k=dev(torch.from_numpy(ks))))
    rs = np.array([0.1, 0.6, 0.25, 0.0], dtype=np.float32)
    both(lay, api.Budget(api.BUDGET_RATIO, ratio=dev(torch.from_numpy(rs))))
    # 19 parts: the last launch places each part after the earlier ones
    # sixteen parts at a time (two rounds)
    log("score_select: part path, 300001 tokens")
    lay = wl.random_case(14, B=1, Hq=4, Hkv=1, d=128, N_max=300001, W=16)
    for r in (0.1, 0.6):
        both(lay, RATIO(r))


@pytest.mark.parametrize("name", ["needle32k", "llama8b_layer"])
def test_workloads_match_the_oracle(name):
    # the call the benchmark times, at the workload's full size, against
    # the two calls and (sequence 0) the oracle's scores and kept sets
    cfg = wl.CONFIGS[name]
    lay = wl.make_layer(cfg)
    log(f"score_select {name}")
    s, idx, cnt = both(lay, RATIO(cfg.ratio))
    ctx = lay.ctx_len.numpy()
    s_ref, _ = orc.window_scores(lay.q_win[:1], lay.k[:1], lay.ctx_len[:1])
    err = check_scores(s[:1], s_ref, ctx[:1], cfg.W, cfg.G)
    nd = check_band(idx[:1], cnt[:cfg.Hkv], s_ref, ctx[:1], cfg.W, cfg.G)
    if lay.needle_pos is not None:
        for b in range(cfg.B):
            for h in range(cfg.Hkv):
                kept = set(idx[b, h, :int(cnt[b * cfg.Hkv + h])].tolist())
                assert set(lay.needle_pos[b, h].tolist()) <= kept, (b, h)
    log(f"  score err {err:.2e}, in-band set differences {nd}")
