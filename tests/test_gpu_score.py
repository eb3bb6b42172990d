"""kv_score on the GPU vs the float64 oracle (scores and row log-sum-exps)."""
import numpy as np
import pytest
import torch

from kv_cache_compression_score_amd import api
from kv_cache_compression_score_amd import workloads as wl
from oracle import oracle as orc

from gpu_helpers import check_scores, dev, log

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, W, N_max, d, dtype, causal, ctx
    (1, 4, 4, 32, 1000, 64, torch.float32, False, None),          # fp32, ragged tail
    (2, 8, 2, 16, 777, 128, torch.bfloat16, False, [777, 300]),   # GQA 4, ragged batch
    (1, 8, 2, 24, 1300, 64, torch.bfloat16, True, None),          # causal, W not /32
    (2, 6, 2, 5, 513, 128, torch.float32, True, [513, 64]),       # fp32 d=128, G=3
    (1, 32, 8, 64, 2048, 128, torch.bfloat16, False, None),       # Llama head shape
    (1, 64, 4, 32, 700, 128, torch.bfloat16, False, None),        # G*W = 512 rows
    (1, 4, 1, 256, 300, 64, torch.bfloat16, True, None),          # G*W = 1024 rows
    (1, 4, 2, 40, 40, 64, torch.bfloat16, True, None),            # W = N, one partial tile
    (2, 4, 1, 8, 130, 128, torch.bfloat16, False, [130, 8]),      # a sequence of only W tokens
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}Hq{c[1]}Hkv{c[2]}W{c[3]}N{c[4]}"
                         f"d{c[5]}{'f32' if c[6] == torch.float32 else 'bf16'}{'c' if c[7] else ''}")
def test_score_small(case):
    B, Hq, Hkv, W, N, d, dt, causal, ctx = case
    log(f"score case {case}")
    lay = wl.random_case(11, B=B, Hq=Hq, Hkv=Hkv, d=d, N_max=N, W=W, dtype=dt, ctx=ctx)
    s_gpu, lse_gpu = api.kv_score(dev(lay.q_win), dev(lay.k), dev(lay.ctx_len),
                                  causal=causal, with_row_lse=True)
    torch.cuda.synchronize()
    s_ref, lse_ref = orc.window_scores(lay.q_win, lay.k, lay.ctx_len, causal=causal)
    err = check_scores(s_gpu.cpu().numpy(), s_ref, lay.ctx_len.numpy(), W, Hq // Hkv)
    np.testing.assert_allclose(lse_gpu.cpu().numpy(), lse_ref, atol=1e-3, rtol=0)
    log(f"  max rel score err {err:.3e}")


PARTITION_CASES = [
    # id, B, Hq, Hkv, W, N_max, ctx (None: random lengths in [0, N_max], seeded)
    ("equal_tiles_unequal_lengths", 2, 4, 2, 4, 64, [64, 33]),
    ("uniform_with_lengths", 3, 8, 2, 16, 700, [700, 700, 700]),
    ("uniform_without_lengths", 3, 8, 2, 16, 700, "none"),
    ("20_sequences", 20, 4, 2, 8, 600, None),                 # two groups of 16 lengths
    ("70_sequences_560_heads", 70, 8, 8, 4, 200, None),       # past 64 sequences and 512 heads
    ("one_long_head_among_short", 5, 8, 2, 16, 20000, [20000, 70, 0, 300, 64]),
]


@pytest.mark.parametrize("case", PARTITION_CASES, ids=lambda c: c[0])
def test_score_partition_shapes(case):
    # The score passes split the heads' tiles into pieces from the lengths
    # (pieces never cross a head; equal lengths take the precomputed
    # partition): scores and row LSEs against the oracle, and kv_score_select
    # equal to kv_score + kv_select bit for bit.
    name, B, Hq, Hkv, W, N, ctx = case
    log(f"score partition {name}")
    if ctx is None:
        rng = np.random.default_rng(B * 1000 + N)
        ctx = [int(x) for x in rng.integers(W, N + 1, size=B)]
        ctx[0] = N
        ctx[-1] = W
    ctx_arg = None if ctx == "none" else ctx
    lay = wl.random_case(31, B=B, Hq=Hq, Hkv=Hkv, d=64, N_max=N, W=W, dtype=torch.bfloat16,
                         ctx=ctx_arg)
    c = None if ctx_arg is None else dev(lay.ctx_len)
    s_gpu, lse_gpu = api.kv_score(dev(lay.q_win), dev(lay.k), c, with_row_lse=True)
    budget = api.Budget(api.BUDGET_RATIO, ratio_scalar=0.2)
    s2, lse2, i2, n2 = api.kv_score_select(dev(lay.q_win), dev(lay.k), c, budget, with_row_lse=True)
    i1, n1 = api.kv_select(s_gpu, c, budget)
    torch.cuda.synchronize()
    lens = lay.ctx_len.numpy()
    nz = np.flatnonzero(lens > 0)   # the oracle takes the non-empty sequences
    s_ref, lse_ref = orc.window_scores(lay.q_win[nz], lay.k[nz], lay.ctx_len[nz])
    check_scores(s_gpu.cpu().numpy()[nz], s_ref, lens[nz], W, Hq // Hkv)
    np.testing.assert_allclose(lse_gpu.cpu().numpy()[nz], lse_ref, atol=1e-3, rtol=0)
    if len(nz) < B:   # an empty sequence has no pieces: its rows see nothing
        assert np.all(np.isneginf(lse_gpu.cpu().numpy()[lens == 0]))
    for b, n in enumerate(lens):
        assert torch.equal(s_gpu[b, :, :n].view(torch.int32), s2[b, :, :n].view(torch.int32))
    assert torch.equal(lse_gpu.view(torch.int32), lse2.view(torch.int32))
    assert torch.equal(n1, n2)
    a1, a2, cnt = i1.cpu().numpy(), i2.cpu().numpy(), n1.cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            k = int(cnt[b * Hkv + h])
            assert np.array_equal(a1[b, h, :k], a2[b, h, :k]), (b, h)


def test_score_scale_argument():
    lay = wl.random_case(3, B=1, Hq=4, Hkv=2, d=64, N_max=400, W=8)
    s_gpu, _ = api.kv_score(dev(lay.q_win), dev(lay.k), None, scale=0.3)
    s_ref, _ = orc.window_scores(lay.q_win, lay.k, None, scale=0.3)
    check_scores(s_gpu.cpu().numpy(), s_ref, [400], 8, 2)


def test_score_sum_invariant_and_determinism():
    lay = wl.random_case(5, B=2, Hq=16, Hkv=4, d=128, N_max=3000, W=64, ctx=[3000, 1111])
    q, k, c = dev(lay.q_win), dev(lay.k), dev(lay.ctx_len)
    s1, _ = api.kv_score(q, k, c)
    s2, _ = api.kv_score(q, k, c)
    torch.cuda.synchronize()
    for b, n in enumerate([3000, 1111]):     # entries t >= n are not written
        assert torch.equal(s1[b, :, :n], s2[b, :, :n])
    for b, n in enumerate([3000, 1111]):
        tot = s1[b, :, :n].double().sum(dim=1).cpu().numpy()
        np.testing.assert_allclose(tot, 64 * 4, rtol=1e-4)


def test_score_zero_queries_uniform():
    lay = wl.random_case(8, B=1, Hq=4, Hkv=1, d=64, N_max=640, W=16)
    q = torch.zeros_like(lay.q_win)
    s, _ = api.kv_score(dev(q), dev(lay.k), None)
    np.testing.assert_allclose(s.cpu().numpy(), 64 / 640, rtol=1e-5)


@pytest.mark.parametrize("spread", [40.0, 100.0])
def test_score_far_outlier_logit(spread):
    # One token whose logit (base 2) sits about `spread` above every other
    # one, at a position the row-statistics pass does not sample for its
    # running reference: 40 leaves that reference far below the maximum,
    # 100 makes the block's sum overflow 2^64 and be redone exactly.
    d, W, N = 64, 16, 1024
    lay = wl.random_case(21, B=1, Hq=4, Hkv=1, d=d, N_max=N, W=W)
    rng = np.random.Generator(np.random.PCG64(22))
    base = rng.standard_normal(d).astype(np.float32)
    q = base + 0.1 * rng.standard_normal((1, 4, W, d)).astype(np.float32)
    u = base / np.linalg.norm(base)
    c = np.log2(np.e) / np.sqrt(d)
    t_star = 64 * 5 + 2          # offset 2 of a 32-token block
    k = lay.k.float().numpy().copy()
    k[0, 0, t_star] = u * spread / (c * np.linalg.norm(base))
    q_t = torch.from_numpy(q).to(lay.q_win.dtype)
    k_t = torch.from_numpy(k).to(lay.k.dtype)
    s_gpu, lse_gpu = api.kv_score(dev(q_t), dev(k_t), None, with_row_lse=True)
    torch.cuda.synchronize()
    s_ref, lse_ref = orc.window_scores(q_t, k_t, None)
    assert s_ref[0, 0, t_star] > 0.99 * W * 4
    check_scores(s_gpu.cpu().numpy(), s_ref, [N], W, 4)
    np.testing.assert_allclose(lse_gpu.cpu().numpy(), lse_ref, atol=1e-3, rtol=0)


@pytest.mark.parametrize("N", [4000, 5000])
def test_score_pass1_chunk_merge_paths(N):
    # One KV head: pass 1 cuts 4000 tokens into 16 chunks (pass 2 merges the
    # partials itself) and 5000 into 20 (pass 2 reads the fold's row LSEs).
    # Either way the scores match the oracle, and asking for the row LSEs
    # (which adds the fold launch) leaves the scores bit for bit unchanged.
    lay = wl.random_case(31, B=1, Hq=4, Hkv=1, d=128, N_max=N, W=48, dtype=torch.bfloat16)
    log(f"score chunk merge N={N}")
    q, k = dev(lay.q_win), dev(lay.k)
    s1, _ = api.kv_score(q, k, None, causal=True)
    s2, lse = api.kv_score(q, k, None, causal=True, with_row_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    s_ref, lse_ref = orc.window_scores(lay.q_win, lay.k, None, causal=True)
    check_scores(s1.cpu().numpy(), s_ref, np.array([N]), 48, 4)
    np.testing.assert_allclose(lse.cpu().numpy(), lse_ref, atol=1e-3, rtol=0)


def test_score_llama8b_layer_full():
    cfg = wl.CONFIGS["llama8b_layer"]
    lay = wl.make_layer(cfg, with_v=False)
    log("score llama8b_layer full")
    s_gpu, lse_gpu = api.kv_score(dev(lay.q_win), dev(lay.k), dev(lay.ctx_len), with_row_lse=True)
    torch.cuda.synchronize()
    s_ref, lse_ref = orc.window_scores(lay.q_win, lay.k, lay.ctx_len)
    err = check_scores(s_gpu.cpu().numpy(), s_ref, lay.ctx_len.numpy(), cfg.W, cfg.G)
    np.testing.assert_allclose(lse_gpu.cpu().numpy(), lse_ref, atol=1e-3, rtol=0)
    log(f"  max rel score err {err:.3e}")


def test_score_long128k_sampled_head():
    # Full 128K context and W = 128 (512 rows per head): the oracle checks one
    # head element by element; every head must sum to W * G.
    cfg = wl.CONFIGS["long128k"]
    lay = wl.make_layer(cfg, 0, with_v=False)
    log("score long128k layer 0")
    s_gpu, _ = api.kv_score(dev(lay.q_win), dev(lay.k), dev(lay.ctx_len))
    torch.cuda.synchronize()
    tot = s_gpu.double().sum(dim=2).cpu().numpy()
    np.testing.assert_allclose(tot, cfg.W * cfg.G, rtol=1e-4)
    h = 5
    s_ref, _ = orc.window_scores(lay.q_win[:, h * 4:(h + 1) * 4], lay.k[:, h:h + 1],
                                 lay.ctx_len)
    err = check_scores(s_gpu[:, h:h + 1].cpu().numpy(), s_ref, lay.ctx_len.numpy(), cfg.W, cfg.G)
    log(f"  head {h} max rel score err {err:.3e}")


# ---- one pass from given row LSEs -----------------------------------------

@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}Hq{c[1]}Hkv{c[2]}W{c[3]}N{c[4]}"
                         f"d{c[5]}{'f32' if c[6] == torch.float32 else 'bf16'}{'c' if c[7] else ''}")
def test_score_from_lse_small(case):
    # The oracle's row LSE (rounded to fp32, with one row set to +inf) goes to
    # both sides; the GPU's one-pass scores must match the oracle's.
    B, Hq, Hkv, W, N, d, dt, causal, ctx = case
    log(f"score_from_lse case {case}")
    lay = wl.random_case(12, B=B, Hq=Hq, Hkv=Hkv, d=d, N_max=N, W=W, dtype=dt, ctx=ctx)
    _, lse = orc.window_scores(lay.q_win, lay.k, lay.ctx_len, causal=causal)
    lse32 = lse.astype(np.float32)
    lse32[0, 0, W - 1] = np.inf
    s_gpu = api.kv_score_from_lse(dev(lay.q_win), dev(lay.k), dev(lay.ctx_len),
                                  dev(torch.from_numpy(lse32)), causal=causal)
    torch.cuda.synchronize()
    s_ref = orc.window_scores_from_lse(lay.q_win, lay.k, lse32.astype(np.float64),
                                       lay.ctx_len, causal=causal)
    err = check_scores(s_gpu.cpu().numpy(), s_ref, lay.ctx_len.numpy(), W, Hq // Hkv)
    log(f"  max rel score err {err:.3e}")


def test_score_from_own_lse_equals_two_pass():
    # Feeding back kv_score's own row LSE reproduces its two-pass scores.
    cfg = wl.CONFIGS["llama8b_layer"]
    lay = wl.make_layer(cfg, with_v=False)
    q, k, c = dev(lay.q_win), dev(lay.k), dev(lay.ctx_len)
    s2, lse = api.kv_score(q, k, c, with_row_lse=True)
    s1 = api.kv_score_from_lse(q, k, c, lse)
    torch.cuda.synchronize()
    a, b = s1.double().cpu().numpy(), s2.double().cpu().numpy()
    big = b > 2.0 ** -92 * cfg.W * cfg.G
    rel = np.abs(a - b)[big] / b[big]
    assert rel.max() < 1e-4, rel.max()
    s_ref, _ = orc.window_scores(lay.q_win, lay.k, lay.ctx_len)
    check_scores(s1.cpu().numpy(), s_ref, lay.ctx_len.numpy(), cfg.W, cfg.G)


def test_score_from_lse_needle32k_full():
    # The one-pass entry point at the size bench.py times (4 x 8 heads x 32K,
    # W = 64): fed the two-pass call's row LSE it must reproduce the two-pass
    # scores on every head, and the oracle on sampled heads.
    cfg = wl.CONFIGS["needle32k"]
    lay = wl.make_layer(cfg, with_v=False)
    log("score from lse needle32k")
    q, k, c = dev(lay.q_win), dev(lay.k), dev(lay.ctx_len)
    s2, lse = api.kv_score(q, k, c, with_row_lse=True)
    s1 = api.kv_score_from_lse(q, k, c, lse)
    torch.cuda.synchronize()
    a, b = s1.double().cpu().numpy(), s2.double().cpu().numpy()
    big = b > 2.0 ** -92 * cfg.W * cfg.G
    rel = np.abs(a - b)[big] / b[big]
    assert rel.max() < 1e-4, rel.max()
    np.testing.assert_allclose(a.sum(axis=2), cfg.W * cfg.G, rtol=1e-4)
    for bb, h in [(0, 2), (3, 6)]:
        s_ref, _ = orc.window_scores(lay.q_win[bb:bb + 1, h * cfg.G:(h + 1) * cfg.G],
                                     lay.k[bb:bb + 1, h:h + 1], lay.ctx_len[bb:bb + 1])
        err = check_scores(s1[bb:bb + 1, h:h + 1].cpu().numpy(), s_ref,
                           lay.ctx_len[bb:bb + 1].numpy(), cfg.W, cfg.G)
        log(f"  ({bb}, {h}) max rel score err {err:.3e}")
