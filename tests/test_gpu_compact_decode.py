"""kv_compact (bit-exact) and kv_decode_attn (1e-2 / 1e-3) vs the oracle."""
import numpy as np
import pytest
import torch

from kv_cache_compression_score_amd import api
from kv_cache_compression_score_amd import workloads as wl
from oracle import oracle as orc

from gpu_helpers import bits, check_decode, dev, log

pytestmark = pytest.mark.gpu


def oracle_selection(seed, B, Hkv, N, ctx, ratio):
    s = np.random.default_rng(seed).random((B, Hkv, N))
    return orc.select(s, ctx, orc.BUDGET_RATIO, ratio=ratio)


CASES = [
    # B, Hq, Hkv, N, d, dtype, ctx, ratio
    (2, 8, 2, 1000, 128, torch.bfloat16, [1000, 333], 0.3),
    (1, 4, 4, 1024, 64, torch.float32, None, 0.25),
    (3, 4, 1, 517, 64, torch.bfloat16, [517, 1, 200], 0.5),
    (1, 32, 8, 4096, 128, torch.bfloat16, None, 0.1),
    (2, 6, 2, 300, 128, torch.float32, [300, 129], 1.0),
    (1, 16, 2, 2000, 64, torch.bfloat16, None, 0.9),       # G = 8
    (1, 24, 2, 700, 128, torch.bfloat16, None, 0.2),       # G = 12 (two query sub-groups)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}Hq{c[1]}Hkv{c[2]}N{c[3]}d{c[4]}"
                         f"{'f32' if c[5] == torch.float32 else 'bf16'}r{c[7]}")
def test_compact_then_decode(case):
    B, Hq, Hkv, N, d, dt, ctx, ratio = case
    log(f"compact/decode case {case}")
    lay = wl.random_case(21, B=B, Hq=Hq, Hkv=Hkv, d=d, N_max=N, W=1, dtype=dt, ctx=ctx)
    ctx_l = lay.ctx_len.tolist()
    idx, cnt = oracle_selection(5, B, Hkv, N, ctx_l, ratio)
    total = int(cnt.sum())
    k_c, v_c, pos, off = api.kv_compact(dev(lay.k), dev(lay.v), dev(torch.from_numpy(idx)),
                                        dev(torch.from_numpy(cnt)), total)
    q = dev(lay.q_dec[0])
    out, lse = api.kv_decode_attn(q, k_c, v_c, off, Hkv)
    torch.cuda.synchronize()
    kc_r, vc_r, pos_r, off_r = orc.compact(lay.k, lay.v, idx, cnt)
    assert np.array_equal(off.cpu().numpy(), off_r)
    assert np.array_equal(pos.cpu().numpy(), pos_r)
    assert np.array_equal(bits(k_c), kc_r.view(bits(k_c).dtype))
    assert np.array_equal(bits(v_c), vc_r.view(bits(v_c).dtype))
    out_r, lse_r = orc.decode(lay.q_dec[0], k_c.cpu(), v_c.cpu(), off_r, Hkv)
    e = check_decode(out.cpu().numpy(), lse.cpu().numpy(), out_r, lse_r)
    log(f"  decode err out {e[0]:.2e} lse {e[1]:.2e}")


def test_compact_truncates_at_capacity():
    lay = wl.random_case(2, B=2, Hq=4, Hkv=2, d=128, N_max=600, W=1)
    idx, cnt = oracle_selection(3, 2, 2, 600, [600, 600], 0.25)
    total = int(cnt.sum())
    cap = total - 77
    k_c, v_c, pos, off = api.kv_compact(dev(lay.k), dev(lay.v), dev(torch.from_numpy(idx)),
                                        dev(torch.from_numpy(cnt)), cap)
    out, lse = api.kv_decode_attn(dev(lay.q_dec[0]), k_c, v_c, off, 2)
    torch.cuda.synchronize()
    kc_r, vc_r, pos_r, off_r = orc.compact(lay.k, lay.v, idx, cnt)
    assert int(off[-1]) == total                       # the true total, not the capacity
    assert np.array_equal(pos.cpu().numpy(), pos_r[:cap])
    assert np.array_equal(bits(k_c), kc_r[:cap])
    # decode reads only rows below the capacity: the last head is clipped
    off_clip = np.minimum(off_r, cap)
    out_r, lse_r = orc.decode(lay.q_dec[0], k_c.cpu(), v_c.cpu(), off_clip, 2)
    check_decode(out.cpu().numpy(), lse.cpu().numpy(), out_r, lse_r)


def test_decode_special_cases():
    # one head with a single row, one head whose rows all fall past the
    # capacity (empty: out = 0, lse = -inf), zero queries (mean of V rows)
    lay = wl.random_case(4, B=1, Hq=6, Hkv=3, d=64, N_max=50, W=1)
    idx = np.full((1, 3, 50), -1, np.int32)
    idx[0, 0, :1] = [7]
    idx[0, 1, :20] = np.arange(0, 40, 2)
    idx[0, 2, :5] = np.arange(5)
    cnt = np.array([1, 20, 5], np.int32)
    k_c, v_c, pos, off = api.kv_compact(dev(lay.k), dev(lay.v), dev(torch.from_numpy(idx)),
                                        dev(torch.from_numpy(cnt)), 21)
    q = torch.zeros(1, 6, 64, dtype=lay.q_dec.dtype)
    q[0, :2] = lay.q_dec[0, 0, :2]
    out, lse = api.kv_decode_attn(dev(q), k_c, v_c, off, 3)
    torch.cuda.synchronize()
    v = lay.v.float()
    o = out.cpu()
    assert torch.equal(o[0, 0], v[0, 0, 7]) and torch.equal(o[0, 1], v[0, 0, 7])
    np.testing.assert_allclose(o[0, 2].numpy(), v[0, 1, 0:40:2].mean(0).numpy(), atol=1e-5)
    np.testing.assert_allclose(lse[0, 2].item(), np.log(20), atol=1e-5)
    assert torch.all(o[0, 4:] == 0) and torch.all(torch.isneginf(lse[0, 4:]))


def test_full_keep_decode_equals_full_cache_decode_bitwise():
    # 100% keep: compaction is the identity layout, so decode over the
    # compacted cache is the very same computation as over the full cache.
    lay = wl.random_case(6, B=2, Hq=8, Hkv=2, d=128, N_max=900, W=16, ctx=[900, 650])
    k, v, c = dev(lay.k), dev(lay.v), dev(lay.ctx_len)
    s, _ = api.kv_score(dev(lay.q_win), k, c)
    idx, cnt = api.kv_select(s, c, api.Budget(api.BUDGET_RATIO, ratio_scalar=1.0))
    k_c, v_c, pos, off = api.kv_compact(k, v, idx, cnt, 2 * 2 * 900)
    q = dev(lay.q_dec[0])
    out, lse = api.kv_decode_attn(q, k_c, v_c, off, 2)
    # the full cache packed directly (no selection involved)
    rows_k = torch.cat([lay.k[b, h, :n] for b, n in enumerate([900, 650]) for h in range(2)])
    rows_v = torch.cat([lay.v[b, h, :n] for b, n in enumerate([900, 650]) for h in range(2)])
    off_f = torch.tensor([0, 900, 1800, 2450, 3100], dtype=torch.int64)
    pad = 3600 - rows_k.shape[0]
    rows_k = torch.cat([rows_k, torch.zeros(pad, 128, dtype=rows_k.dtype)])
    rows_v = torch.cat([rows_v, torch.zeros(pad, 128, dtype=rows_v.dtype)])
    out_f, lse_f = api.kv_decode_attn(q, dev(rows_k), dev(rows_v), dev(off_f), 2)
    torch.cuda.synchronize()
    assert torch.equal(off.cpu(), off_f)
    assert torch.equal(out, out_f) and torch.equal(lse, lse_f)
    out_r, lse_r = orc.attend_full(lay.q_dec[0], lay.k, lay.v, [900, 650])
    check_decode(out.cpu().numpy(), lse.cpu().numpy(), out_r, lse_r)
