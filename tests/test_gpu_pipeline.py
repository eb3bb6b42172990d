"""score -> select -> compact -> decode end to end on the five workloads.

Full sizes throughout; where the float64 oracle would take too long (every
head of a 32K/128K batch) it checks sampled heads element by element, and
properties that hold at any size are checked on every head.
"""
import numpy as np
import pytest
import torch

from kv_cache_compression_score_amd import api
from kv_cache_compression_score_amd import workloads as wl
from oracle import oracle as orc

from gpu_helpers import (FLOOR, MASS_BAND, bits, check_band, check_decode, check_scores,
                         dev, log, mass_count_ok)

pytestmark = pytest.mark.gpu


def budget_of(cfg):
    if cfg.budget_mode == wl.BUDGET_MASS:
        return api.Budget(api.BUDGET_MASS, mass=cfg.ratio, min_ratio=cfg.min_ratio,
                          max_ratio=cfg.max_ratio)
    return api.Budget(api.BUDGET_RATIO, ratio_scalar=cfg.ratio)


def run(lay, cfg):
    q, k, v, c = dev(lay.q_win), dev(lay.k), dev(lay.v), dev(lay.ctx_len)
    B, Hkv, N = lay.k.shape[:3]
    s, row_lse = api.kv_score(q, k, c, with_row_lse=True)
    idx, cnt = api.kv_select(s, c, budget_of(cfg))
    cap = int(np.ceil(B * Hkv * N * cfg.max_ratio)) if cfg.budget_mode == wl.BUDGET_MASS \
        else B * Hkv * orc.budget_count(np.zeros(N), orc.BUDGET_RATIO, ratio=cfg.ratio)
    k_c, v_c, pos, off = api.kv_compact(k, v, idx, cnt, cap)
    qd = dev(lay.q_dec[0])
    out, lse = api.kv_decode_attn(qd, k_c, v_c, off, Hkv)
    # the fused call the benchmark times: the same packed cache and attention,
    # bit for bit
    fk, fv, fpos, foff, fout, flse = api.kv_compact_decode(k, v, idx, cnt, cap, qd)
    torch.cuda.synchronize()
    assert int(off[-1]) <= cap
    n = int(off[-1])
    assert torch.equal(foff, off) and torch.equal(fpos[:n], pos[:n])
    assert torch.equal(fk[:n].view(torch.int16), k_c[:n].view(torch.int16))
    assert torch.equal(fv[:n].view(torch.int16), v_c[:n].view(torch.int16))
    assert torch.equal(fout, out) and torch.equal(flse, lse)
    return dict(s=s.cpu().numpy(), row_lse=row_lse.cpu().numpy(), idx=idx.cpu().numpy(),
                cnt=cnt.cpu().numpy(), k_c=k_c.cpu(), v_c=v_c.cpu(), pos=pos.cpu().numpy(),
                off=off.cpu().numpy(), out=out.cpu().numpy(), lse=lse.cpu().numpy())


def check_compaction(lay, r):
    B, Hkv = lay.k.shape[:2]
    kb, vb = bits(lay.k), bits(lay.v)
    kcb, vcb = bits(r["k_c"]), bits(r["v_c"])
    off = r["off"]
    assert np.array_equal(np.diff(off), r["cnt"])
    for b in range(B):
        for h in range(Hkv):
            i = b * Hkv + h
            lo, hi = off[i], off[i + 1]
            p = r["pos"][lo:hi]
            assert np.array_equal(p, r["idx"][b, h, :hi - lo])
            assert np.all(np.diff(p) > 0)
            assert np.array_equal(kcb[lo:hi], kb[b, h, p])
            assert np.array_equal(vcb[lo:hi], vb[b, h, p])


def check_decode_vs_oracle(lay, r, Hkv):
    out_r, lse_r = orc.decode(lay.q_dec[0], r["k_c"], r["v_c"], r["off"], Hkv)
    return check_decode(r["out"], r["lse"], out_r, lse_r)


@pytest.mark.parametrize("name", ["tiny", "llama8b_layer"])
def test_small_configs_full_oracle(name):
    cfg = wl.CONFIGS[name]
    lay = wl.make_layer(cfg)
    log(f"pipeline {name}")
    r = run(lay, cfg)
    ctx = lay.ctx_len.numpy()
    s_ref, lse_ref = orc.window_scores(lay.q_win, lay.k, lay.ctx_len)
    err = check_scores(r["s"], s_ref, ctx, cfg.W, cfg.G)
    np.testing.assert_allclose(r["row_lse"], lse_ref, atol=1e-3, rtol=0)
    _, k_ref = orc.select(s_ref, ctx, orc.BUDGET_RATIO, ratio=cfg.ratio)
    nd = check_band(r["idx"], r["cnt"], s_ref, ctx, cfg.W, cfg.G, k_ref=k_ref)
    check_compaction(lay, r)
    e = check_decode_vs_oracle(lay, r, cfg.Hkv)
    log(f"  score err {err:.2e}, in-band set differences {nd}, decode err {e}")


def test_needle32k():
    cfg = wl.CONFIGS["needle32k"]
    lay = wl.make_layer(cfg)
    log("pipeline needle32k")
    r = run(lay, cfg)
    ctx = lay.ctx_len.numpy()
    assert np.all(r["cnt"] == 3277)
    # every planted needle survives, on every head of every sequence
    for b in range(cfg.B):
        for h in range(cfg.Hkv):
            kept = set(r["idx"][b, h, :3277].tolist())
            lost = [p for p in lay.needle_pos[b, h].tolist() if p not in kept]
            assert not lost, (b, h, lost)
    tot = r["s"].astype(np.float64).sum(axis=2)
    np.testing.assert_allclose(tot, cfg.W * cfg.G, rtol=1e-4)
    # oracle element by element on sequence 0 (all 8 heads)
    s_ref, lse_ref = orc.window_scores(lay.q_win[:1], lay.k[:1], lay.ctx_len[:1])
    err = check_scores(r["s"][:1], s_ref, ctx[:1], cfg.W, cfg.G)
    np.testing.assert_allclose(r["row_lse"][:1], lse_ref, atol=1e-3, rtol=0)
    nd = check_band(r["idx"][:1], r["cnt"][:cfg.Hkv], s_ref, ctx[:1], cfg.W, cfg.G)
    check_compaction(lay, r)
    e = check_decode_vs_oracle(lay, r, cfg.Hkv)
    log(f"  score err {err:.2e}, in-band set differences {nd}, decode err {e}")


def test_ragged_adaptive_mass_budget():
    cfg = wl.CONFIGS["ragged_adaptive"]
    lay = wl.make_layer(cfg)
    log(f"pipeline ragged_adaptive ctx={lay.ctx_len.tolist()}")
    r = run(lay, cfg)
    ctx = lay.ctx_len.numpy()
    f, lo, hi = cfg.ratio, cfg.min_ratio, cfg.max_ratio
    for b in range(cfg.B):
        n = int(ctx[b])
        k_lo = max(1, int(np.floor(np.float32(lo) * n + 0.5)))
        k_hi = int(np.floor(np.float32(hi) * n + 0.5))
        k = r["cnt"][b * cfg.Hkv:(b + 1) * cfg.Hkv]
        assert np.all((k >= k_lo) & (k <= k_hi)), (b, k, k_lo, k_hi)
    # Stage parity on the GPU's own scores: the count brackets the mass target
    # within the fixed-point band on exact sums, and the kept set is exactly
    # the first k tokens of the order.
    _, k_stage = orc.select(r["s"], ctx, orc.BUDGET_MASS, mass=f, min_ratio=lo, max_ratio=hi)
    dk = 0
    for b in range(cfg.B):
        n = int(ctx[b])
        for h in range(cfg.Hkv):
            i = b * cfg.Hkv + h
            kg = int(r["cnt"][i])
            sh = r["s"][b, h, :n].astype(np.float64)
            if kg != int(k_stage[i]):
                assert mass_count_ok(sh, kg, f, lo, hi), (b, h, kg, int(k_stage[i]))
                dk = max(dk, abs(kg - int(k_stage[i])))
            ref = np.sort(orc.total_order(sh)[:kg])
            assert np.array_equal(r["idx"][b, h, :kg], ref), (b, h)
    # End to end on every sequence against the oracle's own scores: scores
    # within tolerance, kept sets equal outside the 1e-5 band of the k-th
    # score, and each count brackets the oracle-score target within the band
    # that the measured score error allows: with every score within rho
    # relative, C(k) moves by at most rho C(n) on each side (2 rho + rho^2),
    # plus the scores under the floor.
    nd, worst = 0, 0.0
    for b in range(cfg.B):
        n = int(ctx[b])
        s_ref, _ = orc.window_scores(lay.q_win[b:b + 1], lay.k[b:b + 1], lay.ctx_len[b:b + 1])
        err = check_scores(r["s"][b:b + 1], s_ref, ctx[b:b + 1], cfg.W, cfg.G)
        worst = max(worst, err)
        nd += check_band(r["idx"][b:b + 1], r["cnt"][b * cfg.Hkv:(b + 1) * cfg.Hkv], s_ref,
                         ctx[b:b + 1], cfg.W, cfg.G)
        for h in range(cfg.Hkv):
            sh = s_ref[0, h, :n]
            band = 2 * err + err * err + n * FLOOR * cfg.W * cfg.G / sh.sum() + MASS_BAND
            kg = int(r["cnt"][b * cfg.Hkv + h])
            assert mass_count_ok(sh, kg, f, lo, hi, band=band), (b, h, kg, band)
    check_compaction(lay, r)
    e = check_decode_vs_oracle(lay, r, cfg.Hkv)
    log(f"  k range {r['cnt'].min()}..{r['cnt'].max()}, stage max |dk| {dk}, score err "
        f"{worst:.2e}, in-band set differences {nd}, decode err {e}")


def test_long128k_layer():
    cfg = wl.CONFIGS["long128k"]
    lay = wl.make_layer(cfg, 31)
    log("pipeline long128k layer 31")
    r = run(lay, cfg)
    ctx = lay.ctx_len.numpy()
    assert np.all(r["cnt"] == 13107)
    h = 2
    s_ref, _ = orc.window_scores(lay.q_win[:, h * 4:(h + 1) * 4], lay.k[:, h:h + 1], lay.ctx_len)
    err = check_scores(r["s"][:, h:h + 1], s_ref, ctx, cfg.W, cfg.G)
    nd = check_band(r["idx"][:, h:h + 1], r["cnt"][h:h + 1], s_ref, ctx, cfg.W, cfg.G)
    check_compaction(lay, r)
    e = check_decode_vs_oracle(lay, r, cfg.Hkv)
    log(f"  head {h} score err {err:.2e}, in-band diffs {nd}, decode err {e}")


def test_long128k_layers_looped_decode_steps_layer_inner():
    # The 128K workload as configured, on two of its 32 layers: each layer is
    # scored, selected and compacted by the fused call the benchmark times,
    # its compacted cache kept, then decode steps run layer-inner (step s:
    # layer 0, then layer 31) over the kept caches, each checked against the
    # oracle's decode over the same packed rows.
    cfg = wl.CONFIGS["long128k"]
    steps = 4
    caches = []
    for layer in (0, 31):
        lay = wl.make_layer(cfg, layer)
        log(f"long128k layer {layer}: score, select, compact + first decode step")
        q, k, v = dev(lay.q_win), dev(lay.k), dev(lay.v)
        s, _ = api.kv_score(q, k, None)
        idx, cnt = api.kv_select(s, None, api.Budget(api.BUDGET_RATIO, ratio_scalar=cfg.ratio))
        cap = cfg.Hkv * 13107
        k_c, v_c, pos, off, out0, lse0 = api.kv_compact_decode(k, v, idx, cnt, cap,
                                                               dev(lay.q_dec[0]))
        torch.cuda.synchronize()
        assert np.all(cnt.cpu().numpy() == 13107) and int(off[-1]) == cap
        # scores, kept set and packed rows of one sampled head against the oracle
        h = 5 if layer == 0 else 1
        s_ref, _ = orc.window_scores(lay.q_win[:, h * cfg.G:(h + 1) * cfg.G], lay.k[:, h:h + 1],
                                     lay.ctx_len)
        err = check_scores(s.cpu().numpy()[:, h:h + 1], s_ref, lay.ctx_len.numpy(), cfg.W, cfg.G)
        idx_np = idx.cpu().numpy()
        nd = check_band(idx_np[:, h:h + 1], cnt.cpu().numpy()[h:h + 1], s_ref,
                        lay.ctx_len.numpy(), cfg.W, cfg.G)
        kc_np, vc_np, pos_np = bits(k_c), bits(v_c), pos.cpu().numpy()
        kb, vb = bits(lay.k), bits(lay.v)
        for hh in range(cfg.Hkv):
            o0, o1 = int(off[hh]), int(off[hh + 1])
            p = idx_np[0, hh, :13107]
            assert np.array_equal(pos_np[o0:o1], p) and np.all(np.diff(p) > 0)
            assert np.array_equal(kc_np[o0:o1], kb[0, hh, p])
            assert np.array_equal(vc_np[o0:o1], vb[0, hh, p])
        log(f"  head {h} score err {err:.2e}, in-band set differences {nd}")
        caches.append(dict(q_dec=lay.q_dec[:steps], k_c=k_c, v_c=v_c, off=off,
                           first=(out0.cpu().numpy(), lse0.cpu().numpy())))
        del lay, q, k, v, s, idx
    ws = torch.zeros(api.kv_decode_workspace_size(1, cfg.Hq, cfg.Hkv, cfg.d, cfg.Hkv * 13107),
                     device="cuda", dtype=torch.uint8)
    worst = (0.0, 0.0)
    for step in range(steps):
        for c in caches:
            out, lse = api.kv_decode_attn(dev(c["q_dec"][step]), c["k_c"], c["v_c"], c["off"],
                                          cfg.Hkv, workspace=ws)
            torch.cuda.synchronize()
            if step == 0:   # the fused call's own attention, bit for bit
                assert np.array_equal(out.cpu().numpy(), c["first"][0])
                assert np.array_equal(lse.cpu().numpy(), c["first"][1])
            out_r, lse_r = orc.decode(c["q_dec"][step], c["k_c"].cpu(), c["v_c"].cpu(),
                                      c["off"].cpu().numpy(), cfg.Hkv)
            e = check_decode(out.cpu().numpy(), lse.cpu().numpy(), out_r, lse_r)
            worst = (max(worst[0], e[0]), max(worst[1], e[1]))
    log(f"  {steps} decode steps x 2 layers, layer-inner: max err out {worst[0]:.2e}, "
        f"lse {worst[1]:.2e}")
