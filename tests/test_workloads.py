"""Seeded workload generators: reproducibility and the planted-needle check."""
import numpy as np
import torch

from kv_cache_compression_score_amd import workloads as wl
from oracle import oracle as orc


def test_generation_is_reproducible():
    cfg = wl.CONFIGS["ragged_adaptive"]
    a = wl.make_layer(cfg, B=2, N_max=4096)
    b = wl.make_layer(cfg, B=2, N_max=4096)
    for x, y in [(a.k, b.k), (a.v, b.v), (a.q_win, b.q_win), (a.q_dec, b.q_dec),
                 (a.ctx_len, b.ctx_len)]:
        assert torch.equal(x, y)
    assert a.k.dtype == torch.bfloat16
    for bb in range(2):
        n = int(a.ctx_len[bb])
        assert 2048 <= n <= 4096
        assert torch.count_nonzero(a.k[bb, :, n:]) == 0


def test_layers_have_independent_streams():
    cfg = wl.CONFIGS["long128k"]
    a = wl.make_layer(cfg, 0, N_max=256, with_v=False)
    b = wl.make_layer(cfg, 31, N_max=256, with_v=False)
    assert not torch.equal(a.k, b.k)
    assert torch.equal(b.k, wl.make_layer(cfg, 31, N_max=256, with_v=False).k)


def test_tiny_is_fp32_gaussian():
    cfg = wl.CONFIGS["tiny"]
    t = wl.make_layer(cfg)
    assert t.k.dtype == torch.float32 and t.k.shape == (1, 4, 1024, 64)
    assert abs(float(t.k.std()) - 1.0) < 0.02


def test_needles_are_retained_by_the_oracle():
    # The planted keys (3x the mean key norm along the window's mean query
    # direction) must survive a 10% budget; one sequence at full 32K length.
    cfg = wl.CONFIGS["needle32k"]
    lay = wl.make_layer(cfg, B=1)
    s, _ = orc.window_scores(lay.q_win, lay.k, lay.ctx_len)
    kept, cnt = orc.select(s, lay.ctx_len, orc.BUDGET_RATIO, ratio=cfg.ratio)
    assert np.all(cnt == 3277)
    for h in range(cfg.Hkv):
        keep = set(kept[0, h, :cnt[h]].tolist())
        missing = [p for p in lay.needle_pos[0, h].tolist() if p not in keep]
        assert not missing, f"head {h} lost needles {missing}"


def test_device_drawn_layer_follows_the_same_recipe():
    # make_layer_device (run here on the CPU generator): reproducible, the same
    # context lengths as the host-drawn layer, zero padding rows, needles at
    # the recorded positions, independent layers.
    import dataclasses
    cfg = dataclasses.replace(wl.CONFIGS["ragged_adaptive"], B=3, N_max=4096)
    a = wl.make_layer_device(cfg, 0, "cpu")
    b = wl.make_layer_device(cfg, 0, "cpu")
    assert torch.equal(a.k, b.k) and torch.equal(a.q_dec, b.q_dec)
    assert torch.equal(a.ctx_len, wl.make_layer(cfg, B=3, N_max=4096, with_v=False).ctx_len)
    for bb in range(3):
        n = int(a.ctx_len[bb])
        assert torch.count_nonzero(a.k[bb, :, n:]) == 0 and torch.count_nonzero(a.v[bb, :, n:]) == 0
    ncfg = dataclasses.replace(wl.CONFIGS["needle32k"], B=1, N_max=2048)
    lay = wl.make_layer_device(ncfg, 0, "cpu")
    for h in range(ncfg.Hkv):
        rows = lay.k[0, h, torch.from_numpy(lay.needle_pos[0, h])]
        assert torch.equal(rows, rows[:1].expand_as(rows))      # one planted key per head
    lcfg = dataclasses.replace(wl.CONFIGS["long128k"], N_max=256)
    assert not torch.equal(wl.make_layer_device(lcfg, 0, "cpu").k,
                           wl.make_layer_device(lcfg, 1, "cpu").k)
