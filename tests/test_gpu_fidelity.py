"""Fidelity report (output and log-sum-exp loss terms) on the GPU vs the oracle."""
import numpy as np
import pytest
import torch

from kv_cache_compression_score_amd import api, fidelity
from kv_cache_compression_score_amd import workloads as wl
from oracle import oracle as orc

from gpu_helpers import dev, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,steps", [("llama8b_layer", 2), ("ragged_adaptive", 1),
                                        ("needle32k", 1)])
def test_fidelity_matches_oracle(name, steps):
    cfg = wl.CONFIGS[name]
    B = 2 if name == "ragged_adaptive" else None
    lay = wl.make_layer(cfg, B=B, N_max=8192 if name == "ragged_adaptive" else None)
    log(f"fidelity {name}")
    q, k, v, c = dev(lay.q_win), dev(lay.k), dev(lay.v), dev(lay.ctx_len)
    s, _ = api.kv_score(q, k, c)
    if cfg.budget_mode == wl.BUDGET_MASS:
        bud = api.Budget(api.BUDGET_MASS, mass=cfg.ratio, min_ratio=cfg.min_ratio,
                         max_ratio=cfg.max_ratio)
    else:
        bud = api.Budget(api.BUDGET_RATIO, ratio_scalar=cfg.ratio)
    idx, cnt = api.kv_select(s, c, bud)
    cap = int(cnt.sum().item())
    k_c, v_c, _, off = api.kv_compact(k, v, idx, cnt, cap)
    for st in range(min(steps, len(lay.q_dec))):
        qd = dev(lay.q_dec[st])
        out_c, lse_c = api.kv_decode_attn(qd, k_c, v_c, off, cfg.Hkv)
        out_f, lse_f = fidelity.full_cache_decode(qd, k, v, c)
        f_gpu = fidelity.fidelity(out_c, lse_c, out_f, lse_f)
        torch.cuda.synchronize()
        f_ref = orc.fidelity(lay.q_dec[st], lay.k, lay.v, idx.cpu().numpy(), cnt.cpu().numpy(),
                             lay.ctx_len)
        # each output within 1e-2 and each lse within 1e-3 of the oracle, so the
        # per-query differences agree within 2e-2 per element / 2e-3
        d_gpu = out_c.double().cpu().numpy() - out_f.double().cpu().numpy()
        B_, Hq, d = d_gpu.shape
        assert np.abs(np.sqrt(f_gpu["out_err2"]) - np.sqrt(f_ref["out_err2"])).max() \
            <= 2e-2 * np.sqrt(d)
        np.testing.assert_allclose(f_gpu["lse_diff"], f_ref["lse_diff"], atol=2e-3)
        assert (f_gpu["lse_diff"] <= 1e-3).all()
        log(f"  step {st}: {fidelity.summary(f_gpu)}")
