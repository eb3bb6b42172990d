"""Fidelity of a compacted cache: the two loss terms of "KVSculpt: KV Cache
Compression as Distillation", section 2.B, measured with the library's own
kernels.

For decode queries q, Y / ell are the attention output and log-sum-exp over
the full cache and Y^ / ell^ over the compacted one:
    out_err2 = ||Y^ - Y||^2 per query,   lse_diff = ell^ - ell per query,
    loss     = sum out_err2 + sum lse_diff^2.
The full-cache reference is built with kv_select at ratio 1 (every token, in
order) and kv_compact, then read by kv_decode_attn like any compacted cache;
only the final norms of the [B][Hq][d] outputs are taken on the host.
"""
from __future__ import annotations

import numpy as np
import torch

from . import api


def full_cache_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      ctx_len: torch.Tensor, *, scale: float = 0.0):
    """(out, lse) of decode over every cached row of every head."""
    B, Hkv, N_max, d = k.shape
    scores = torch.zeros(B, Hkv, N_max, device=k.device, dtype=torch.float32)
    idx, cnt = api.kv_select(scores, ctx_len, api.Budget(api.BUDGET_RATIO, ratio_scalar=1.0))
    cap = int(Hkv * ctx_len.to(torch.int64).sum().item())
    k_f, v_f, _, off = api.kv_compact(k, v, idx, cnt, cap)
    return api.kv_decode_attn(q, k_f, v_f, off, Hkv, scale=scale)


def fidelity(out_c: torch.Tensor, lse_c: torch.Tensor, out_full: torch.Tensor,
             lse_full: torch.Tensor) -> dict:
    """Loss terms from the decode outputs of the compacted and full caches."""
    yh, y = out_c.double().cpu().numpy(), out_full.double().cpu().numpy()
    lh, ell = lse_c.double().cpu().numpy(), lse_full.double().cpu().numpy()
    err2 = ((yh - y) ** 2).sum(axis=-1)
    norm2 = (y ** 2).sum(axis=-1)
    dl = lh - ell
    return {"out_err2": err2, "out_norm2": norm2, "lse_diff": dl,
            "loss": float(err2.sum() + (dl ** 2).sum())}


def summary(f: dict) -> dict:
    """Scalars for a report line."""
    rel = np.sqrt(f["out_err2"] / np.maximum(f["out_norm2"], 1e-300))
    return {"queries": int(f["out_err2"].size), "loss": f["loss"],
            "mean_rel_out_err": float(rel.mean()), "max_rel_out_err": float(rel.max()),
            "mean_lse_diff": float(f["lse_diff"].mean()),
            "min_lse_diff": float(f["lse_diff"].min()),
            "mean_kept_mass": float(np.exp(f["lse_diff"]).mean())}
