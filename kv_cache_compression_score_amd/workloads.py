"""Seeded synthetic workloads for the score -> select -> compact -> decode path.

This module only draws random inputs and lays them out; it holds none of the
method's arithmetic (no logits, softmax, budgets, selection or attention), so
both the HIP path and the float64 oracle may take their inputs from it.

The five workloads stand in for the long-context suites the pages evaluate on
(RULER, LongBench, Needle-in-a-Haystack); no item of any suite is used.

Draw order inside one (config, layer) stream, from one
``numpy.random.Generator(PCG64)``:
  context lengths -> per-channel key scales -> K -> V -> window queries
  -> needle positions / Zipf permutations -> decode queries.
Multi-layer workloads give each layer its own child stream
(``SeedSequence(seed).spawn(L)``) so any single layer can be regenerated
without drawing the ones before it.

Floating-point values are drawn in fp32 and rounded to bf16 with
round-to-nearest-even (``torch.Tensor.to(torch.bfloat16)``); consumers read
those rounded values.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

# Budget modes, mirrored by name in the C header.
BUDGET_K = 0
BUDGET_RATIO = 1
BUDGET_THRESHOLD = 2
BUDGET_MASS = 3


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    L: int
    Hq: int
    Hkv: int
    d: int
    N_max: int
    W: int
    dtype: torch.dtype
    budget_mode: int
    ratio: float = 0.0          # kept fraction (ratio mode) / mass fraction (mass mode)
    min_ratio: float = 0.0
    max_ratio: float = 1.0
    ctx_range: Optional[tuple] = None   # inclusive (lo, hi) for ragged batches
    channel_lognormal: bool = False
    needles: int = 0
    zipf: float = 0.0
    decode_steps: int = 0
    seed: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


CONFIGS = {
    # fp32, no GQA; the small case every path can afford in full.
    "tiny": Config("tiny", B=1, L=1, Hq=4, Hkv=4, d=64, N_max=1024, W=32,
                   dtype=torch.float32, budget_mode=BUDGET_RATIO, ratio=0.25,
                   decode_steps=1),
    # One Llama-3-8B-shaped layer with outlier key channels.
    "llama8b_layer": Config("llama8b_layer", B=1, L=1, Hq=32, Hkv=8, d=128, N_max=8192,
                            W=64, dtype=torch.bfloat16, budget_mode=BUDGET_RATIO,
                            ratio=0.20, channel_lognormal=True, decode_steps=1),
    # Batch 4 at 32K with 64 planted needle keys per head.
    "needle32k": Config("needle32k", B=4, L=1, Hq=32, Hkv=8, d=128, N_max=32768, W=64,
                        dtype=torch.bfloat16, budget_mode=BUDGET_RATIO, ratio=0.10,
                        channel_lognormal=True, needles=64, decode_steps=1),
    # 32 layers at 128K, 128 decode steps per layer.
    "long128k": Config("long128k", B=1, L=32, Hq=32, Hkv=8, d=128, N_max=131072, W=128,
                       dtype=torch.bfloat16, budget_mode=BUDGET_RATIO, ratio=0.10,
                       channel_lognormal=True, decode_steps=128),
    # Ragged batch of 16 with Zipf(1.1) key norms and a score-mass budget.
    "ragged_adaptive": Config("ragged_adaptive", B=16, L=1, Hq=32, Hkv=8, d=128,
                              N_max=32768, W=64, dtype=torch.bfloat16,
                              budget_mode=BUDGET_MASS, ratio=0.95, min_ratio=0.02,
                              max_ratio=0.50, ctx_range=(2048, 32768), zipf=1.1,
                              decode_steps=1),
}


@dataclasses.dataclass
class Layer:
    """One layer's inputs, as CPU tensors in the config's dtype."""
    cfg: Config
    layer: int
    ctx_len: torch.Tensor      # [B] int32
    q_win: torch.Tensor        # [B][Hq][W][d]
    k: torch.Tensor            # [B][Hkv][N_max][d], rows >= ctx_len[b] are zero
    v: torch.Tensor            # [B][Hkv][N_max][d]
    q_dec: torch.Tensor        # [steps][B][Hq][d]
    needle_pos: Optional[np.ndarray] = None   # [B][Hkv][needles] int64


def _round(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)


def layer_rng(cfg: Config, layer: int) -> np.random.Generator:
    if cfg.L == 1:
        return np.random.Generator(np.random.PCG64(cfg.seed))
    child = np.random.SeedSequence(cfg.seed).spawn(cfg.L)[layer]
    return np.random.Generator(np.random.PCG64(child))


def make_layer(cfg: Config, layer: int = 0, *, B: Optional[int] = None,
               N_max: Optional[int] = None, with_v: bool = True) -> Layer:
    """Generate one layer of ``cfg``.

    ``B``/``N_max`` shrink the batch or context for quick cases (the draw
    order is unchanged, so a shrunk case is a different, equally seeded
    input).  ``with_v=False`` skips V (zeros) for score-only uses.
    """
    B = cfg.B if B is None else B
    N_max = cfg.N_max if N_max is None else N_max
    rng = layer_rng(cfg, layer)
    Hq, Hkv, d, W = cfg.Hq, cfg.Hkv, cfg.d, cfg.W

    if cfg.ctx_range is not None:
        lo, hi = cfg.ctx_range
        hi = min(hi, N_max)
        lo = min(lo, hi)
        ctx = rng.integers(lo, hi + 1, size=B, dtype=np.int64)
    else:
        ctx = np.full(B, N_max, dtype=np.int64)

    if cfg.channel_lognormal:
        ch_scale = np.exp(rng.standard_normal((Hkv, d))).astype(np.float32)
    else:
        ch_scale = None

    k = rng.standard_normal((B, Hkv, N_max, d), dtype=np.float32)
    if ch_scale is not None:
        k *= ch_scale[None, :, None, :]
    if with_v:
        v = rng.standard_normal((B, Hkv, N_max, d), dtype=np.float32)
    else:
        v = np.zeros((B, Hkv, N_max, d), dtype=np.float32)
    q_win = rng.standard_normal((B, Hq, W, d), dtype=np.float32)

    # Zero the padding rows of ragged sequences.
    for b in range(B):
        k[b, :, ctx[b]:, :] = 0.0
        v[b, :, ctx[b]:, :] = 0.0

    if cfg.zipf > 0.0:
        for b in range(B):
            n = int(ctx[b])
            ranks = np.arange(1, n + 1, dtype=np.float64)
            f = ranks ** (-cfg.zipf)
            f /= np.sqrt(np.mean(f * f))
            for h in range(Hkv):
                perm = rng.permutation(n)       # token t gets rank perm[t] + 1
                k[b, h, :n, :] *= f[perm].astype(np.float32)[:, None]

    q_win_t = _round(q_win, cfg.dtype)
    k_t = _round(k, cfg.dtype)

    needle_pos = None
    if cfg.needles > 0:
        G = cfg.G
        qf = q_win_t.to(torch.float64).numpy()
        needle_pos = np.zeros((B, Hkv, cfg.needles), dtype=np.int64)
        kf = k_t.to(torch.float32)
        for b in range(B):
            n = int(ctx[b])
            for h in range(Hkv):
                rows = qf[b, h * G:(h + 1) * G].reshape(G * W, d)
                u = rows.mean(axis=0)
                u /= np.linalg.norm(u)
                mean_norm = float(torch.linalg.vector_norm(
                    kf[b, h, :n].to(torch.float64), dim=1).mean())
                pos = rng.choice(n, size=cfg.needles, replace=False)
                needle_pos[b, h] = np.sort(pos)
                key = torch.from_numpy((3.0 * mean_norm * u).astype(np.float32)).to(cfg.dtype)
                k_t[b, h, torch.from_numpy(pos), :] = key

    steps = max(cfg.decode_steps, 1)
    q_dec = rng.standard_normal((steps, B, Hq, d), dtype=np.float32)

    return Layer(cfg=cfg, layer=layer,
                 ctx_len=torch.from_numpy(ctx.astype(np.int32)),
                 q_win=q_win_t, k=k_t, v=_round(v, cfg.dtype),
                 q_dec=_round(q_dec, cfg.dtype), needle_pos=needle_pos)


def random_case(seed: int, *, B: int, Hq: int, Hkv: int, d: int, N_max: int, W: int,
                dtype: torch.dtype = torch.bfloat16, ctx: Optional[list] = None,
                key_scale: float = 1.0, steps: int = 1) -> Layer:
    """A small seeded i.i.d. N(0,1) case of arbitrary shape (parity tests)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx_arr = np.full(B, N_max, dtype=np.int64) if ctx is None else np.asarray(ctx, np.int64)
    k = rng.standard_normal((B, Hkv, N_max, d), dtype=np.float32) * np.float32(key_scale)
    v = rng.standard_normal((B, Hkv, N_max, d), dtype=np.float32)
    q = rng.standard_normal((B, Hq, W, d), dtype=np.float32)
    for b in range(B):
        k[b, :, ctx_arr[b]:, :] = 0.0
        v[b, :, ctx_arr[b]:, :] = 0.0
    q_dec = rng.standard_normal((steps, B, Hq, d), dtype=np.float32)
    cfg = Config("random", B=B, L=1, Hq=Hq, Hkv=Hkv, d=d, N_max=N_max, W=W, dtype=dtype,
                 budget_mode=BUDGET_RATIO, ratio=0.25, decode_steps=steps, seed=seed)
    return Layer(cfg=cfg, layer=0, ctx_len=torch.from_numpy(ctx_arr.astype(np.int32)),
                 q_win=_round(q, dtype), k=_round(k, dtype), v=_round(v, dtype),
                 q_dec=_round(q_dec, dtype))


def make_layer_device(cfg: Config, layer: int = 0, device="cuda") -> Layer:
    """``make_layer``'s recipe drawn on the device, for sizes where drawing on
    the host takes minutes (the 32 layers of long128k, the ragged batch).

    The same distributions, scales, padding, Zipf profile, needles and draw
    order as ``make_layer``; the context lengths are the first draws of the
    same PCG64 stream (so a ragged batch has the same lengths), everything
    else comes from torch's device generator seeded from (seed, layer), so
    the values differ from the host-drawn layer.  Returns device tensors."""
    B, N_max = cfg.B, cfg.N_max
    Hq, Hkv, d, W = cfg.Hq, cfg.Hkv, cfg.d, cfg.W
    rng = layer_rng(cfg, layer)
    if cfg.ctx_range is not None:
        lo, hi = cfg.ctx_range
        hi = min(hi, N_max)
        lo = min(lo, hi)
        ctx = rng.integers(lo, hi + 1, size=B, dtype=np.int64)
    else:
        ctx = np.full(B, N_max, dtype=np.int64)
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([cfg.seed, layer, 1]).generate_state(1)[0]))
    f32 = dict(device=device, dtype=torch.float32, generator=g)
    ch_scale = torch.exp(torch.randn(Hkv, d, **f32)) if cfg.channel_lognormal else None
    k = torch.randn(B, Hkv, N_max, d, **f32)
    if ch_scale is not None:
        k *= ch_scale[None, :, None, :]
    v = torch.randn(B, Hkv, N_max, d, **f32)
    q_win = torch.randn(B, Hq, W, d, **f32)
    for b in range(B):
        k[b, :, ctx[b]:, :] = 0.0
        v[b, :, ctx[b]:, :] = 0.0
    if cfg.zipf > 0.0:
        for b in range(B):
            n = int(ctx[b])
            f = torch.arange(1, n + 1, device=device, dtype=torch.float64) ** (-cfg.zipf)
            f = (f / torch.sqrt(torch.mean(f * f))).to(torch.float32)
            for h in range(Hkv):
                perm = torch.randperm(n, device=device, generator=g)
                k[b, h, :n, :] *= f[perm][:, None]
    k_t = k.to(cfg.dtype)
    del k
    q_t = q_win.to(cfg.dtype)
    needle_pos = None
    if cfg.needles > 0:
        G = cfg.G
        needle_pos = np.zeros((B, Hkv, cfg.needles), dtype=np.int64)
        for b in range(B):
            n = int(ctx[b])
            for h in range(Hkv):
                u = q_t[b, h * G:(h + 1) * G].reshape(G * W, d).double().mean(dim=0)
                u = u / torch.linalg.vector_norm(u)
                mean_norm = torch.linalg.vector_norm(k_t[b, h, :n].double(), dim=1).mean()
                pos = torch.randperm(n, device=device, generator=g)[:cfg.needles]
                pos = torch.sort(pos).values
                needle_pos[b, h] = pos.cpu().numpy()
                k_t[b, h, pos, :] = (3.0 * mean_norm * u).to(torch.float32).to(cfg.dtype)
    steps = max(cfg.decode_steps, 1)
    q_dec = torch.randn(steps, B, Hq, d, **f32).to(cfg.dtype)
    return Layer(cfg=cfg, layer=layer,
                 ctx_len=torch.from_numpy(ctx.astype(np.int32)).to(device),
                 q_win=q_t, k=k_t, v=v.to(cfg.dtype), q_dec=q_dec, needle_pos=needle_pos)
