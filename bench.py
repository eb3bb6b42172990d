#!/usr/bin/env python3
"""Throughput of the score -> select -> compact -> decode path on one GPU.

One step = kv_score_select (kv_score and kv_select in one call) +
kv_compact_decode (kv_compact and kv_decode_attn in one pass over the kept
rows) over one batch of the chosen
synthetic workload (default: batch 4 at 32K context, 32 query / 8 KV heads,
d = 128, W = 64, keep 10%, one decode step), inputs resident in HBM before
timing starts.  Prints one JSON line:

  value       cached tokens per second over the whole step, from the median
              step time with cold caches: before every timed step, outside
              its events, a 1 GiB buffer is read so that the L2 caches and
              the 256 MB Infinity Cache hold nothing of the step's data
              (step_ms_warm: the same steps back to back; step_ms_warm_graph:
              the step captured once as a HIP graph and replayed back to back)
  roofline    the kernel with the most GPU time: algorithmic FLOPs (MFMA
              kernels) or bytes (HBM kernels) per launch / its mean duration,
              from hipEvents that the library's dispatches stamp on their own
              stream, over a second run of as many cold steps right after the
              timed ones (stamped dispatches lengthen a step by a few us, so
              the steps that give `value` carry none; that run's step times
              are step_ms_cold_kernel_events); `traffic` is the
              HBM bytes per launch that rocprofv3's FETCH_SIZE + WRITE_SIZE
              counters read for that kernel (scaled by the ratio of known to
              counted bytes of a plain device copy), taken from the committed
              summary under profiles/ and reported only while the kernel's
              sources still hash to the recorded value
  targets     the stage-level fractions: score (both passes) against the
              bf16 MFMA peak, select + compact + decode against HBM
  copy_gbps   a 1 GiB device-to-device copy (read + write bytes / time)
  launch_shapes  workgroups and threads per workgroup of each kernel's launch
  gpu         device name, ROCm and torch versions, and the clocks amd-smi
              reports while the step runs back to back
  unfused     the same step with kv_compact and kv_decode_attn as two calls;
              decode_hbm_gbps is that decode's rate; score_then_select:
              kv_score and kv_select as two calls
  fidelity    output / log-sum-exp loss terms of the compacted cache
              against the full cache for the step's decode queries (and,
              fidelity_window_query, for the last window row of each head)
  vector_routing  VECTOR three-way routing (route, routed compaction,
              decode rebuilding dropped values) at the same memory budget
  score_one_pass  kv_score_from_lse (row LSEs given, as a prefill pass
              yields them): one sweep over K instead of two
  workloads   the other workloads' steps (tiny, llama8b_layer,
              ragged_adaptive) and long128k as configured: 32 layers scored,
              selected and compacted, then 128 decode steps layer-inner over
              the 32 compacted caches
  cpu_baseline the float64 oracle on a bounded sample on the host cores,
              per stage, for every workload measured
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from kv_cache_compression_score_amd import _lib, api, fidelity  # noqa: E402
from kv_cache_compression_score_amd import workloads as wl  # noqa: E402

METRIC = "cached tokens/sec scored+selected+compacted at 32K ctx; decode-attn HBM GB/s"
PEAK_HBM_GBPS = 8000.0
PEAK_TFLOPS = {torch.bfloat16: 2500.0, torch.float32: 157.3}
DEV = torch.device("cuda:0")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="needle32k", choices=sorted(wl.CONFIGS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true",
                   help="only the headline workload (no other workloads, VECTOR, fidelity)")
    p.add_argument("--score-then-select", action="store_true",
                   help="time kv_score + kv_select as two calls instead of kv_score_select")
    p.add_argument("--cpu-seqs", type=int, default=4,
                   help="sequences of the batch the oracle baseline processes")
    return p.parse_args()


def budget_of(cfg: wl.Config):
    if cfg.budget_mode == wl.BUDGET_MASS:
        return api.Budget(api.BUDGET_MASS, mass=cfg.ratio, min_ratio=cfg.min_ratio,
                          max_ratio=cfg.max_ratio)
    return api.Budget(api.BUDGET_RATIO, ratio_scalar=cfg.ratio)


def capacity_of(cfg: wl.Config, B: int, Hkv: int, N: int) -> int:
    if cfg.budget_mode == wl.BUDGET_MASS:
        return int(math.ceil(B * Hkv * N * cfg.max_ratio))
    return B * Hkv * max(1, int(math.floor(float(np.float32(cfg.ratio)) * N + 0.5)))


class Pipeline:
    """One layer's buffers and the step that runs the whole path over them."""

    def __init__(self, lay: wl.Layer, fused: bool = True):
        cfg = lay.cfg
        self.cfg = cfg
        self.fused = fused
        self.q = lay.q_win.to(DEV)
        self.k = lay.k.to(DEV)
        self.v = lay.v.to(DEV)
        self.c = lay.ctx_len.to(DEV)
        self.qd = lay.q_dec[0].to(DEV)
        B, Hkv, N, D = lay.k.shape
        self.budget = budget_of(cfg)
        self.cap = capacity_of(cfg, B, Hkv, N)
        f32 = torch.float32
        self.scores = torch.empty(B, Hkv, N, device=DEV, dtype=f32)
        self.ws_s = torch.zeros(api.kv_score_select_workspace_size(B, cfg.Hq, Hkv, N, cfg.W, D),
                                device=DEV, dtype=torch.uint8)
        self.two_calls = False   # kv_score + kv_select instead of kv_score_select
        self.idx = torch.empty(B, Hkv, N, device=DEV, dtype=torch.int32)
        self.cnt = torch.empty(B * Hkv, device=DEV, dtype=torch.int32)
        self.comp = (torch.empty(self.cap, D, device=DEV, dtype=lay.k.dtype),
                     torch.empty(self.cap, D, device=DEV, dtype=lay.k.dtype),
                     torch.empty(self.cap, device=DEV, dtype=torch.int32),
                     torch.empty(B * Hkv + 1, device=DEV, dtype=torch.int64))
        self.out = torch.empty(B, cfg.Hq, D, device=DEV, dtype=f32)
        self.lse = torch.empty(B, cfg.Hq, device=DEV, dtype=f32)
        self.ws_d = torch.zeros(api.kv_decode_workspace_size(B, cfg.Hq, Hkv, D, self.cap),
                                device=DEV, dtype=torch.uint8)

    def step(self):
        if self.two_calls:
            api.kv_score(self.q, self.k, self.c, scores=self.scores, workspace=self.ws_s)
            api.kv_select(self.scores, self.c, self.budget, kept_idx=self.idx,
                          kept_count=self.cnt)
        else:
            api.kv_score_select(self.q, self.k, self.c, self.budget, scores=self.scores,
                                kept_idx=self.idx, kept_count=self.cnt, workspace=self.ws_s)
        if self.fused:
            api.kv_compact_decode(self.k, self.v, self.idx, self.cnt, self.cap, self.qd,
                                  out=self.comp, attn_out=self.out, lse=self.lse,
                                  workspace=self.ws_d)
            return
        k_c, v_c, _, off = api.kv_compact(self.k, self.v, self.idx, self.cnt, self.cap,
                                          out=self.comp)
        api.kv_decode_attn(self.qd, k_c, v_c, off, self.cfg.Hkv, out=self.out, lse=self.lse,
                           workspace=self.ws_d)


def settle_clocks(step, seconds: float = 0.1, flush=None) -> int:
    """Run the step untimed for about `seconds` of wall time.  From a cold
    start the GPU needs a few tens of ms of sustained load before its clocks
    settle (the first steps run up to 20% slower), so the warmup steps alone
    would leave the timed region on the ramp.  The clocks settle again when
    the load changes: with `flush`, each step is preceded by it, as in the
    cold timed steps (after back-to-back steps, the first 40 or so flushed
    steps run 3-6% slower).  Returns the steps run."""
    n = 0
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(10):
            if flush is not None:
                flush()
            step()
        n += 10
        torch.cuda.synchronize()
    return n


def _timing_start(only):
    L = _lib.lib()
    L.kv_timing_only(only.encode() if only else None)
    L.kv_timing_enable(1)


def _timing_stop() -> dict:
    L = _lib.lib()
    buf = (_lib.KvKernelTime * 64)()
    n = L.kv_timing_read(buf, 64)
    L.kv_timing_enable(0)
    L.kv_timing_only(None)
    if n < 0:
        raise RuntimeError(f"kv_timing_read failed: {n}")
    # name -> (mean ms, launches, (workgroups, threads per workgroup) of the last launch)
    return {buf[i].name.decode(): (buf[i].total_ms / buf[i].launches, buf[i].launches,
                                   (int(buf[i].grid), int(buf[i].block))) for i in range(n)}


def timed_steps(step, steps: int, only=None, events: bool = True):
    """Wall-clock ms per step (back to back) and the event timings of the same
    steps: every kernel, or (only=name) one kernel, so that only one launch
    per step is a timed dispatch (the events are stamped by the dispatch
    itself, which still slows a timed launch by a few us); events=False
    times no dispatch at all."""
    torch.cuda.synchronize()
    if events:
        _timing_start(only)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    return ms, (_timing_stop() if events else {})


def _spread(ms) -> dict:
    ms = np.sort(np.asarray(ms, dtype=np.float64))
    return {"median": float(np.median(ms)), "p10": float(np.percentile(ms, 10)),
            "p90": float(np.percentile(ms, 90)), "steps": int(ms.size)}


class Flush:
    """Reads a 1 GiB buffer, so that neither the L2 caches nor the 256 MB
    Infinity Cache hold anything of the next step's data (a read leaves no
    dirty lines whose write-back would land inside the next step)."""

    def __init__(self):
        self.buf = torch.ones(1 << 28, device=DEV, dtype=torch.float32)

    def __call__(self):
        self.buf.sum()


def step_distribution(step, steps: int, flush=None, only=None):
    """Per-step times (ms) from torch events around each step on the stream
    the library launches on; `flush`, if given, runs before every step,
    outside its events.  With `only`, that kernel's dispatches stamp their
    own events over the same steps.  Returns (spread, wall ms of the loop,
    kernel timings)."""
    st = torch.cuda.current_stream()
    ev = []
    torch.cuda.synchronize()
    if only is not None:
        _timing_start(only)
    t0 = time.perf_counter()
    for _ in range(steps):
        if flush is not None:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        step()
        e1.record(st)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    kt = _timing_stop() if only is not None else {}
    return _spread([a.elapsed_time(b) for a, b in ev]), wall, kt


def graph_steps(step, steps: int) -> dict:
    """The step captured once as a HIP graph (static buffers: the library
    allocates nothing and records no memset) and replayed back to back,
    each replay between events on the current stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    settle_clocks(g.replay)
    spread, _, _ = step_distribution(g.replay, steps)
    del g
    return spread


def gpu_clocks(step):
    """The GPU's clocks while `step` runs back to back (each tool a child
    process, 30 s at most): rocm-smi's sclk / mclk, and amd-smi's per-XCD
    figures as it reports them (on this part its `clk` field has read both
    values that agree with rocm-smi and values below its own 500 MHz minimum
    under load, so rocm-smi's sclk is the reading to use).  Skipped under a
    profiler."""
    import subprocess
    if any(k.startswith("ROCPROF") for k in os.environ):
        # under rocprofv3 every child process starts with the profiler's
        # library loaded, and the tools' interpreter launch is refused there
        return {"skipped": "run under a profiler"}

    def under_load(cmd):
        try:
            p = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
        except OSError as e:
            return None, str(e)
        t_end = time.perf_counter() + 30.0
        while p.poll() is None and time.perf_counter() < t_end:
            for _ in range(20):
                step()
            torch.cuda.synchronize()
        if p.poll() is None:
            p.kill()
        out, err = p.communicate()
        if p.returncode != 0:
            return None, f"{cmd[0]} exit {p.returncode}: {err.strip()[:200]}"
        try:
            return json.loads(out), None
        except ValueError:
            return None, f"{cmd[0]}: no JSON"

    res = {"sampled": "while the step ran back to back"}
    rep, err = under_load(["rocm-smi", "--showclocks", "--json"])
    if rep:
        card = next(iter(rep.values()))
        res["rocm_smi"] = {k.rstrip(":"): v for k, v in card.items() if "clock" in k}
    else:
        res["rocm_smi_error"] = err
    rep, err = under_load(["amd-smi", "metric", "--clock", "--json"])
    try:
        clk = rep["gpu_data"][0]["clock"]
        res["amd_smi_clk_mhz"] = {k: v["clk"]["value"] for k, v in clk.items()
                                  if isinstance(v, dict) and isinstance(v.get("clk"), dict)}
    except (TypeError, KeyError, IndexError):
        res["amd_smi_error"] = err
    return res


def one_pass_score_ms(pipe: Pipeline, steps: int) -> float:
    """Mean event time of kv_score_from_lse (the score stage when the row
    LSEs come from the prefill), fed the row LSEs of a two-pass call."""
    _, lse = api.kv_score(pipe.q, pipe.k, pipe.c, with_row_lse=True)
    out = torch.empty_like(pipe.scores)
    for _ in range(3):
        api.kv_score_from_lse(pipe.q, pipe.k, pipe.c, lse, scores=out)
    torch.cuda.synchronize()
    _timing_start("score_colsum")
    for _ in range(steps):
        api.kv_score_from_lse(pipe.q, pipe.k, pipe.c, lse, scores=out)
    torch.cuda.synchronize()
    return _timing_stop()["score_colsum"][0]


def vector_measure(pipe: Pipeline, steps: int) -> dict:
    """VECTOR routing at the same memory as the headline's 10% keep (p_c =
    0.9, p_a = 0.05: keys for 15% of the tokens, values for 5%), with a
    seeded random linear map W and rotary base 500000, timed per kernel over
    `steps` route + compact + decode passes."""
    cfg = pipe.cfg
    B, Hkv, N, D = pipe.k.shape
    g = torch.Generator().manual_seed(7)
    w = (torch.randn(Hkv, D, D, generator=g) / math.sqrt(D)).to(DEV)
    p_c, p_a, base = 0.9, 0.05, 500000.0

    def one():
        r = api.kv_vector_route(pipe.scores, pipe.c, pipe.k, pipe.v, w, p_c=p_c, p_a=p_a,
                                rope_base=base)
        pool_idx, pool_count, _, apx_pos, apx_count = r
        cap = B * Hkv * N // 4
        comp = api.kv_vector_compact(pipe.k, pipe.v, pool_idx, pool_count, apx_pos, apx_count,
                                     cap, cap)
        k_c, v_c, pos, vmap, off, voff = comp
        api.kv_vector_decode(pipe.qd, k_c, v_c, vmap, pos, off, w, Hkv, v_capacity_rows=cap,
                             rope_base=base)
        return pool_count, apx_count

    pool_count, apx_count = one()
    torch.cuda.synchronize()
    _timing_start(None)
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    kt = {k: v[0] for k, v in _timing_stop().items()}
    rows = int(pool_count.sum().item())
    vrows = rows - int(apx_count.sum().item())
    esz = pipe.k.element_size()
    t_route = sum(kt[k] for k in ("vector_counts", "vector_pool", "vector_residual", "vector_apx"))
    t_comp = kt["vector_vmap"] + kt["vector_copy"]
    t_dec = kt["vector_decode_split"] + kt["vector_decode_merge"]
    dec_bytes = rows * D * esz + vrows * D * esz + rows * 8 + B * cfg.Hq * D * (esz + 4)
    return {"p_c": p_c, "p_a": p_a, "key_rows": rows, "value_rows": vrows,
            "kernels_ms": kt, "route_ms": t_route, "compact_ms": t_comp, "decode_ms": t_dec,
            "residual_tflops": 2.0 * D * D * rows / (kt["vector_residual"] * 1e-3) / 1e12,
            "decode_gbps": dec_bytes / (t_dec * 1e-3) / 1e9}


COPY_BYTES = 1 << 30


def copy_gbps(reps: int = 5) -> float:
    """Read + write bandwidth of a plain 1 GiB device copy (torch copy_)."""
    src = torch.empty(COPY_BYTES // 4, device=DEV, dtype=torch.float32).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    sec = ev[0].elapsed_time(ev[1]) * 1e-3 / reps
    del src, dst
    return 2.0 * COPY_BYTES / sec / 1e9


# Sources each timed kernel is built from (the traffic figures are tied to them).
KERNEL_SOURCES = {
    "score_rowstats": ("score.hip", "common.hpp"), "score_colsum": ("score.hip", "common.hpp"),
    "score_fold": ("score.hip", "common.hpp"), "select": ("select.hip", "common.hpp"),
    "compact": ("compact.hip", "common.hpp"), "decode_split": ("decode.hip", "common.hpp"),
    "compact_decode": ("decode.hip", "common.hpp"),
    "decode_merge": ("decode.hip", "common.hpp"),
}
CSRC = os.path.join(ROOT, "kv_cache_compression_score_amd", "csrc")


def source_hash(kernel: str) -> str:
    """Hash of the kernel's sources and of the build script (its flags)."""
    h = hashlib.sha256()
    paths = [os.path.join(CSRC, f) for f in KERNEL_SOURCES[kernel]]
    paths.append(os.path.join(ROOT, "kv_cache_compression_score_amd", "build.py"))
    for p in paths:
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from profiles/hbm_traffic_<workload>.md, or None
    when absent or when the kernel's sources changed since the counters ran."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    pat = re.compile(r"^traffic: kernel=(\S+) src=(\S+) bytes_per_launch=(\d+)")
    with open(path) as fh:
        for line in fh:
            m = pat.match(line.strip())
            if m and m.group(1) == kernel and m.group(2) == source_hash(kernel):
                return int(m.group(3))
    return None


def accounting(cfg: wl.Config, B, Hkv, D, esz, ctx, kept) -> dict:
    """Algorithmic work of one step: FLOPs of one score pass and the bytes
    each HBM stage must move (d = D, element size esz)."""
    th = int(Hkv * np.asarray(ctx, dtype=np.int64).sum())          # token-heads scored
    G, W = cfg.G, cfg.W
    qo = B * cfg.Hq * D * (esz + 4.0) + 4.0 * B * cfg.Hq           # queries in, out + lse
    a = {"token_heads": th, "flop_pass": 2.0 * G * W * D * th,
         "bytes_sel": 4.0 * th + 4.0 * kept + 4.0 * B * Hkv,
         "bytes_comp": kept * (4.0 * D * esz + 8.0) + 8.0 * (B * Hkv + 1),
         "bytes_dec": 2.0 * kept * D * esz + qo}
    a["bytes_cd"] = a["bytes_comp"] + qo     # fused: kept rows read and written once
    return a


def stage_targets(kt_ms: dict, acc: dict, peak_f: float) -> dict:
    """Stage-level fractions of the two bars: both score passes against the
    MFMA peak (algorithmic FLOPs = one pass's), and select + compact +
    decode against the HBM peak, from the per-kernel event means."""
    t = {k: v * 1e-3 for k, v in kt_ms.items()}
    t_score = t["score_rowstats"] + t.get("score_fold", 0.0) + t["score_colsum"]
    t_scd = t["select"] + t["compact_decode"] + t["decode_merge"]
    return {"score_ms": t_score * 1e3,
            "score_algorithmic_tflops": acc["flop_pass"] / t_score / 1e12,
            "score_frac_of_mfma_peak": acc["flop_pass"] / t_score / 1e12 / peak_f,
            "score_executed_frac": 2 * acc["flop_pass"] / t_score / 1e12 / peak_f,
            "score_target": 0.5,
            "select_compact_decode_ms": t_scd * 1e3,
            "select_compact_decode_gbps": (acc["bytes_sel"] + acc["bytes_cd"]) / t_scd / 1e9,
            "select_compact_decode_frac_of_hbm_peak":
                (acc["bytes_sel"] + acc["bytes_cd"]) / t_scd / 1e9 / PEAK_HBM_GBPS,
            "select_compact_decode_target": 0.6}


# ---- the float64 oracle on the host ----------------------------------------

def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def oracle_stages(cfg: wl.Config, q_win, k, v, ctx, q_dec, budget_kw, threads=None) -> dict:
    """Seconds per stage of the float64 oracle (score, select, compact,
    decode) on CPU tensors; `threads` limits the BLAS pool."""
    from oracle import oracle as orc
    import contextlib
    lim = contextlib.nullcontext()
    if threads is not None:
        from threadpoolctl import threadpool_limits
        lim = threadpool_limits(limits=threads)
    with lim:
        t = [time.perf_counter()]
        s, _ = orc.window_scores(q_win, k, ctx)
        t.append(time.perf_counter())
        idx, cnt = orc.select(s, ctx, **budget_kw)
        t.append(time.perf_counter())
        k_c, v_c, pos, off = orc.compact(k, v, idx, cnt)
        t.append(time.perf_counter())
        kc = torch.from_numpy(k_c).view(k.dtype) if k.dtype == torch.bfloat16 else k_c
        vc = torch.from_numpy(v_c).view(k.dtype) if k.dtype == torch.bfloat16 else v_c
        orc.decode(q_dec, kc, vc, off, cfg.Hkv)
        t.append(time.perf_counter())
    return dict(zip(("score", "select", "compact", "decode"),
                    (t[i + 1] - t[i] for i in range(4))))


def oracle_budget_kw(cfg: wl.Config) -> dict:
    from oracle import oracle as orc
    if cfg.budget_mode == wl.BUDGET_MASS:
        return dict(mode=orc.BUDGET_MASS, mass=cfg.ratio, min_ratio=cfg.min_ratio,
                    max_ratio=cfg.max_ratio)
    return dict(mode=orc.BUDGET_RATIO, ratio=cfg.ratio)


def oracle_on_sequences(lay: wl.Layer, seqs, threads=None) -> dict:
    """The oracle on the given sequences of a layer (all KV heads)."""
    cfg = lay.cfg
    sl = list(seqs)
    cpu = lambda t: t.detach().cpu()
    ctx = cpu(lay.ctx_len)[sl]
    st = oracle_stages(cfg, cpu(lay.q_win)[sl], cpu(lay.k)[sl], cpu(lay.v)[sl], ctx,
                       cpu(lay.q_dec[0])[sl], oracle_budget_kw(cfg), threads)
    tokens = int(ctx.sum())
    dt = sum(st.values())
    return {"stage_s": st, "total_s": dt, "tokens": tokens, "tokens_per_s": tokens / dt,
            "sample": f"sequences {sl} of {cfg.B} ({tokens} cached tokens, all {cfg.Hkv} KV "
                      f"heads)", "threads": "all" if threads is None else threads}


# ---- the headline workload -------------------------------------------------

def measure_headline(lay: wl.Layer, args, extras: bool) -> dict:
    cfg = lay.cfg
    pipe = Pipeline(lay)
    pipe.two_calls = bool(getattr(args, "score_then_select", False))
    log("bench: device copy bandwidth")
    copy_bw = copy_gbps()
    log(f"bench: {torch.cuda.get_device_name(0)}; copy {copy_bw:.0f} GB/s; warmup {args.warmup}")
    settle = settle_clocks(pipe.step)
    log(f"bench: {settle} untimed steps while the clocks settle")

    # Per-kernel breakdown (every launch timed) to find the roofline kernel.
    ms_all, kt = timed_steps(pipe.step, args.steps)
    log(f"bench: {ms_all:.4f} ms per step with every launch timed; per-kernel mean ms "
        + ", ".join(f"{k}={v[0]:.4f}" for k, v in kt.items()))
    B, Hkv, N, D = lay.k.shape
    esz = lay.k.element_size()
    ctx = lay.ctx_len.cpu().numpy().astype(np.int64)
    tokens = int(ctx.sum())
    kept = int(pipe.cnt.sum().item())
    acc = accounting(cfg, B, Hkv, D, esz, ctx, kept)
    peak_f = PEAK_TFLOPS[lay.k.dtype]
    work = {"score_rowstats": ("mfma", acc["flop_pass"]), "score_colsum": ("mfma", acc["flop_pass"]),
            "select": ("hbm", acc["bytes_sel"]), "compact_decode": ("hbm", acc["bytes_cd"])}
    dom = max(work, key=lambda k: kt.get(k, (0.0,))[0])

    # The timed region: K cold steps (a 1 GiB read before each, outside its
    # events), events on the roofline kernel's dispatches.
    flush = Flush()
    settle_clocks(pipe.step, flush=flush)
    for _ in range(args.warmup):
        flush()
        pipe.step()
    torch.cuda.synchronize()
    log(f"bench: {args.warmup} warmup steps, timing {args.steps} cold steps")
    cold, wall_cold, _ = step_distribution(pipe.step, args.steps, flush)
    # The roofline kernel's own dispatch-stamped events, over as many cold
    # steps again: stamping a dispatch lengthens the step by a few us, so
    # the steps above carry no stamps.  The first 40 or so stamped steps
    # run slower than the rest (that kernel up to 3 us), so 40 stamped
    # steps go first, untimed.
    step_distribution(pipe.step, 40, flush, only=dom)
    log(f"bench: {args.steps} more cold steps with events on {dom}'s dispatches")
    cold_ev, _, kt_dom = step_distribution(pipe.step, args.steps, flush, only=dom)
    bound, amount = work[dom]
    t_dom = kt_dom[dom][0] * 1e-3
    if bound == "mfma":
        achieved, peak, unit = amount / t_dom / 1e12, peak_f, "TFLOP/s"
    else:
        achieved, peak, unit = amount / t_dom / 1e9, PEAK_HBM_GBPS, "GB/s"
    # the same steps back to back (warm: data of the previous step may still
    # be cached), one by one and as a wall-clock loop
    settle_clocks(pipe.step)
    warm, _, _ = step_distribution(pipe.step, args.steps)
    ms_b2b, _ = timed_steps(pipe.step, args.steps, events=False)
    warm_graph = graph_steps(pipe.step, args.steps)
    clocks = gpu_clocks(pipe.step)
    res = {
        "metric": METRIC,
        "value": tokens / (cold["median"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": cold["median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if lay.k.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "ctx": int(N), "Hq": cfg.Hq, "Hkv": Hkv,
                   "d": D, "W": cfg.W, "budget": "mass" if cfg.budget_mode == wl.BUDGET_MASS
                   else f"ratio {cfg.ratio}", "kept_rows": kept, "timing": "cold caches"},
        "roofline": {"kernel": dom, "bound": bound, "achieved": achieved, "peak": peak,
                     "unit": unit, "frac": achieved / peak,
                     "traffic": measured_traffic(dom, cfg.name)},
        "targets": stage_targets({k: v[0] for k, v in kt.items()}, acc, peak_f),
        "step_ms_cold": cold,
        "step_ms_cold_kernel_events": cold_ev,
        "step_ms_warm": warm,
        "warm_back_to_back_ms_per_step": ms_b2b,
        "timed_region_wall_ms": wall_cold,
        "copy_gbps": copy_bw,
        "kernels_ms": {k: v[0] for k, v in kt.items()},
        "step_ms_warm_graph": warm_graph,
        "launch_shapes": {k: {"workgroups": v[2][0], "threads": v[2][1]} for k, v in kt.items()},
        "gpu": {"name": torch.cuda.get_device_name(0), "rocm": torch.version.hip,
                "torch": torch.__version__, "clocks": clocks},
        "cpu_baseline": None,
    }
    if extras:
        t_one = one_pass_score_ms(pipe, args.steps) * 1e-3
        res["score_one_pass"] = {"ms": t_one * 1e3,
                                 "algorithmic_tflops": acc["flop_pass"] / t_one / 1e12,
                                 "algorithmic_frac": acc["flop_pass"] / t_one / 1e12 / peak_f}
        pipe.two_calls = True
        ms_two, kt_two = timed_steps(pipe.step, args.steps)
        pipe.two_calls = False
        res["score_then_select"] = {"ms_per_step_every_launch_timed": ms_two,
                                    "kernels_ms": {k: v[0] for k, v in kt_two.items()}}
        pipe.fused = False
        ms_unf, kt_unf = timed_steps(pipe.step, args.steps)
        pipe.fused = True
        t_unf = {k: v[0] * 1e-3 for k, v in kt_unf.items()}
        t_dec = t_unf["decode_split"] + t_unf["decode_merge"]
        res["decode_hbm_gbps"] = acc["bytes_dec"] / t_dec / 1e9
        res["unfused"] = {"ms_per_step_every_launch_timed": ms_unf,
                          "fused_ms_per_step_every_launch_timed": ms_all,
                          "compact_ms": t_unf["compact"] * 1e3, "decode_ms": t_dec * 1e3,
                          "compact_gbps": acc["bytes_comp"] / t_unf["compact"] / 1e9}
        res["vector_routing"] = vector_measure(pipe, args.steps)
        # Quality beside throughput: loss terms of the step's compacted cache
        # against the full cache, for the workload's decode queries and for
        # the last window row of every query head.
        pipe.step()
        out_f, lse_f = fidelity.full_cache_decode(pipe.qd, pipe.k, pipe.v, pipe.c)
        res["fidelity"] = fidelity.summary(fidelity.fidelity(pipe.out, pipe.lse, out_f, lse_f))
        q_last = pipe.q[:, :, -1, :].contiguous()
        out_w, lse_w = api.kv_decode_attn(q_last, pipe.comp[0], pipe.comp[1], pipe.comp[3],
                                          cfg.Hkv, workspace=pipe.ws_d)
        out_f, lse_f = fidelity.full_cache_decode(q_last, pipe.k, pipe.v, pipe.c)
        res["fidelity_window_query"] = fidelity.summary(
            fidelity.fidelity(out_w, lse_w, out_f, lse_f))
    del flush, pipe
    torch.cuda.empty_cache()
    return res


# ---- the other workloads ---------------------------------------------------

def measure_workload(lay: wl.Layer, steps: int) -> dict:
    """Step time (cold and warm medians) and per-kernel means of a single-layer
    workload, with its stage-level fractions."""
    cfg = lay.cfg
    pipe = Pipeline(lay)
    settle_clocks(pipe.step)
    _, kt = timed_steps(pipe.step, steps)
    flush = Flush()
    settle_clocks(pipe.step, flush=flush)
    cold, _, _ = step_distribution(pipe.step, steps, flush)
    settle_clocks(pipe.step)
    warm, _, _ = step_distribution(pipe.step, steps)
    B, Hkv, N, D = lay.k.shape
    ctx = lay.ctx_len.cpu().numpy().astype(np.int64)
    kept = int(pipe.cnt.sum().item())
    acc = accounting(cfg, B, Hkv, D, lay.k.element_size(), ctx, kept)
    tokens = int(ctx.sum())
    k_hist = None
    if cfg.budget_mode == wl.BUDGET_MASS:
        r = pipe.cnt.cpu().numpy() / np.repeat(ctx, Hkv)
        k_hist = {"kept_fraction_min": float(r.min()), "median": float(np.median(r)),
                  "max": float(r.max()),
                  "at_lower_clamp": int(np.sum(np.isclose(r, cfg.min_ratio, atol=1e-3))),
                  "at_upper_clamp": int(np.sum(np.isclose(r, cfg.max_ratio, atol=1e-3))),
                  "heads": int(r.size)}
    out = {"config": {"B": B, "ctx": int(N), "ctx_total": tokens, "Hq": cfg.Hq, "Hkv": Hkv,
                      "d": D, "W": cfg.W, "kept_rows": kept},
           "tokens_per_s_cold": tokens / (cold["median"] * 1e-3),
           "step_ms_cold": cold, "step_ms_warm": warm,
           "kernels_ms": {k: v[0] for k, v in kt.items()},
           "targets": stage_targets({k: v[0] for k, v in kt.items()}, acc,
                                    PEAK_TFLOPS[lay.k.dtype])}
    if k_hist:
        out["kept_fraction"] = k_hist
    del flush, pipe
    torch.cuda.empty_cache()
    return out


class LongContext:
    """The 128K workload as configured: L layers, each scored, selected and
    compacted into a cache of its own, then S decode steps layer-inner (step
    s: layers 0..L-1, each a fresh query over that layer's compacted cache)."""

    def __init__(self, cfg: wl.Config, layers: int):
        self.cfg = cfg
        self.lays = [wl.make_layer_device(cfg, l, DEV) for l in range(layers)]
        B, Hkv, N, D = self.lays[0].k.shape
        self.shape = (B, Hkv, N, D)
        self.budget = budget_of(cfg)
        self.cap = capacity_of(cfg, B, Hkv, N)
        self.scores = torch.empty(B, Hkv, N, device=DEV, dtype=torch.float32)
        self.ws_s = torch.zeros(api.kv_score_select_workspace_size(B, cfg.Hq, Hkv, N, cfg.W, D),
                                device=DEV, dtype=torch.uint8)
        self.idx = torch.empty(B, Hkv, N, device=DEV, dtype=torch.int32)
        self.cnt = torch.empty(B * Hkv, device=DEV, dtype=torch.int32)
        dt = self.lays[0].k.dtype
        self.caches = [(torch.empty(self.cap, D, device=DEV, dtype=dt),
                        torch.empty(self.cap, D, device=DEV, dtype=dt),
                        torch.empty(self.cap, device=DEV, dtype=torch.int32),
                        torch.empty(B * Hkv + 1, device=DEV, dtype=torch.int64))
                       for _ in self.lays]
        self.out = torch.empty(B, cfg.Hq, D, device=DEV, dtype=torch.float32)
        self.lse = torch.empty(B, cfg.Hq, device=DEV, dtype=torch.float32)
        self.ws_d = torch.zeros(api.kv_decode_workspace_size(B, cfg.Hq, Hkv, D, self.cap),
                                device=DEV, dtype=torch.uint8)

    def compress(self):
        for lay, cache in zip(self.lays, self.caches):
            api.kv_score_select(lay.q_win, lay.k, None, self.budget, scores=self.scores,
                                kept_idx=self.idx, kept_count=self.cnt, workspace=self.ws_s)
            api.kv_compact(lay.k, lay.v, self.idx, self.cnt, self.cap, out=cache)

    def decode(self, steps: int):
        for s in range(steps):
            for lay, cache in zip(self.lays, self.caches):
                api.kv_decode_attn(lay.q_dec[s], cache[0], cache[1], cache[3], self.cfg.Hkv,
                                   out=self.out, lse=self.lse, workspace=self.ws_d)


def measure_long128k(layers: int = 32, steps: int = 128, reps: int = 3) -> dict:
    cfg = wl.CONFIGS["long128k"]
    log(f"bench: long128k, {layers} layers drawn on the device")
    lc = LongContext(cfg, layers)
    B, Hkv, N, D = lc.shape
    esz = lc.lays[0].k.element_size()
    settle_clocks(lc.compress, 0.2)
    # compression of all layers, wall clock (each layer's K and V are read
    # once per pass: 17 GB cycle through, so nothing stays cached)
    walls = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        lc.compress()
        torch.cuda.synchronize()
        walls.append((time.perf_counter() - t0) * 1e3)
    _, kt_c = timed_steps(lc.compress, 1)
    kept = int(lc.cnt.sum().item())
    # decode: every call's kernels timed (eager), then the whole S x L loop
    # captured as one HIP graph and replayed (launch overhead out of the way)
    _, kt_d = timed_steps(lambda: lc.decode(steps), 1)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lc.decode(1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        lc.decode(steps)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    replays = []
    for _ in range(reps):
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        replays.append((time.perf_counter() - t0) * 1e3)
    calls = steps * layers
    bytes_call = 2.0 * kept * D * esz + B * cfg.Hq * D * (esz + 4.0) + 4.0 * B * cfg.Hq
    t_split, t_merge = kt_d["decode_split"][0], kt_d["decode_merge"][0]
    t_graph = float(np.median(replays)) * 1e-3
    compress_ms = float(np.median(walls))
    tokens = N * B * layers
    acc = accounting(cfg, B, Hkv, D, esz, [N] * B, kept)
    res = {"config": {"B": B, "ctx": N, "layers": layers, "Hq": cfg.Hq, "Hkv": Hkv, "d": D,
                      "W": cfg.W, "budget": f"ratio {cfg.ratio}", "kept_rows_per_layer": kept,
                      "decode_steps": steps, "data": "drawn on the device (torch generator)"},
           "compress_ms_all_layers": compress_ms,
           "compress_ms_per_layer": compress_ms / layers,
           "tokens_per_s": tokens / (compress_ms * 1e-3),
           "compress_kernels_ms": {k: v[0] for k, v in kt_c.items()},
           "score_frac_of_mfma_peak": acc["flop_pass"] / (
               (kt_c["score_rowstats"][0] + kt_c.get("score_fold", (0.0,))[0]
                + kt_c["score_colsum"][0]) * 1e-3) / 1e12 / PEAK_TFLOPS[torch.bfloat16],
           "compacted_cache_gb": 2.0 * kept * D * esz * layers / 1e9,
           "decode_calls": calls,
           "decode_graph_ms": t_graph * 1e3,
           "decode_us_per_call_graph": t_graph / calls * 1e6,
           "decode_gbps_graph": bytes_call * calls / t_graph / 1e9,
           "decode_split_us": t_split * 1e3, "decode_merge_us": t_merge * 1e3,
           "decode_gbps_kernels": bytes_call / ((t_split + t_merge) * 1e-3) / 1e9,
           "decode_split_gbps": (2.0 * kept * D * esz) / (t_split * 1e-3) / 1e9}
    res["decode_frac_of_hbm_peak"] = res["decode_gbps_graph"] / PEAK_HBM_GBPS
    del g, lc
    torch.cuda.empty_cache()
    return res


def oracle_long128k_head(layer_tensors: wl.Layer, h: int = 0) -> dict:
    """The oracle on one KV head of one 128K layer (its 4 query heads and
    128 window rows over 131072 tokens), scaled to the layer's 8 heads."""
    cfg = layer_tensors.cfg
    G = cfg.G
    cpu = lambda t: t.detach().cpu()
    lay = layer_tensors
    one_head = dataclass_with(cfg, Hq=G, Hkv=1)
    st = oracle_stages(one_head, cpu(lay.q_win[:, h * G:(h + 1) * G]), cpu(lay.k[:, h:h + 1]),
                       cpu(lay.v[:, h:h + 1]), cpu(lay.ctx_len),
                       cpu(lay.q_dec[0][:, h * G:(h + 1) * G]), oracle_budget_kw(cfg))
    dt = sum(st.values())
    n = int(lay.ctx_len.sum())
    return {"stage_s": st, "total_s": dt, "tokens_per_s": n / (dt * cfg.Hkv),
            "sample": f"KV head {h} of layer 0 ({n} tokens, {G} query heads x {cfg.W} window "
                      f"rows); tokens/s counts all {cfg.Hkv} heads of a token (one head's time "
                      f"x {cfg.Hkv})", "threads": "all"}


def dataclass_with(cfg, **kw):
    import dataclasses
    return dataclasses.replace(cfg, **kw)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this path runs on one GPU; every stage is independent "
                          "per (sequence, KV head), so more GPUs shard heads with no exchange "
                          "and no multi-GPU run is provided", "n_gpus": args.gpus}))
        sys.exit(2)
    cores = len(os.sched_getaffinity(0))
    cfg = wl.CONFIGS[args.workload]

    if cfg.name == "long128k":
        res = long128k_line(args, cores)
        print(json.dumps(res), flush=True)
        return

    log(f"bench: generating {cfg.name}")
    lay = wl.make_layer(cfg) if cfg.name != "ragged_adaptive" else wl.make_layer_device(cfg)
    extras = not args.no_extras and cfg.name == "needle32k"
    res = measure_headline(lay, args, extras)
    cb = None
    if not args.no_cpu_baseline:
        log("bench: oracle baseline on the host")
        nseq = min(args.cpu_seqs, cfg.B)
        o = oracle_on_sequences(lay, range(nseq))
        frac = nseq / cfg.B
        kt = res["kernels_ms"]
        gpu_s = {"score": (kt["score_rowstats"] + kt.get("score_fold", 0.0)
                           + kt["score_colsum"]) * 1e-3,
                 "select": kt["select"] * 1e-3,
                 "compact_decode": (kt["compact_decode"] + kt["decode_merge"]) * 1e-3}
        cpu_s = dict(o["stage_s"], compact_decode=o["stage_s"]["compact"] + o["stage_s"]["decode"])
        cb = {"value": o["tokens_per_s"], "unit": "tokens/s", "cores": cores,
              "blas_threads": blas_threads(), "kind": "oracle",
              "sample": o["sample"] + f": float64 score+select+compact+decode, "
                                      f"{o['total_s']:.2f} s",
              "stage_s": o["stage_s"], "fraction_of_batch": frac,
              "stage_speedup": {k: cpu_s[k] / frac / gpu_s[k] for k in gpu_s}}
    del lay
    if extras:
        res["workloads"] = {}
        per = {}
        for name in ("tiny", "llama8b_layer", "ragged_adaptive"):
            c = wl.CONFIGS[name]
            log(f"bench: workload {name}")
            lw = wl.make_layer(c) if name != "ragged_adaptive" else wl.make_layer_device(c)
            res["workloads"][name] = measure_workload(lw, args.steps)
            if not args.no_cpu_baseline:
                seqs = range(c.B) if c.B <= 2 else range(2)
                per[name] = {"all_threads": oracle_on_sequences(lw, seqs)}
                if name in ("tiny", "llama8b_layer"):
                    per[name]["one_thread"] = oracle_on_sequences(lw, seqs, threads=1)
            del lw
            torch.cuda.empty_cache()
        res["workloads"]["long128k"] = measure_long128k()
        if not args.no_cpu_baseline:
            l0 = wl.make_layer_device(wl.CONFIGS["long128k"], 0, DEV)
            per["long128k"] = {"all_threads": oracle_long128k_head(l0)}
            del l0
            torch.cuda.empty_cache()
        if cb is not None:
            cb["per_workload"] = per
    res["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)


def long128k_line(args, cores) -> dict:
    """The JSON line for --workload long128k: one step = the 32 layers
    scored, selected and compacted (value: cached tokens/s over the layers),
    with the 128 decode steps layer-inner reported beside it; the roofline
    kernel is the decode split, which holds most of the GPU time."""
    r = measure_long128k()
    cfg = wl.CONFIGS["long128k"]
    c = r["config"]
    res = {"metric": METRIC, "value": r["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
           "steps": 1, "warmup": 0, "ms_per_step": r["compress_ms_all_layers"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": dict(c, workload=cfg.name),
           "roofline": {"kernel": "decode_split", "bound": "hbm",
                        "achieved": r["decode_split_gbps"], "peak": PEAK_HBM_GBPS,
                        "unit": "GB/s", "frac": r["decode_split_gbps"] / PEAK_HBM_GBPS,
                        "traffic": measured_traffic("decode_split", cfg.name)},
           "long128k": r, "cpu_baseline": None}
    if not args.no_cpu_baseline:
        l0 = wl.make_layer_device(cfg, 0, DEV)
        o = oracle_long128k_head(l0)
        res["cpu_baseline"] = {"value": o["tokens_per_s"], "unit": "tokens/s", "cores": cores,
                               "blas_threads": blas_threads(), "kind": "oracle",
                               "sample": o["sample"], "stage_s": o["stage_s"]}
    return res


if __name__ == "__main__":
    main()
