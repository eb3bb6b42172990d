#!/usr/bin/env python3
"""Throughput of the score -> select -> compact -> decode path on one GPU.

One step = kv_score + kv_select + kv_compact_decode (kv_compact and
kv_decode_attn in one pass over the kept rows) over one batch
of the chosen synthetic workload (default: batch 4 at 32K context, 32 query
/ 8 KV heads, d = 128, W = 64, keep 10%, one decode step), inputs resident
in HBM before timing starts.  Prints one JSON line:

  value       cached tokens per second over the whole step
  roofline    the kernel with the most GPU time: algorithmic FLOPs (MFMA
              kernels) or bytes (HBM kernels) per launch / its mean duration,
              durations from hipEvents the library records on its launch
              stream around every kernel of the timed steps; `traffic` is the
              HBM bytes per launch that rocprofv3's FETCH_SIZE + WRITE_SIZE
              counters read for that kernel (scaled by the ratio of known to
              counted bytes of a plain device copy), taken from the committed
              summary under profiles/ and reported only while the kernel's
              sources still hash to the recorded value
  copy_gbps   a 1 GiB device-to-device copy (read + write bytes / time)
  unfused     the same step with kv_compact and kv_decode_attn as two calls;
              decode_hbm_gbps is that decode's rate
  fidelity    output / log-sum-exp loss terms of the compacted cache
              against the full cache for the step's decode queries (and,
              fidelity_window_query, for the last window row of each head)
  vector_routing  VECTOR three-way routing (route, routed compaction,
              decode rebuilding dropped values) at the same memory budget
  score_one_pass  kv_score_from_lse (row LSEs given, as a prefill pass
              yields them): one sweep over K instead of two
  cpu_baseline the float64 oracle on a bounded sample on the host cores
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import math
import os
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


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="needle32k", choices=sorted(wl.CONFIGS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seqs", type=int, default=4,
                   help="sequences of the batch the oracle baseline processes")
    return p.parse_args()


class Pipeline:
    def __init__(self, lay: wl.Layer, fused: bool = True):
        cfg = lay.cfg
        self.cfg = cfg
        self.fused = fused
        d = torch.device("cuda:0")
        self.q = lay.q_win.to(d)
        self.k = lay.k.to(d)
        self.v = lay.v.to(d)
        self.c = lay.ctx_len.to(d)
        self.qd = lay.q_dec[0].to(d)
        B, Hkv, N, D = lay.k.shape
        if cfg.budget_mode == wl.BUDGET_MASS:
            self.budget = api.Budget(api.BUDGET_MASS, mass=cfg.ratio, min_ratio=cfg.min_ratio,
                                     max_ratio=cfg.max_ratio)
            self.cap = int(math.ceil(B * Hkv * N * cfg.max_ratio))
        else:
            self.budget = api.Budget(api.BUDGET_RATIO, ratio_scalar=cfg.ratio)
            self.cap = B * Hkv * max(1, int(math.floor(float(np.float32(cfg.ratio)) * N + 0.5)))
        f32 = torch.float32
        self.scores = torch.empty(B, Hkv, N, device=d, dtype=f32)
        self.ws_s = torch.zeros(api.kv_score_workspace_size(B, cfg.Hq, Hkv, N, cfg.W, D),
                                device=d, dtype=torch.uint8)
        self.idx = torch.empty(B, Hkv, N, device=d, dtype=torch.int32)
        self.cnt = torch.empty(B * Hkv, device=d, dtype=torch.int32)
        self.comp = (torch.empty(self.cap, D, device=d, dtype=lay.k.dtype),
                     torch.empty(self.cap, D, device=d, dtype=lay.k.dtype),
                     torch.empty(self.cap, device=d, dtype=torch.int32),
                     torch.empty(B * Hkv + 1, device=d, dtype=torch.int64))
        self.out = torch.empty(B, cfg.Hq, D, device=d, dtype=f32)
        self.lse = torch.empty(B, cfg.Hq, device=d, dtype=f32)
        self.ws_d = torch.zeros(api.kv_decode_workspace_size(B, cfg.Hq, Hkv, D, self.cap),
                                device=d, dtype=torch.uint8)

    def step(self):
        api.kv_score(self.q, self.k, self.c, scores=self.scores, workspace=self.ws_s)
        api.kv_select(self.scores, self.c, self.budget, kept_idx=self.idx, kept_count=self.cnt)
        if self.fused:
            api.kv_compact_decode(self.k, self.v, self.idx, self.cnt, self.cap, self.qd,
                                  out=self.comp, attn_out=self.out, lse=self.lse,
                                  workspace=self.ws_d)
            return
        k_c, v_c, _, off = api.kv_compact(self.k, self.v, self.idx, self.cnt, self.cap,
                                          out=self.comp)
        api.kv_decode_attn(self.qd, k_c, v_c, off, self.cfg.Hkv, out=self.out, lse=self.lse,
                           workspace=self.ws_d)


def settle_clocks(pipe: Pipeline, seconds: float = 0.1) -> int:
    """Run the step untimed for about `seconds` of wall time.  From a cold
    start the GPU needs a few tens of ms of sustained load before its clocks
    settle (the first steps run up to 20% slower), so the warmup steps alone
    would leave the timed region on the ramp.  Returns the steps run."""
    n = 0
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(10):
            pipe.step()
        n += 10
        torch.cuda.synchronize()
    return n


def timed_steps(pipe: Pipeline, steps: int, only=None):
    """Wall-clock ms per step and the event timings of the same steps: every
    kernel, or (only=name) one kernel, so that only one launch per step is a
    timed dispatch (the events are stamped by the dispatch itself, which still
    slows a timed launch by a few us)."""
    L = _lib.lib()
    torch.cuda.synchronize()
    L.kv_timing_only(only.encode() if only else None)
    L.kv_timing_enable(1)
    t0 = time.perf_counter()
    for _ in range(steps):
        pipe.step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    buf = (_lib.KvKernelTime * 32)()
    n = L.kv_timing_read(buf, 32)
    L.kv_timing_enable(0)
    L.kv_timing_only(None)
    if n < 0:
        raise RuntimeError(f"kv_timing_read failed: {n}")
    return ms, {buf[i].name.decode(): (buf[i].total_ms / buf[i].launches, buf[i].launches)
                for i in range(n)}


def one_pass_score_ms(pipe: Pipeline, steps: int) -> float:
    """Mean event time of kv_score_from_lse (the score stage when the row
    LSEs come from the prefill), fed the row LSEs of a two-pass call."""
    L = _lib.lib()
    _, lse = api.kv_score(pipe.q, pipe.k, pipe.c, with_row_lse=True)
    out = torch.empty_like(pipe.scores)
    for _ in range(3):
        api.kv_score_from_lse(pipe.q, pipe.k, pipe.c, lse, scores=out)
    torch.cuda.synchronize()
    L.kv_timing_only(b"score_colsum")
    L.kv_timing_enable(1)
    for _ in range(steps):
        api.kv_score_from_lse(pipe.q, pipe.k, pipe.c, lse, scores=out)
    torch.cuda.synchronize()
    buf = (_lib.KvKernelTime * 4)()
    n = L.kv_timing_read(buf, 4)
    L.kv_timing_enable(0)
    L.kv_timing_only(None)
    if n != 1:
        raise RuntimeError(f"kv_timing_read returned {n}")
    return buf[0].total_ms / buf[0].launches


def vector_measure(pipe: Pipeline, steps: int) -> dict:
    """VECTOR routing at the same memory as the headline's 10% keep (p_c =
    0.9, p_a = 0.05: keys for 15% of the tokens, values for 5%), with a
    seeded random linear map W and rotary base 500000, timed per kernel over
    `steps` route + compact + decode passes."""
    L = _lib.lib()
    cfg = pipe.cfg
    B, Hkv, N, D = pipe.k.shape
    g = torch.Generator().manual_seed(7)
    w = (torch.randn(Hkv, D, D, generator=g) / math.sqrt(D)).to("cuda:0")
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
    L.kv_timing_enable(1)
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    buf = (_lib.KvKernelTime * 32)()
    n = L.kv_timing_read(buf, 32)
    L.kv_timing_enable(0)
    kt = {buf[i].name.decode(): buf[i].total_ms / buf[i].launches for i in range(n)}
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
    src = torch.empty(COPY_BYTES // 4, device="cuda:0", dtype=torch.float32).fill_(1.0)
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


def step_distribution(pipe: Pipeline, steps: int, flush=None) -> dict:
    """Per-step times (ms) from torch events around each step on the stream the
    library launches on: median, p10 and p90.  `flush`, if given, runs before
    every step, outside the timed interval."""
    st = torch.cuda.current_stream()
    ev = []
    for _ in range(steps):
        if flush is not None:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        pipe.step()
        e1.record(st)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    ms = np.sort(np.array([a.elapsed_time(b) for a, b in ev]))
    return {"median": float(np.median(ms)), "p10": float(np.percentile(ms, 10)),
            "p90": float(np.percentile(ms, 90)), "steps": steps}


def cpu_baseline(lay: wl.Layer, nseq: int):
    """The float64 oracle, as it stands, on the first nseq sequences."""
    from oracle import oracle as orc
    cfg = lay.cfg
    sl = slice(0, nseq)
    ctx = lay.ctx_len[sl]
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    t = [time.perf_counter()]
    s, _ = orc.window_scores(lay.q_win[sl], lay.k[sl], ctx)
    t.append(time.perf_counter())
    if cfg.budget_mode == wl.BUDGET_MASS:
        idx, cnt = orc.select(s, ctx, orc.BUDGET_MASS, mass=cfg.ratio,
                              min_ratio=cfg.min_ratio, max_ratio=cfg.max_ratio)
    else:
        idx, cnt = orc.select(s, ctx, orc.BUDGET_RATIO, ratio=cfg.ratio)
    t.append(time.perf_counter())
    k_c, v_c, pos, off = orc.compact(lay.k[sl], lay.v[sl], idx, cnt)
    t.append(time.perf_counter())
    kc = torch.from_numpy(k_c).view(lay.k.dtype) if lay.k.dtype == torch.bfloat16 else k_c
    vc = torch.from_numpy(v_c).view(lay.k.dtype) if lay.k.dtype == torch.bfloat16 else v_c
    orc.decode(lay.q_dec[0][sl], kc, vc, off, cfg.Hkv)
    t.append(time.perf_counter())
    dt = t[-1] - t[0]
    tokens = int(ctx.sum())
    stages = dict(zip(("score", "select", "compact", "decode"),
                      (t[i + 1] - t[i] for i in range(4))))
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"sequences 0..{nseq - 1} of the batch ({tokens} cached tokens, all "
                      f"{cfg.Hkv} KV heads): float64 score+select+compact+decode, {dt:.2f} s",
            "stage_s": stages, "fraction_of_batch": nseq / lay.cfg.B}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this path runs on one GPU; every stage is independent "
                          "per (sequence, KV head), so more GPUs shard heads with no exchange "
                          "and no multi-GPU run is provided", "n_gpus": args.gpus}))
        sys.exit(2)

    cfg = wl.CONFIGS[args.workload]
    log(f"bench: generating {cfg.name}")
    lay = wl.make_layer(cfg)
    pipe = Pipeline(lay)
    log("bench: device copy bandwidth")
    copy_bw = copy_gbps()
    log(f"bench: {torch.cuda.get_device_name(0)}; copy {copy_bw:.0f} GB/s; warmup {args.warmup}")
    settle = settle_clocks(pipe)
    log(f"bench: {settle} untimed steps while the clocks settle")

    # Per-kernel breakdown (every launch timed), then the timed region with
    # events on the roofline kernel only.
    ms_all, kt = timed_steps(pipe, args.steps)
    log(f"bench: {ms_all:.4f} ms per step with every launch timed; per-kernel mean ms "
        + ", ".join(f"{k}={v[0]:.4f}" for k, v in kt.items()))

    B, Hkv, N, D = lay.k.shape
    G, W = cfg.G, cfg.W
    esz = lay.k.element_size()
    ctx = lay.ctx_len.numpy().astype(np.int64)
    tokens = int(ctx.sum())
    th = int(Hkv * ctx.sum())                       # token-heads scored
    kept = int(pipe.cnt.sum().item())
    flop_pass = 2.0 * G * W * D * th
    bytes_sel = 4.0 * th + 4.0 * kept + 4.0 * B * Hkv
    bytes_comp = kept * (4.0 * D * esz + 8.0) + 8.0 * (B * Hkv + 1)
    bytes_dec = 2.0 * kept * D * esz + B * cfg.Hq * D * (esz + 4.0) + 4.0 * B * cfg.Hq
    # fused: the kept rows are read and written once, plus the queries and outputs
    bytes_cd = bytes_comp + B * cfg.Hq * D * (esz + 4.0) + 4.0 * B * cfg.Hq
    peak_f = PEAK_TFLOPS[lay.k.dtype]
    work = {"score_rowstats": ("mfma", flop_pass), "score_colsum": ("mfma", flop_pass),
            "select": ("hbm", bytes_sel), "compact_decode": ("hbm", bytes_cd)}
    dom = max(work, key=lambda k: kt.get(k, (0.0,))[0])
    # the host work since the last step leaves the GPU idle long enough for
    # its clocks to drop: settle them again, right before the warmup steps
    settle_clocks(pipe)
    for _ in range(args.warmup):
        pipe.step()
    torch.cuda.synchronize()
    log(f"bench: {args.warmup} warmup steps, timing {args.steps} steps (events on {dom})")
    ms, kt_dom = timed_steps(pipe, args.steps, only=dom)
    bound, amount = work[dom]
    t_dom = kt_dom[dom][0] * 1e-3
    if bound == "mfma":
        achieved, peak, unit = amount / t_dom / 1e12, peak_f, "TFLOP/s"
    else:
        achieved, peak, unit = amount / t_dom / 1e9, PEAK_HBM_GBPS, "GB/s"
    t_one = one_pass_score_ms(pipe, args.steps) * 1e-3
    pipe.fused = False
    ms_unf, kt_unf = timed_steps(pipe, args.steps)
    pipe.fused = True
    t_unf = {k: v[0] * 1e-3 for k, v in kt_unf.items()}
    t_dec = t_unf["decode_split"] + t_unf["decode_merge"]
    vec = vector_measure(pipe, args.steps)
    # per-step spread, back to back and from cold caches (a 1 GiB buffer
    # overwritten before every step, outside the timed interval)
    # Cold: a 1 GiB buffer is read before every step, so that the L2 and the
    # 256 MB Infinity Cache hold nothing of the step's data, and nothing
    # dirty.  (Overwriting the buffer instead leaves up to 256 MB of dirty
    # lines whose write-back lands inside the next step: reported apart.)
    settle_clocks(pipe)
    warm = step_distribution(pipe, args.steps)
    buf = torch.ones(1 << 28, device="cuda", dtype=torch.float32)
    cold = step_distribution(pipe, args.steps, lambda: buf.sum())
    cold_w = step_distribution(pipe, args.steps, lambda: buf.fill_(1.0))
    del buf
    t = {k: v[0] * 1e-3 for k, v in kt.items()}
    t_score = t["score_rowstats"] + t.get("score_fold", 0.0) + t["score_colsum"]   # fold: row LSEs asked for
    t_cd = t["compact_decode"] + t["decode_merge"]
    t_scd = t["select"] + t_cd
    res = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if lay.k.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "ctx": int(N), "Hq": cfg.Hq, "Hkv": Hkv,
                   "d": D, "W": W, "budget": "mass" if cfg.budget_mode == wl.BUDGET_MASS
                   else f"ratio {cfg.ratio}", "kept_rows": kept},
        "roofline": {"kernel": dom, "bound": bound, "achieved": achieved, "peak": peak,
                     "unit": unit, "frac": achieved / peak,
                     "traffic": measured_traffic(dom, cfg.name)},
        "copy_gbps": copy_bw,
        "decode_hbm_gbps": bytes_dec / t_dec / 1e9,
        "unfused": {"ms_per_step_every_launch_timed": ms_unf,
                    "fused_ms_per_step_every_launch_timed": ms_all,
                    "compact_ms": t_unf["compact"] * 1e3,
                    "decode_ms": t_dec * 1e3,
                    "compact_gbps": bytes_comp / t_unf["compact"] / 1e9},
        "score_stage": {"ms": t_score * 1e3,
                        "algorithmic_tflops": flop_pass / t_score / 1e12,
                        "algorithmic_frac": flop_pass / t_score / 1e12 / peak_f,
                        "executed_frac": 2 * flop_pass / t_score / 1e12 / peak_f},
        "score_one_pass": {"ms": t_one * 1e3,
                           "algorithmic_tflops": flop_pass / t_one / 1e12,
                           "algorithmic_frac": flop_pass / t_one / 1e12 / peak_f},
        "vector_routing": vec,
        "select_compact_decode": {"ms": t_scd * 1e3,
                                  "gbps": (bytes_sel + bytes_cd) / t_scd / 1e9,
                                  "frac": (bytes_sel + bytes_cd) / t_scd / 1e9 / PEAK_HBM_GBPS},
        "kernels_ms": {k: v[0] for k, v in kt.items()},
        "step_ms_warm": warm,
        "step_ms_cold": cold,
        "step_ms_after_1gib_write": cold_w,
        "cpu_baseline": None,
    }
    # Quality beside throughput: loss terms of the step's compacted cache
    # against the full cache for the step's decode queries.
    # Two query sets: the workload's i.i.d. decode queries, and the last
    # window row of every query head (the window is the method's own proxy
    # for the queries to come).
    out_f, lse_f = fidelity.full_cache_decode(pipe.qd, pipe.k, pipe.v, pipe.c)
    res["fidelity"] = fidelity.summary(fidelity.fidelity(pipe.out, pipe.lse, out_f, lse_f))
    q_last = pipe.q[:, :, -1, :].contiguous()
    out_w, lse_w = api.kv_decode_attn(q_last, pipe.comp[0], pipe.comp[1], pipe.comp[3],
                                      cfg.Hkv, workspace=pipe.ws_d)
    out_f, lse_f = fidelity.full_cache_decode(q_last, pipe.k, pipe.v, pipe.c)
    res["fidelity_window_query"] = fidelity.summary(fidelity.fidelity(out_w, lse_w, out_f, lse_f))
    del out_f, lse_f, out_w, lse_w
    if not args.no_cpu_baseline:
        log("bench: oracle baseline on the host")
        cb = cpu_baseline(lay, min(args.cpu_seqs, B))
        gpu_s = {"score": t_score, "select": t["select"], "compact_decode": t_cd}
        cpu_s = dict(cb["stage_s"], compact_decode=cb["stage_s"]["compact"] + cb["stage_s"]["decode"])
        cb["stage_speedup"] = {k: cpu_s[k] / cb["fraction_of_batch"] / gpu_s[k] for k in gpu_s}
        res["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
