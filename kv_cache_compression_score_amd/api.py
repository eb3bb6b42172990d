"""Python binding of libkvcc.so: the four C entry points over torch tensors.

Each function only checks and marshals arguments (device pointers, sizes,
the current HIP stream) and allocates outputs and workspace through torch;
every step of the computation runs in the library's HIP kernels.  Calls are
asynchronous on ``torch.cuda.current_stream()``.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import torch

from ._lib import KV_BF16, KV_F32, KvBudget, lib

BUDGET_K = 0
BUDGET_RATIO = 1
BUDGET_THRESHOLD = 2
BUDGET_MASS = 3


class KvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().kv_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


@dataclasses.dataclass
class Budget:
    """Per-head budget; see kv_budget in include/kvcc.h."""
    mode: int = BUDGET_RATIO
    k: Optional[torch.Tensor] = None        # device int32 [B*Hkv]
    ratio: Optional[torch.Tensor] = None    # device fp32 [B*Hkv]
    k_scalar: int = 0
    ratio_scalar: float = 0.0
    tau: float = 0.0
    mass: float = 0.0
    min_ratio: float = 0.0
    max_ratio: float = 1.0
    n_sink: int = 0                         # first tokens always kept
    n_recent: int = 0                       # last tokens always kept

    def to_c(self) -> KvBudget:
        return KvBudget(self.mode, _ptr(self.k), _ptr(self.ratio), int(self.k_scalar),
                        float(self.ratio_scalar), float(self.tau), float(self.mass),
                        float(self.min_ratio), float(self.max_ratio),
                        int(self.n_sink), int(self.n_recent))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KV_BF16
    if t.dtype == torch.float32:
        return KV_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _call(fn: str, status: int):
    if status != 0:
        raise KvError(fn, status)


def kv_score_workspace_size(B, Hq, Hkv, N_max, W, d) -> int:
    return int(lib().kv_score_workspace_size(B, Hq, Hkv, N_max, W, d))


def _check_lengths(ctx_len, ctx_len_host, B: int, N_max: int, W: int, causal: bool):
    """Per-sequence preconditions the library cannot check on the host:
    0 <= n_b <= N_max, and W <= n_b when the window is causal (its rows sit
    at the last W positions).  Uses ctx_len_host when given; otherwise a
    causal call reads the device lengths back (one synchronisation)."""
    if ctx_len is None:
        if causal and W > N_max:
            raise ValueError(f"causal scoring needs W <= n_b (W={W}, N_max={N_max})")
        return
    if ctx_len_host is None:
        if not causal:
            return
        ctx_len_host = ctx_len.cpu()
    n = [int(x) for x in (ctx_len_host.tolist() if hasattr(ctx_len_host, "tolist")
                          else ctx_len_host)]
    if len(n) != B:
        raise ValueError(f"ctx_len has {len(n)} entries, expected {B}")
    for b, nb in enumerate(n):
        if not 0 <= nb <= N_max:
            raise ValueError(f"ctx_len[{b}] = {nb} outside [0, {N_max}]")
        if causal and nb < W:
            raise ValueError(f"causal scoring needs W <= n_b: ctx_len[{b}] = {nb} < W = {W}")


def kv_score(q_win: torch.Tensor, k: torch.Tensor, ctx_len: Optional[torch.Tensor] = None, *,
             scale: float = 0.0, causal: bool = False, with_row_lse: bool = False,
             scores: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
             ctx_len_host=None):
    """Window scores [B][Hkv][N_max] fp32 (and row LSE [B][Hq][W] if asked).

    ctx_len_host (host sequence of the B lengths) lets the binding check the
    per-sequence limits without reading ctx_len back."""
    _check(q_win, "q_win"); _check(k, "k")
    B, Hq, W, d = q_win.shape
    _, Hkv, N_max, _ = k.shape
    _check_lengths(ctx_len, ctx_len_host, B, N_max, W, causal)
    if scores is None:
        scores = torch.empty(B, Hkv, N_max, device=k.device, dtype=torch.float32)
    row_lse = torch.empty(B, Hq, W, device=k.device, dtype=torch.float32) if with_row_lse else None
    need = kv_score_workspace_size(B, Hq, Hkv, N_max, W, d)
    if workspace is None:
        workspace = torch.zeros(max(need, 1), device=k.device, dtype=torch.uint8)
    if ctx_len is not None:
        _check(ctx_len, "ctx_len")
    _call("kv_score", lib().kv_score(
        _ptr(q_win), _ptr(k), _ptr(ctx_len), _ptr(scores), _ptr(row_lse),
        B, Hq, Hkv, N_max, W, d, _dtype_code(k), int(bool(causal)), float(scale),
        _ptr(workspace), workspace.numel(), _stream()))
    return scores, row_lse


def kv_score_from_lse(q_win: torch.Tensor, k: torch.Tensor, ctx_len: Optional[torch.Tensor],
                      row_lse_in: torch.Tensor, *, scale: float = 0.0, causal: bool = False,
                      scores: Optional[torch.Tensor] = None, ctx_len_host=None):
    """Window scores [B][Hkv][N_max] fp32 in one sweep, given the row LSE [B][Hq][W]."""
    _check(q_win, "q_win"); _check(k, "k"); _check(row_lse_in, "row_lse_in")
    B, Hq, W, d = q_win.shape
    _, Hkv, N_max, _ = k.shape
    _check_lengths(ctx_len, ctx_len_host, B, N_max, W, causal)
    if row_lse_in.dtype != torch.float32 or tuple(row_lse_in.shape) != (B, Hq, W):
        raise ValueError("row_lse_in must be fp32 [B][Hq][W]")
    if scores is None:
        scores = torch.empty(B, Hkv, N_max, device=k.device, dtype=torch.float32)
    if ctx_len is not None:
        _check(ctx_len, "ctx_len")
    _call("kv_score_from_lse", lib().kv_score_from_lse(
        _ptr(q_win), _ptr(k), _ptr(ctx_len), _ptr(row_lse_in), _ptr(scores),
        B, Hq, Hkv, N_max, W, d, _dtype_code(k), int(bool(causal)), float(scale), _stream()))
    return scores


def kv_score_select_workspace_size(B, Hq, Hkv, N_max, W, d) -> int:
    return int(lib().kv_score_select_workspace_size(B, Hq, Hkv, N_max, W, d))


def kv_score_select(q_win: torch.Tensor, k: torch.Tensor, ctx_len: Optional[torch.Tensor],
                    budget: Budget, *, scale: float = 0.0, causal: bool = False,
                    with_row_lse: bool = False, scores: Optional[torch.Tensor] = None,
                    kept_idx: Optional[torch.Tensor] = None,
                    kept_count: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, ctx_len_host=None):
    """kv_score then kv_select in one call: (scores, row_lse or None, kept_idx, kept_count)."""
    _check(q_win, "q_win"); _check(k, "k")
    B, Hq, W, d = q_win.shape
    _, Hkv, N_max, _ = k.shape
    _check_lengths(ctx_len, ctx_len_host, B, N_max, W, causal)
    dev = k.device
    if scores is None:
        scores = torch.empty(B, Hkv, N_max, device=dev, dtype=torch.float32)
    row_lse = torch.empty(B, Hq, W, device=dev, dtype=torch.float32) if with_row_lse else None
    if kept_idx is None:
        kept_idx = torch.empty(B, Hkv, N_max, device=dev, dtype=torch.int32)
    if kept_count is None:
        kept_count = torch.empty(B * Hkv, device=dev, dtype=torch.int32)
    need = kv_score_select_workspace_size(B, Hq, Hkv, N_max, W, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=dev, dtype=torch.uint8)
    if ctx_len is not None:
        _check(ctx_len, "ctx_len")
    cb = budget.to_c()
    _call("kv_score_select", lib().kv_score_select(
        _ptr(q_win), _ptr(k), _ptr(ctx_len), ctypes.byref(cb), _ptr(scores), _ptr(row_lse),
        _ptr(kept_idx), _ptr(kept_count), B, Hq, Hkv, N_max, W, d, _dtype_code(k),
        int(bool(causal)), float(scale), _ptr(workspace), workspace.numel(), _stream()))
    return scores, row_lse, kept_idx, kept_count


def kv_select(scores: torch.Tensor, ctx_len: Optional[torch.Tensor], budget: Budget, *,
              kept_idx: Optional[torch.Tensor] = None, kept_count: Optional[torch.Tensor] = None):
    """Kept indices [B][Hkv][N_max] int32 (first count valid, ascending) and counts [B*Hkv]."""
    _check(scores, "scores")
    B, Hkv, N_max = scores.shape
    if kept_idx is None:
        kept_idx = torch.empty(B, Hkv, N_max, device=scores.device, dtype=torch.int32)
    if kept_count is None:
        kept_count = torch.empty(B * Hkv, device=scores.device, dtype=torch.int32)
    need = int(lib().kv_select_workspace_size(B, Hkv, N_max))
    ws = torch.empty(need, device=scores.device, dtype=torch.uint8) if need else None
    cb = budget.to_c()
    _call("kv_select", lib().kv_select(
        _ptr(scores), _ptr(ctx_len), B, Hkv, N_max, ctypes.byref(cb),
        _ptr(kept_idx), _ptr(kept_count), _ptr(ws), need, _stream()))
    return kept_idx, kept_count


def kv_compact(k: torch.Tensor, v: torch.Tensor, kept_idx: torch.Tensor,
               kept_count: torch.Tensor, capacity_rows: int, *, out=None):
    """Packed (k_c, v_c, pos, offsets); k_c/v_c [capacity_rows][d] in k's dtype."""
    _check(k, "k"); _check(v, "v")
    B, Hkv, N_max, d = k.shape
    if out is None:
        k_c = torch.empty(capacity_rows, d, device=k.device, dtype=k.dtype)
        v_c = torch.empty(capacity_rows, d, device=k.device, dtype=k.dtype)
        pos = torch.empty(capacity_rows, device=k.device, dtype=torch.int32)
        offsets = torch.empty(B * Hkv + 1, device=k.device, dtype=torch.int64)
    else:
        k_c, v_c, pos, offsets = out
    _call("kv_compact", lib().kv_compact(
        _ptr(k), _ptr(v), B, Hkv, N_max, d, _dtype_code(k), _ptr(kept_idx), _ptr(kept_count),
        _ptr(k_c), _ptr(v_c), _ptr(pos), _ptr(offsets), int(capacity_rows), _stream()))
    return k_c, v_c, pos, offsets


def kv_decode_workspace_size(B, Hq, Hkv, d, capacity_rows) -> int:
    return int(lib().kv_decode_workspace_size(B, Hq, Hkv, d, capacity_rows))


def kv_decode_attn(q: torch.Tensor, k_c: torch.Tensor, v_c: torch.Tensor,
                   offsets: torch.Tensor, Hkv: int, *, scale: float = 0.0,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None):
    """Decode attention (out [B][Hq][d] fp32, lse [B][Hq] fp32) over the packed cache."""
    _check(q, "q"); _check(k_c, "k_c"); _check(v_c, "v_c"); _check(offsets, "offsets")
    B, Hq, d = q.shape
    cap = k_c.shape[0]
    if out is None:
        out = torch.empty(B, Hq, d, device=q.device, dtype=torch.float32)
    if lse is None:
        lse = torch.empty(B, Hq, device=q.device, dtype=torch.float32)
    need = kv_decode_workspace_size(B, Hq, Hkv, d, cap)
    if workspace is None:
        workspace = torch.zeros(max(need, 1), device=q.device, dtype=torch.uint8)
    _call("kv_decode_attn", lib().kv_decode_attn(
        _ptr(q), _ptr(k_c), _ptr(v_c), _ptr(offsets), B, Hq, Hkv, d, _dtype_code(q),
        float(scale), cap, _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream()))
    return out, lse


def kv_decode_attn_noalloc(q: torch.Tensor, k_c: torch.Tensor, v_c: torch.Tensor,
                           offsets: torch.Tensor, Hkv: int, out: torch.Tensor,
                           lse: torch.Tensor, *, scale: float = 0.0):
    """kv_decode_attn with no workspace and no allocation: the caller passes
    out [B][Hq][d] fp32 and lse [B][Hq] fp32; the library's per-GPU scratch
    holds the partials (calls overlapping on one GPU race)."""
    for t, name in ((q, "q"), (k_c, "k_c"), (v_c, "v_c"), (offsets, "offsets"), (out, "out"),
                    (lse, "lse")):
        _check(t, name)
    B, Hq, d = q.shape
    if tuple(out.shape) != (B, Hq, d) or tuple(lse.shape) != (B, Hq) or \
            out.dtype != torch.float32 or lse.dtype != torch.float32:
        raise ValueError("out must be fp32 [B][Hq][d] and lse fp32 [B][Hq]")
    _call("kv_decode_attn_noalloc", lib().kv_decode_attn_noalloc(
        _ptr(q), _ptr(k_c), _ptr(v_c), _ptr(offsets), B, Hq, Hkv, d, _dtype_code(q),
        float(scale), k_c.shape[0], _ptr(out), _ptr(lse), _stream()))
    return out, lse


def kv_compact_decode(k: torch.Tensor, v: torch.Tensor, kept_idx: torch.Tensor,
                      kept_count: torch.Tensor, capacity_rows: int, q: torch.Tensor, *,
                      scale: float = 0.0, out=None, attn_out: Optional[torch.Tensor] = None,
                      lse: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None):
    """kv_compact and kv_decode_attn in one pass: (k_c, v_c, pos, offsets, out, lse)."""
    _check(k, "k"); _check(v, "v"); _check(q, "q")
    if q.dtype != k.dtype or v.dtype != k.dtype:
        raise ValueError("q, k and v must share one dtype")
    B, Hkv, N_max, d = k.shape
    Hq = q.shape[1]
    if out is None:
        k_c = torch.empty(capacity_rows, d, device=k.device, dtype=k.dtype)
        v_c = torch.empty(capacity_rows, d, device=k.device, dtype=k.dtype)
        pos = torch.empty(capacity_rows, device=k.device, dtype=torch.int32)
        offsets = torch.empty(B * Hkv + 1, device=k.device, dtype=torch.int64)
    else:
        k_c, v_c, pos, offsets = out
    if attn_out is None:
        attn_out = torch.empty(B, Hq, d, device=q.device, dtype=torch.float32)
    if lse is None:
        lse = torch.empty(B, Hq, device=q.device, dtype=torch.float32)
    need = kv_decode_workspace_size(B, Hq, Hkv, d, capacity_rows)
    if workspace is None:
        workspace = torch.zeros(max(need, 1), device=q.device, dtype=torch.uint8)
    _call("kv_compact_decode", lib().kv_compact_decode(
        _ptr(k), _ptr(v), _ptr(kept_idx), _ptr(kept_count), B, Hq, Hkv, N_max, d,
        _dtype_code(k), int(capacity_rows), _ptr(q), float(scale), _ptr(k_c), _ptr(v_c),
        _ptr(pos), _ptr(offsets), _ptr(attn_out), _ptr(lse), _ptr(workspace), workspace.numel(),
        _stream()))
    return k_c, v_c, pos, offsets, attn_out, lse


# ---- VECTOR three-way routing ------------------------------------------------

def kv_vector_route(scores: torch.Tensor, ctx_len: Optional[torch.Tensor], k: torch.Tensor,
                    v: torch.Tensor, w: torch.Tensor, *, p_c: float, p_a: float,
                    rope_base: float = 0.0):
    """(pool_idx, pool_count, neg_eps, apx_pos, apx_count); see kv_vector_route in kvcc.h."""
    _check(scores, "scores"); _check(k, "k"); _check(v, "v"); _check(w, "w")
    B, Hkv, N_max, d = k.shape
    if w.dtype != torch.float32 or tuple(w.shape) != (Hkv, d, d):
        raise ValueError("w must be fp32 [Hkv][d][d]")
    dev = k.device
    pool_idx = torch.empty(B, Hkv, N_max, device=dev, dtype=torch.int32)
    pool_count = torch.empty(B * Hkv, device=dev, dtype=torch.int32)
    neg_eps = torch.empty(B, Hkv, N_max, device=dev, dtype=torch.float32)
    apx_pos = torch.empty(B, Hkv, N_max, device=dev, dtype=torch.int32)
    apx_count = torch.empty(B * Hkv, device=dev, dtype=torch.int32)
    need = int(lib().kv_vector_route_workspace_size(B, Hkv))
    ws = torch.empty(max(need, 1), device=dev, dtype=torch.uint8)
    if ctx_len is not None:
        _check(ctx_len, "ctx_len")
    _call("kv_vector_route", lib().kv_vector_route(
        _ptr(scores), _ptr(ctx_len), _ptr(k), _ptr(v), _ptr(w), B, Hkv, N_max, d, _dtype_code(k),
        float(p_c), float(p_a), float(rope_base), _ptr(pool_idx), _ptr(pool_count), _ptr(neg_eps),
        _ptr(apx_pos), _ptr(apx_count), _ptr(ws), ws.numel(), _stream()))
    return pool_idx, pool_count, neg_eps, apx_pos, apx_count


def kv_vector_compact(k: torch.Tensor, v: torch.Tensor, pool_idx: torch.Tensor,
                      pool_count: torch.Tensor, apx_pos: torch.Tensor, apx_count: torch.Tensor,
                      capacity_rows: int, v_capacity_rows: int):
    """(k_c, v_c, pos, vmap, offsets, voffsets) of the routed cache."""
    _check(k, "k"); _check(v, "v")
    B, Hkv, N_max, d = k.shape
    dev = k.device
    k_c = torch.empty(capacity_rows, d, device=dev, dtype=k.dtype)
    v_c = torch.empty(max(v_capacity_rows, 1), d, device=dev, dtype=k.dtype)
    pos = torch.empty(capacity_rows, device=dev, dtype=torch.int32)
    vmap = torch.empty(capacity_rows, device=dev, dtype=torch.int32)
    offsets = torch.empty(B * Hkv + 1, device=dev, dtype=torch.int64)
    voffsets = torch.empty(B * Hkv + 1, device=dev, dtype=torch.int64)
    _call("kv_vector_compact", lib().kv_vector_compact(
        _ptr(k), _ptr(v), B, Hkv, N_max, d, _dtype_code(k), _ptr(pool_idx), _ptr(pool_count),
        _ptr(apx_pos), _ptr(apx_count), _ptr(k_c), _ptr(v_c), _ptr(pos), _ptr(vmap),
        _ptr(offsets), _ptr(voffsets), int(capacity_rows), int(v_capacity_rows), _stream()))
    return k_c, v_c, pos, vmap, offsets, voffsets


def kv_vector_decode(q: torch.Tensor, k_c: torch.Tensor, v_c: torch.Tensor, vmap: torch.Tensor,
                     pos: torch.Tensor, offsets: torch.Tensor, w: torch.Tensor, Hkv: int, *,
                     v_capacity_rows: int, rope_base: float = 0.0, scale: float = 0.0,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None):
    """Decode (out [B][Hq][d] fp32, lse [B][Hq] fp32) over the routed cache."""
    _check(q, "q"); _check(k_c, "k_c"); _check(w, "w")
    B, Hq, d = q.shape
    cap = k_c.shape[0]
    if out is None:
        out = torch.empty(B, Hq, d, device=q.device, dtype=torch.float32)
    if lse is None:
        lse = torch.empty(B, Hq, device=q.device, dtype=torch.float32)
    need = int(lib().kv_vector_decode_workspace_size(B, Hq, Hkv, d, cap))
    if workspace is None:
        workspace = torch.zeros(max(need, 1), device=q.device, dtype=torch.uint8)
    _call("kv_vector_decode", lib().kv_vector_decode(
        _ptr(q), _ptr(k_c), _ptr(v_c), _ptr(vmap), _ptr(pos), _ptr(offsets), _ptr(w),
        float(rope_base), B, Hq, Hkv, d, _dtype_code(q), float(scale), cap, int(v_capacity_rows),
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream()))
    return out, lse
