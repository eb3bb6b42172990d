"""Float64 CPU oracle for the score -> select -> compact -> decode path.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP
library or its Python binding and imports nothing from them; the product path
never calls it.

Every function is the plain definition written out in numpy float64, one
(sequence, KV head) at a time, with library primitives (a matmul, exp, a
stable sort, a cumulative sum) as its steps and no blocking or fusion.

What the pages fix and what this module reads into them
-------------------------------------------------------
* "A Simple Plug-in for Improving Eviction-Based KV Cache Compression"
  (VECTOR), section "Enonce du Probleme": importance-based eviction (SnapKV,
  KeyDiff) scores the cached tokens and permanently drops the low scorers.
  The pages name SnapKV's query-aware attention score but never write it out;
  the score taken here is the observation-window attention score: the last W
  queries of each query head attend (softmax over every cached key of the
  sequence) and each token's probabilities are summed over the W window rows
  and over the query heads of its KV head's GQA group.
* "KVSculpt: KV Cache Compression as Distillation", section 2.B: the
  log-sum-exp ell of the attention logits is the per-row normaliser this
  score divides by; ``window_scores`` also returns it.
* "KVzap: Fast, Adaptive, and Faithful KV Cache Pruning", section 2.3
  ("Seuillage"): tokens whose score falls below a fixed threshold tau are
  dropped, so the kept fraction adapts to the input; here a score equal to
  tau is kept.
* "KV Cache Transform Coding for Compact Storage in LLM Inference", section
  3, and the KVzap page, section 1: the edited cache keeps the plain K/V
  layout that a standard attention kernel reads, so the compacted cache is a
  dense packed subset of rows in original order, and decode is ordinary
  softmax attention over it.

Readings where the pages are silent (each also listed in the design notes):
softmax scale 1/sqrt(d) applied after the dot product; scores summed (not
averaged) over the GQA group, so they total W*G per KV head; query head j
belongs to KV head j // G; window row w of a sequence of length n sits at
position n - W + w, and ``causal=True`` hides tokens after it (default off:
every window row sees every key); ties in score go to the lower token index
and -0.0 equals +0.0; ratio budgets keep clamp(floor(r*n + 1/2), 1, n)
tokens with r widened from fp32; the mass budget keeps the fewest top tokens
whose summed score reaches f times the head's total; decode is one fresh
query per query head over the compacted rows only.
"""
from __future__ import annotations

import math

import numpy as np

BUDGET_K = 0
BUDGET_RATIO = 1
BUDGET_THRESHOLD = 2
BUDGET_MASS = 3


def _f64(x) -> np.ndarray:
    """Widen a numpy array or CPU torch tensor (fp32/bf16) exactly to float64."""
    if hasattr(x, "detach"):
        t = x.detach().cpu()
        if t.is_floating_point():
            t = t.double()
        return t.numpy()
    return np.asarray(x, dtype=np.float64)


def _ints(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x, dtype=np.int64)


def _ctx(ctx_len, B: int, N_max: int) -> np.ndarray:
    if ctx_len is None:
        return np.full(B, N_max, dtype=np.int64)
    return _ints(ctx_len)


def _scale(scale, d: int) -> float:
    return 1.0 / math.sqrt(d) if scale is None or scale <= 0 else float(np.float32(scale))


def window_scores(q_win, k, ctx_len=None, scale=None, causal=False):
    """Observation-window scores and row log-sum-exps.

    q_win [B][Hq][W][d], k [B][Hkv][N_max][d], ctx_len [B] (None: all N_max).
    Returns ``(scores, lse)``: scores [B][Hkv][N_max] float64 with entries at
    t >= ctx_len[b] left at 0, and lse [B][Hq][W] float64 (natural log).

    For row r = (query head j, window row w) of KV head h = j // G:
      l[r, t]  = scale * <q[r], k[t]>              (t < n; causal hides t > n-W+w)
      lse[r]   = m + log(sum_t exp(l[r, t] - m)),  m = max_t l[r, t]
      s[h, t]  = sum_r exp(l[r, t] - lse[r])
    """
    q = _f64(q_win)
    kk = _f64(k)
    B, Hq, W, d = q.shape
    _, Hkv, N_max, _ = kk.shape
    G = Hq // Hkv
    sc = _scale(scale, d)
    ctx = _ctx(ctx_len, B, N_max)
    scores = np.zeros((B, Hkv, N_max), dtype=np.float64)
    lse = np.zeros((B, Hq, W), dtype=np.float64)
    for b in range(B):
        n = int(ctx[b])
        for h in range(Hkv):
            rows = q[b, h * G:(h + 1) * G].reshape(G * W, d)
            logits = sc * (rows @ kk[b, h, :n].T)               # [G*W, n]
            if causal:
                w_of_row = np.tile(np.arange(W), G)
                last = n - W + w_of_row                           # last visible token per row
                hidden = np.arange(n)[None, :] > last[:, None]
                logits[hidden] = -np.inf
            m = logits.max(axis=1, keepdims=True)
            row_lse = m + np.log(np.exp(logits - m).sum(axis=1, keepdims=True))
            p = np.exp(logits - row_lse)
            scores[b, h, :n] = p.sum(axis=0)
            lse[b, h * G:(h + 1) * G] = row_lse.reshape(G, W)
    return scores, lse


def window_scores_from_lse(q_win, k, row_lse, ctx_len=None, scale=None, causal=False):
    """Window scores with the row normalisers given instead of computed.

    A prefill attention pass already yields each window row's log-sum-exp
    ell ("KVSculpt: KV Cache Compression as Distillation", section 2.B), and
    pruning runs after that attention op ("KVzap: Fast, Adaptive, and
    Faithful KV Cache Pruning", section 2.3).  With row_lse [B][Hq][W]
    (natural log) supplied:
      s[h, t] = sum_r exp(l[r, t] - row_lse[r])
    with l and the causal rule as in ``window_scores``.  A row whose row_lse
    is +inf adds nothing.  Returns scores [B][Hkv][N_max] float64.
    """
    q = _f64(q_win)
    kk = _f64(k)
    given = _f64(row_lse)
    B, Hq, W, d = q.shape
    _, Hkv, N_max, _ = kk.shape
    G = Hq // Hkv
    sc = _scale(scale, d)
    ctx = _ctx(ctx_len, B, N_max)
    scores = np.zeros((B, Hkv, N_max), dtype=np.float64)
    for b in range(B):
        n = int(ctx[b])
        for h in range(Hkv):
            rows = q[b, h * G:(h + 1) * G].reshape(G * W, d)
            logits = sc * (rows @ kk[b, h, :n].T)               # [G*W, n]
            if causal:
                w_of_row = np.tile(np.arange(W), G)
                hidden = np.arange(n)[None, :] > (n - W + w_of_row)[:, None]
                logits[hidden] = -np.inf
            norm = given[b, h * G:(h + 1) * G].reshape(G * W, 1)
            with np.errstate(invalid="ignore"):
                p = np.exp(logits - norm)
            p[np.isinf(norm[:, 0])] = 0.0
            scores[b, h, :n] = p.sum(axis=0)
    return scores


def protected_mask(n: int, n_sink: int = 0, n_recent: int = 0) -> np.ndarray:
    """Tokens a head always keeps: the first n_sink (attention sinks) and the
    last n_recent (the recent window).  "KVzap: Fast, Adaptive, and Faithful
    KV Cache Pruning", section 2.3, keeps a sliding window of recent tokens
    whatever their score; "KV Cache Transform Coding for Compact Storage in
    LLM Inference", section 3, leaves the first tokens (attention sinks) and
    the most recent ones uncompressed."""
    p = np.zeros(n, dtype=bool)
    p[:max(0, min(int(n_sink), n))] = True
    if n_recent > 0:
        p[max(0, n - int(n_recent)):] = True
    return p


def total_order(s: np.ndarray, protected=None) -> np.ndarray:
    """Token indices of one head from first to last: protected tokens first
    (by index), then higher score first, equal scores by lower index (-0.0
    and +0.0 compare equal)."""
    s = np.asarray(s, dtype=np.float64)
    idx = np.arange(s.shape[0])
    if protected is None or not np.any(protected):
        return np.lexsort((idx, -s))
    p = np.asarray(protected, dtype=bool)
    return np.lexsort((idx, np.where(p, 0.0, -s), (~p).astype(np.int8)))


def exact_prefix_sums(values):
    """Exact prefix sums of float values, as Python integers in units of
    2^-1074 (every finite double is an integer multiple of it), so the
    mass budget's C(k) is the true sum of the first k scores with no
    rounding at all."""
    out = []
    acc = 0
    for x in np.asarray(values, dtype=np.float64).tolist():
        num, den = x.as_integer_ratio()            # den = 2^m, m <= 1074
        acc += num << (1074 - den.bit_length() + 1)
        out.append(acc)
    return out


def mass_count(s_ordered, f: float) -> int:
    """Fewest k >= 1 with C(k) >= f * C(n), C(k) the exact sum of the first k
    entries of s_ordered and f the fp32 fraction (an exact dyadic rational);
    n when no shorter prefix reaches it."""
    c = exact_prefix_sums(s_ordered)
    num, den = float(np.float32(f)).as_integer_ratio()
    target = num * c[-1]                           # compare C(k) * den >= num * C(n)
    for k, ck in enumerate(c, start=1):
        if ck * den >= target:
            return k
    return len(c)


def _round_half_up(x: float) -> int:
    return int(math.floor(x + 0.5))


def _clamp_bounds(n: int, min_ratio: float, max_ratio: float):
    lo = max(1, _round_half_up(float(np.float32(min_ratio)) * n))
    hi = min(n, max(1, _round_half_up(float(np.float32(max_ratio)) * n)))
    return min(lo, hi), hi


def budget_count(s, mode: int, *, k=None, ratio=None, tau=None, mass=None,
                 min_ratio: float = 0.0, max_ratio: float = 1.0, protected=None) -> int:
    """Number of tokens one head keeps, from its n scores ``s``.

    BUDGET_K:         clamp(k, 1, n)
    BUDGET_RATIO:     clamp(floor(r*n + 1/2), 1, n), r the fp32 ratio widened
    BUDGET_THRESHOLD: #{t : t protected or s_t >= tau}, tau fp32, then clamped
                      to [max(1, round(min_ratio*n)), round(max_ratio*n)]
    BUDGET_MASS:      fewest k >= 1 whose first-k score sum C(k) in the
                      total order (protected tokens first, with their real
                      scores) reaches f*C(n) (f fp32; sums and the comparison
                      exact, see ``mass_count``), then the same clamp as the
                      threshold mode
    Protected tokens count toward k and are always kept: the result is at
    least their number.
    """
    s = np.asarray(s, dtype=np.float64)
    n = s.shape[0]
    if n == 0:
        return 0
    p = np.zeros(n, dtype=bool) if protected is None else np.asarray(protected, dtype=bool)
    n_prot = int(np.count_nonzero(p))
    if mode == BUDGET_K:
        kk = min(max(int(k), 1), n)
    elif mode == BUDGET_RATIO:
        r = float(np.float32(ratio))
        kk = min(max(int(math.floor(r * n + 0.5)), 1), n)
    elif mode == BUDGET_THRESHOLD:
        lo, hi = _clamp_bounds(n, min_ratio, max_ratio)
        t = float(np.float32(tau))
        cnt = int(np.count_nonzero(p | (s >= t)))
        kk = min(max(cnt, lo), hi)
    elif mode == BUDGET_MASS:
        lo, hi = _clamp_bounds(n, min_ratio, max_ratio)
        kk = mass_count(s[total_order(s, p)], mass)
        kk = min(max(kk, lo), hi)
    else:
        raise ValueError(f"unknown budget mode {mode}")
    return int(min(max(kk, n_prot), n))


def select(scores, ctx_len=None, mode=BUDGET_RATIO, n_sink: int = 0, n_recent: int = 0,
           **params):
    """Per-head kept token indices.

    scores [B][Hkv][N_max]; params as ``budget_count`` (``k``/``ratio`` may
    also be per-head arrays of length B*Hkv); n_sink / n_recent protect the
    first / last tokens of every head (``protected_mask``).  Returns
    ``(kept_idx, count)``: kept_idx [B][Hkv][N_max] int32 (first count entries
    valid, ascending, the rest -1) and count [B*Hkv] int32.  The kept set of a
    head is the first count tokens of ``total_order``.
    """
    s_all = _f64(scores)
    B, Hkv, N_max = s_all.shape
    ctx = _ctx(ctx_len, B, N_max)
    kept = np.full((B, Hkv, N_max), -1, dtype=np.int32)
    count = np.zeros(B * Hkv, dtype=np.int32)
    for b in range(B):
        n = int(ctx[b])
        for h in range(Hkv):
            i = b * Hkv + h
            p = dict(params)
            for key in ("k", "ratio"):
                if key in p and p[key] is not None and np.ndim(p[key]) > 0:
                    p[key] = np.asarray(p[key]).reshape(-1)[i]
            s = s_all[b, h, :n]
            prot = protected_mask(n, n_sink, n_recent)
            kk = budget_count(s, mode, protected=prot, **p)
            idx = np.sort(total_order(s, prot)[:kk])
            kept[b, h, :kk] = idx
            count[i] = kk
    return kept, count


def compact(k, v, kept_idx, count):
    """Gather the kept rows of every head into one packed cache.

    Heads are laid out (sequence, KV head) row-major; offsets [B*Hkv+1] int64
    is the exclusive prefix sum of count.  Returns numpy arrays
    ``(k_c [total][d], v_c [total][d], pos [total] int32, offsets)`` with
    k_c/v_c in the input's own element type, so equality is bitwise.
    """
    if hasattr(k, "detach"):
        import torch  # only to keep bf16 bytes intact
        kn = k.detach().cpu().view(torch.int16).numpy() if k.dtype == torch.bfloat16 \
            else k.detach().cpu().numpy()
        vn = v.detach().cpu().view(torch.int16).numpy() if v.dtype == torch.bfloat16 \
            else v.detach().cpu().numpy()
    else:
        kn, vn = np.asarray(k), np.asarray(v)
    idx = _ints(kept_idx)
    cnt = _ints(count)
    B, Hkv = kn.shape[0], kn.shape[1]
    offsets = np.zeros(B * Hkv + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(cnt)
    kc, vc, pos = [], [], []
    for b in range(B):
        for h in range(Hkv):
            c = int(cnt[b * Hkv + h])
            sel = idx[b, h, :c]
            kc.append(kn[b, h, sel])
            vc.append(vn[b, h, sel])
            pos.append(sel.astype(np.int32))
    d = kn.shape[-1]
    k_c = np.concatenate(kc) if kc else np.zeros((0, d), kn.dtype)
    v_c = np.concatenate(vc) if vc else np.zeros((0, d), vn.dtype)
    return k_c, v_c, np.concatenate(pos), offsets


def decode(q, k_c, v_c, offsets, Hkv: int, scale=None):
    """One decode query per query head over the compacted cache.

    q [B][Hq][d]; k_c, v_c [total][d] (float arrays or bf16 tensors);
    offsets [B*Hkv+1].  For query head j of KV head h = j // G with rows
    o..o+k-1:  u_i = scale*<q, K_c[o+i]>,  out = sum_i softmax(u)_i V_c[o+i],
    lse = m + log(sum_i exp(u_i - m)).  A head with no rows has an empty sum:
    lse = log 0 = -inf, and its output is taken as 0.
    Returns (out [B][Hq][d], lse [B][Hq]).
    """
    qq = _f64(q)
    kc = _f64(k_c)
    vc = _f64(v_c)
    off = _ints(offsets)
    B, Hq, d = qq.shape
    G = Hq // Hkv
    sc = _scale(scale, d)
    out = np.zeros((B, Hq, d), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    for b in range(B):
        for j in range(Hq):
            h = j // G
            lo, hi = int(off[b * Hkv + h]), int(off[b * Hkv + h + 1])
            if hi <= lo:
                lse[b, j] = -math.inf
                continue
            u = sc * (kc[lo:hi] @ qq[b, j])
            m = u.max()
            e = np.exp(u - m)
            z = e.sum()
            out[b, j] = (e @ vc[lo:hi]) / z
            lse[b, j] = m + math.log(z)
    return out, lse


def attend_full(q, k, v, ctx_len=None, scale=None):
    """Decode over the whole (uncompressed) cache: the 100%-keep reference."""
    kk = _f64(k)
    vv = _f64(v)
    B, Hkv, N_max, d = kk.shape
    ctx = _ctx(ctx_len, B, N_max)
    rows_k, rows_v = [], []
    offsets = np.zeros(B * Hkv + 1, dtype=np.int64)
    i = 0
    for b in range(B):
        for h in range(Hkv):
            n = int(ctx[b])
            rows_k.append(kk[b, h, :n])
            rows_v.append(vv[b, h, :n])
            offsets[i + 1] = offsets[i] + n
            i += 1
    return decode(q, np.concatenate(rows_k), np.concatenate(rows_v), offsets, Hkv, scale)


def fidelity(q, k, v, kept_idx, count, ctx_len=None, scale=None):
    """Loss terms of "KVSculpt: KV Cache Compression as Distillation", section
    2.B, for a compacted cache against the full one, over decode queries q
    [B][Hq][d]: with Y, ell the attention output and log-sum-exp over the full
    cache and Y^, ell^ over the kept rows,
      out_err2[b, j] = ||Y^ - Y||^2,  lse_diff[b, j] = ell^ - ell,
      loss = sum out_err2 + sum lse_diff^2   (the Frobenius norms squared).
    Returns a dict of those plus out_norm2 = ||Y||^2.
    """
    kk = _f64(k)
    vv = _f64(v)
    idx = _ints(kept_idx)
    cnt = _ints(count)
    B, Hkv = kk.shape[0], kk.shape[1]
    rows_k, rows_v = [], []
    offsets = np.zeros(B * Hkv + 1, dtype=np.int64)
    for b in range(B):
        for h in range(Hkv):
            i = b * Hkv + h
            sel = idx[b, h, :int(cnt[i])]
            rows_k.append(kk[b, h, sel])
            rows_v.append(vv[b, h, sel])
            offsets[i + 1] = offsets[i] + len(sel)
    y_hat, l_hat = decode(q, np.concatenate(rows_k), np.concatenate(rows_v), offsets, Hkv, scale)
    y, ell = attend_full(q, k, v, ctx_len, scale)
    err2 = ((y_hat - y) ** 2).sum(axis=-1)
    dl = l_hat - ell
    return {"out_err2": err2, "out_norm2": (y ** 2).sum(axis=-1), "lse_diff": dl,
            "loss": float(err2.sum() + (dl ** 2).sum())}


# ---- VECTOR three-way routing ----------------------------------------------
#
# "A Simple Plug-in for Improving Eviction-Based KV Cache Compression"
# (VECTOR), section "Methodologie: VECTOR" / "Pipeline d'Allocation en Trois
# Voies": for a target removed fraction p_c and an approximated fraction p_a,
# the base eviction score picks an enlarged pool of 1 - p_c + p_a of the
# tokens; each pool token's reconstruction residual eps = ||V - W RoPE^-1(K)||^2
# is computed with an offline linear map W (keys rotated back to position 0
# first); keys are kept for the whole pool, the 2 p_a lowest-residual tokens
# drop their values (rebuilt as W RoPE^-1(K) on use), and the remaining
# 1 - p_c - p_a keep exact K and V.  Readings: counts are
# k_pool = clamp(floor((1 - p_c + p_a) n + 1/2), 1, n) and
# k_apx = min(k_pool, floor(2 p_a n + 1/2)) (p_c, p_a fp32, arithmetic in
# float64); rotary position encoding rotates adjacent pairs (2i, 2i+1) by
# pos * base^(-2i/d) (base = 0: no rotation); ties in eps go to the lower
# token index.

def rope_inverse(x, pos, base: float):
    """Rotate each adjacent pair (2i, 2i+1) of rows x [m][d] back by
    pos[m] * base^(-2i/d) (the inverse of rotary position encoding)."""
    x = _f64(x)
    if base == 0.0:
        return x.copy()
    m, d = x.shape
    i = np.arange(d // 2, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * base ** (-2.0 * i / d)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[:, 0::2], x[:, 1::2]
    out = np.empty_like(x)
    out[:, 0::2] = xe * c + xo * s
    out[:, 1::2] = -xe * s + xo * c
    return out


def vector_counts(n: int, p_c: float, p_a: float):
    """(k_pool, k_apx) of a head with n tokens."""
    pc, pa = float(np.float32(p_c)), float(np.float32(p_a))
    k_pool = int(min(max(math.floor((1.0 - pc + pa) * n + 0.5), 1), n))
    k_apx = int(min(k_pool, math.floor(2.0 * pa * n + 0.5)))
    return k_pool, k_apx


def vector_residuals(k, v, w, pool_idx, pool_count, rope_base: float = 0.0):
    """eps[b][h][j] = ||V_t - W_h RoPE^-1(K_t)||^2 for pool entry j (token
    t = pool_idx[b,h,j], position t), +inf beyond the pool.  w [Hkv][d][d]
    maps a de-rotated key to a value (out = w @ in)."""
    kk, vv, ww = _f64(k), _f64(v), _f64(w)
    idx, cnt = _ints(pool_idx), _ints(pool_count)
    B, Hkv, N_max, d = kk.shape
    eps = np.full((B, Hkv, N_max), np.inf)
    for b in range(B):
        for h in range(Hkv):
            c = int(cnt[b * Hkv + h])
            t = idx[b, h, :c]
            kt = rope_inverse(kk[b, h, t], t, rope_base)
            r = vv[b, h, t] - kt @ ww[h].T
            eps[b, h, :c] = (r * r).sum(axis=1)
    return eps


def vector_route(scores, k, v, w, ctx_len=None, p_c: float = 0.9, p_a: float = 0.05,
                 rope_base: float = 0.0):
    """Pool, residuals and the approximated subset of every head.

    Returns (pool_idx, pool_count, eps, apx) with pool_idx/pool_count as
    ``select`` at the pool ratio, eps as ``vector_residuals`` and apx
    [B][Hkv][N_max] bool: True for the pool entries whose value is dropped.
    """
    s_all = _f64(scores)
    B, Hkv, N_max = s_all.shape
    ctx = _ctx(ctx_len, B, N_max)
    kp = np.array([vector_counts(int(ctx[b]), p_c, p_a)[0] for b in range(B)
                   for _ in range(Hkv)], dtype=np.int64)
    pool_idx, pool_count = select(s_all, ctx, BUDGET_K, k=kp)
    eps = vector_residuals(k, v, w, pool_idx, pool_count, rope_base)
    apx = np.zeros((B, Hkv, N_max), dtype=bool)
    for b in range(B):
        ka = vector_counts(int(ctx[b]), p_c, p_a)[1]
        for h in range(Hkv):
            c = int(pool_count[b * Hkv + h])
            # lowest residual first, lower token index (= lower pool entry) on ties
            order = np.lexsort((np.arange(c), eps[b, h, :c]))
            apx[b, h, order[:ka]] = True
    return pool_idx, pool_count, eps, apx


def vector_decode(q, k, v, w, pool_idx, pool_count, apx, Hkv: int, rope_base: float = 0.0,
                  scale=None):
    """Decode over the routed cache: every pool row's key, its exact value or,
    for approximated entries, W RoPE^-1(K).  Returns (out, lse) as ``decode``."""
    kk, vv, ww = _f64(k), _f64(v), _f64(w)
    idx, cnt = _ints(pool_idx), _ints(pool_count)
    B = kk.shape[0]
    rows_k, rows_v = [], []
    offsets = np.zeros(B * Hkv + 1, dtype=np.int64)
    for b in range(B):
        for h in range(Hkv):
            i = b * Hkv + h
            c = int(cnt[i])
            t = idx[b, h, :c]
            val = vv[b, h, t].copy()
            a = np.asarray(apx[b, h, :c], dtype=bool)
            if a.any():
                val[a] = rope_inverse(kk[b, h, t[a]], t[a], rope_base) @ ww[h].T
            rows_k.append(kk[b, h, t])
            rows_v.append(val)
            offsets[i + 1] = offsets[i] + c
    return decode(q, np.concatenate(rows_k), np.concatenate(rows_v), offsets, Hkv, scale)
