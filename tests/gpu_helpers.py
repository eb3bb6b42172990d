"""Shared checks for the GPU parity tests (HIP path vs the float64 oracle).

Tolerances:
* scores: relative 2e-3 where the oracle score is at least 2^-92 * W * G;
  below that floor the GPU value only has to stay below it (fp32 exp2 terms
  underflow near 2^-126, and a score that small is irrelevant to selection);
* kept sets, stage by stage: identical (the oracle selects on the GPU's own
  fp32 scores); end to end: they may differ only on tokens whose oracle score
  lies within 1e-5 relative of the k-th oracle score (plus the same floor);
* gathered K/V, positions, counts and offsets: bit-exact;
* decode: out within 1e-2 absolute, lse within 1e-3 absolute;
* mass-budget counts: a GPU count may differ from the oracle's only if it
  brackets f * C(n) to within a band on exact sums (``mass_count_ok``).
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from fractions import Fraction

from oracle import oracle as orc

FLOOR = 2.0 ** -92
SCORE_RTOL = 2e-3
BAND_RTOL = 1e-5


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().cuda()


def check_scores(s_gpu, s_ref, ctx, W, G, rtol=SCORE_RTOL) -> float:
    """Assert the score tolerance over every valid token; return max rel err."""
    s_gpu = np.asarray(s_gpu, dtype=np.float64)
    floor = FLOOR * W * G
    worst = 0.0
    B, Hkv = s_ref.shape[:2]
    for b in range(B):
        n = int(ctx[b])
        for h in range(Hkv):
            g, r = s_gpu[b, h, :n], s_ref[b, h, :n]
            assert np.all(np.isfinite(g)), f"non-finite score at b={b} h={h}"
            big = r >= floor
            if np.any(big):
                rel = np.abs(g[big] - r[big]) / r[big]
                worst = max(worst, float(rel.max()))
                assert rel.max() <= rtol, (b, h, int(np.argmax(rel)), float(rel.max()))
            assert np.all(g[~big] <= floor * (1 + rtol)), (b, h)
    return worst


def kth_oracle_score(s_ref_head, k):
    order = orc.total_order(s_ref_head)
    return float(s_ref_head[order[k - 1]])


def check_band(kept_gpu, cnt_gpu, s_ref, ctx, W, G, k_ref=None) -> int:
    """End-to-end kept sets (A20 ii); returns the number of in-band differences."""
    B, Hkv = s_ref.shape[:2]
    floor = FLOOR * W * G
    diffs = 0
    for b in range(B):
        n = int(ctx[b])
        for h in range(Hkv):
            i = b * Hkv + h
            k = int(cnt_gpu[i])
            if k_ref is not None:
                assert k == int(k_ref[i]), (b, h, k, int(k_ref[i]))
            s = s_ref[b, h, :n]
            ref_set = set(orc.total_order(s)[:k].tolist())
            got = kept_gpu[b, h, :k]
            assert np.all(np.diff(got) > 0) and got.min() >= 0 and got.max() < n
            gpu_set = set(got.tolist())
            sym = ref_set ^ gpu_set
            if sym:
                sk = kth_oracle_score(s, k)
                for t in sym:
                    assert abs(s[t] - sk) <= BAND_RTOL * sk + floor, \
                        (b, h, t, float(s[t]), sk)
                diffs += len(sym)
    return diffs


def check_decode(out_g, lse_g, out_r, lse_r, atol_out=1e-2, atol_lse=1e-3):
    out_g = np.asarray(out_g, np.float64)
    lse_g = np.asarray(lse_g, np.float64)
    e_out = float(np.max(np.abs(out_g - out_r))) if out_r.size else 0.0
    fin = np.isfinite(lse_r)
    assert np.array_equal(fin, np.isfinite(lse_g))
    e_lse = float(np.max(np.abs(lse_g[fin] - lse_r[fin]))) if fin.any() else 0.0
    assert e_out <= atol_out, e_out
    assert e_lse <= atol_lse, e_lse
    return e_out, e_lse


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw element bits of a CPU tensor (bf16 -> int16, fp32 -> int32)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    return t.numpy()


def ratio_k(n: int, r: float) -> int:
    return min(max(int(math.floor(float(np.float32(r)) * n + 0.5)), 1), n)


# The mass budget's count band, relative to the head's total C(n).  The GPU
# sums scores in 64-bit fixed point at 2^(61 - floor(log2 C(n))): each score
# is truncated by less than 2^-61 C(n), so its C(k) falls short of the exact
# sum by less than k 2^-61 C(n), and its target ceil(f * total) (double
# products) is off by less than 2^-51 C(n).  Its count therefore brackets
# f * C(n) on exact sums to within (2 n 2^-61 + 2^-50) C(n) < 1.2e-13 C(n)
# for n <= 2^17; 1e-12 covers that.
MASS_BAND = 1e-12


def mass_count_range(s_head, f, lo, hi, band, prot=None):
    """The counts a mass budget may return for one head when C(k) is known to
    within band * C(n): every clamp of a k with C(k) >= f C(n) - band C(n) and
    C(k - 1) < f C(n) + band C(n), C the exact prefix sums of the scores in
    the total order (protected tokens first).  Returns (k_min, k_max); the
    clamp of a monotone interval is the interval of the clamped ends."""
    s_head = np.asarray(s_head, dtype=np.float64)
    n = len(s_head)
    c = orc.exact_prefix_sums(s_head[orc.total_order(s_head, prot)])
    total = Fraction(c[-1])
    target = Fraction(float(np.float32(f))) * total
    slack = Fraction(band) * total
    k_a = next(k for k in range(1, n + 1) if c[k - 1] >= target - slack)
    k_b = max(k for k in range(1, n + 1) if k == 1 or c[k - 2] < target + slack)
    n_prot = 0 if prot is None else int(np.count_nonzero(prot))
    k_lo = max(1, int(np.floor(np.float32(lo) * n + 0.5)))
    k_hi = min(n, max(1, int(np.floor(np.float32(hi) * n + 0.5))))
    k_lo = min(k_lo, k_hi)
    clamp = lambda k: min(max(min(max(k, k_lo), k_hi), n_prot), n)
    return clamp(k_a), clamp(k_b)


def mass_count_ok(s_head, k_g, f, lo, hi, band=MASS_BAND, prot=None):
    k_min, k_max = mass_count_range(s_head, f, lo, hi, band, prot)
    return k_min <= k_g <= k_max


def mass_between(s_head, k1, k2, prot=None):
    """Exact score mass of the tokens ranked between two counts, relative to
    the head's total."""
    s_head = np.asarray(s_head, dtype=np.float64)
    c = orc.exact_prefix_sums(s_head[orc.total_order(s_head, prot)])
    a, b = sorted((k1, k2))
    if a == b or c[-1] == 0:
        return 0.0
    return float(Fraction(c[b - 1] - (c[a - 1] if a > 0 else 0), c[-1]))
