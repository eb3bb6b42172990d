"""Pure-Python brute force for tiny cases (TEST INFRASTRUCTURE).

A second, independent route to the same quantities as ``oracle.oracle``:
explicit loops, ``math.exp`` and exactly rounded ``math.fsum`` sums, and
selection by pairwise rank counting instead of sorting.  Only the tests use
it, to pin the numpy oracle; sizes must stay tiny (N <= a few hundred).
The definitions followed are the ones stated in ``oracle.oracle``.
"""
from __future__ import annotations

import itertools
import math


def score(q, k, n: int, G: int, scale: float, causal: bool = False):
    """Scores of one KV head.

    q: list over the G query heads of lists of W rows (lists of floats);
    k: list of >= n key rows.  Returns (scores[n], lse[G][W]).
    """
    W = len(q[0])
    logits = []          # one row of n logits (None = hidden) per (j, w)
    for j in range(G):
        for w in range(W):
            row = []
            for t in range(n):
                if causal and t > n - W + w:
                    row.append(None)
                    continue
                row.append(scale * math.fsum(a * b for a, b in zip(q[j][w], k[t])))
            logits.append(row)
    lse = []
    probs = []
    for row in logits:
        vis = [x for x in row if x is not None]
        m = max(vis)
        z = math.fsum(math.exp(x - m) for x in vis)
        l_r = m + math.log(z)
        lse.append(l_r)
        probs.append([0.0 if x is None else math.exp(x - l_r) for x in row])
    scores = [math.fsum(p[t] for p in probs) for t in range(n)]
    return scores, [lse[j * W:(j + 1) * W] for j in range(G)]


def score_from_lse(q, k, n: int, G: int, scale: float, lse, causal: bool = False):
    """Scores of one KV head with given row normalisers lse[G][W]."""
    W = len(q[0])
    out = [0.0] * n
    terms = [[] for _ in range(n)]
    for j in range(G):
        for w in range(W):
            if lse[j][w] == math.inf:
                continue
            for t in range(n):
                if causal and t > n - W + w:
                    continue
                x = scale * math.fsum(a * b for a, b in zip(q[j][w], k[t]))
                terms[t].append(math.exp(x - lse[j][w]))
    for t in range(n):
        out[t] = math.fsum(terms[t])
    return out


def precedes(s, a: int, b: int) -> bool:
    """Token a comes before token b: higher score, or equal score and lower index."""
    return s[a] > s[b] or (s[a] == s[b] and a < b)


def rank(s, t: int) -> int:
    """How many tokens come before t (pairwise counting, no sort)."""
    return sum(1 for u in range(len(s)) if u != t and precedes(s, u, t))


def top_k(s, k: int):
    """Kept set of size k, ascending: the tokens whose rank is below k."""
    return [t for t in range(len(s)) if rank(s, t) < k]


def top_k_by_subsets(s, k: int):
    """For distinct scores: the k-subset with the largest exact score sum."""
    best, best_sum = None, None
    for sub in itertools.combinations(range(len(s)), k):
        tot = math.fsum(s[t] for t in sub)
        if best_sum is None or tot > best_sum:
            best, best_sum = list(sub), tot
    return best


def mass_count(s, f: float) -> int:
    """Fewest k >= 1 whose top-k exact sum reaches f times the exact total."""
    n = len(s)
    order = sorted(range(n), key=lambda t: rank(s, t))
    total = math.fsum(s)
    for k in range(1, n + 1):
        if math.fsum(s[t] for t in order[:k]) >= f * total:
            return k
    return n


def precedes_protected(s, prot, a: int, b: int) -> bool:
    """Protected tokens come first (by index), then the plain order."""
    if prot[a] != prot[b]:
        return prot[a]
    if prot[a]:
        return a < b
    return precedes(s, a, b)


def top_k_protected(s, prot, k: int):
    """Kept set with protected tokens: max(k, #protected) tokens of lowest
    rank under precedes_protected, ascending."""
    n = len(s)
    k = min(n, max(k, sum(1 for x in prot if x)))
    return [t for t in range(n)
            if sum(1 for u in range(n) if u != t and precedes_protected(s, prot, u, t)) < k]


def mass_count_protected(s, prot, f: float) -> int:
    """Fewest k >= 1 whose first-k exact sum (protected first, real scores)
    reaches f times the exact total (before any clamp)."""
    n = len(s)
    rk = {t: sum(1 for u in range(n) if u != t and precedes_protected(s, prot, u, t))
          for t in range(n)}
    order = sorted(range(n), key=lambda t: rk[t])
    total = math.fsum(s)
    for k in range(1, n + 1):
        if math.fsum(s[t] for t in order[:k]) >= f * total:
            return k
    return n


def attend(q, k_rows, v_rows, scale: float):
    """Softmax attention of one query over the given rows: (out, lse)."""
    u = [scale * math.fsum(a * b for a, b in zip(q, kr)) for kr in k_rows]
    m = max(u)
    e = [math.exp(x - m) for x in u]
    z = math.fsum(e)
    d = len(v_rows[0])
    out = [math.fsum(e[i] * v_rows[i][c] for i in range(len(e))) / z for c in range(d)]
    return out, m + math.log(z)


def rope_rotate(x, pos: int, base: float, sign: float):
    """Rotate adjacent pairs (2i, 2i+1) of a list by sign * pos * base^(-2i/d)."""
    d = len(x)
    out = list(x)
    if base == 0.0:
        return out
    for i in range(d // 2):
        a = sign * pos * base ** (-2.0 * i / d)
        c, s_ = math.cos(a), math.sin(a)
        out[2 * i] = x[2 * i] * c - x[2 * i + 1] * s_
        out[2 * i + 1] = x[2 * i] * s_ + x[2 * i + 1] * c
    return out


def residual(v_row, k_row, w, pos: int, base: float):
    """||v - w * rotate(k, -pos)||^2 with explicit loops (w: list of rows)."""
    kr = rope_rotate(k_row, pos, base, -1.0)
    d = len(v_row)
    terms = []
    for o in range(d):
        rec = math.fsum(w[o][i] * kr[i] for i in range(d))
        terms.append((v_row[o] - rec) ** 2)
    return math.fsum(terms)
