"""Brute-force replay of H2O eviction, written independently of the oracle.

Pure Python, positions kept in a set, every attention row stored as a
{position: probability} dict, and every score recomputed from scratch (sum over
all stored rows) whenever a decision is taken. It follows the same readings of
the pages as the oracle but shares no code with it:

  * H2O blog (ttsmallhot.github.io), §2.2: budget k = k_heavy + k_local; the
    running score of a token is the sum of the attention it received; the
    lowest-scoring token outside the recent tokens is dropped.
  * "H2O Heavy-Hitter Oracle 分析", §3.2: victim = argmin of the score; the new
    token always joins.

Where the oracle picks the prompt's heavy hitters with one sort (top-k), this
replay shrinks the prompt cache by repeatedly removing the (score, position)
minimum outside the window, a different route to the same set.

With `uniform=True` every query is taken as zero, so each row is exactly uniform
and all arithmetic is done in `fractions.Fraction` (exact).
"""
from __future__ import annotations

import math
from fractions import Fraction


def _softmax_row(qi, K, keys, d, uniform):
    if uniform:
        w = Fraction(1, len(keys))
        return {j: w for j in keys}
    logits = [sum(a * b for a, b in zip(qi, K[j])) / math.sqrt(d) for j in keys]
    m = max(logits)
    e = [math.exp(x - m) for x in logits]
    s = sum(e)
    return {j: x / s for j, x in zip(keys, e)}


def replay(Q, K, V, T, k_heavy, k_local, uniform=False):
    """Q, K, V: lists of length N (positions 0..N-1) of d-vectors.

    Positions 0..T-1 are the prompt, T..N-1 the decoded tokens.
    Returns dict with: outs (list of d-vectors, one per decode step), kept
    (sorted final kept positions), prefill_kept, victims (list of (t, pos)),
    scores (position -> final score), gaps (relative gap between the two lowest
    candidates at each decode decision).
    """
    N = len(K)
    d = len(K[0]) if N else 0
    k = k_heavy + k_local
    rows = []

    def score(p):
        return sum(r.get(p, 0) for r in rows)

    for i in range(T):
        rows.append(_softmax_row(Q[i], K, list(range(i + 1)), d, uniform))
    cache = set(range(T))
    while len(cache) > k:
        cand = [p for p in cache if p < T - k_local]
        cache.remove(min(cand, key=lambda p: (score(p), p)))
    prefill_kept = sorted(cache)

    outs, victims, gaps = [], [], []
    for t in range(T, N):
        keys = sorted(cache) + [t]
        row = _softmax_row(Q[t], K, keys, d, uniform)
        rows.append(row)
        outs.append([sum(row[j] * V[j][c] for j in keys) for c in range(d)])
        cache.add(t)
        if len(cache) > k:
            cand = sorted((score(p), p) for p in cache if p <= t - k_local)
            victim = cand[0][1]
            if len(cand) > 1:
                a, b = cand[0][0], cand[1][0]
                gaps.append(float(abs(b - a)) / max(float(abs(a)), float(abs(b)), 1e-300))
            cache.remove(victim)
            victims.append((t, victim))
    scores = {p: score(p) for p in range(N)}
    return {"outs": outs, "kept": sorted(cache), "prefill_kept": prefill_kept,
            "victims": victims, "scores": scores, "gaps": gaps}
