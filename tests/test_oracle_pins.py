"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these checks retypes the oracle's formulas: they use a library routine
(float64 scaled_dot_product_attention), closed forms (harmonic numbers, uniform
means, exact fractions), invariants of the method (the Full and Local baselines
of the H2O blog §3.1.1; conservation of attention mass) and an independent
brute-force replay.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import (UnitCache, ParityError, adopt_prefill_kept, decode, prefill, run_unit,
                    seed_positions)
from tests.bruteforce import replay


def rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def sdpa64(Q, K, V):
    """Full causal attention via torch's own routine, float64 on the CPU."""
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x))[None, None] for x in (Q, K, V))
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)[0, 0].numpy()


def harmonic(n):
    return sum((Fraction(1, i) for i in range(1, n + 1)), Fraction(0))


# ---------------------------------------------------------------- prefill -------

@pytest.mark.parametrize("T,d", [(1, 4), (37, 16), (128, 64)])
def test_prefill_output_matches_library_sdpa(T, d):
    rng = np.random.default_rng(T * 7 + d)
    Q, K, V = rand(rng, T, d, scale=1.5), rand(rng, T, d, scale=1.5), rand(rng, T, d)
    O, _ = prefill(UnitCache(4, 4, d), Q, K, V)
    np.testing.assert_allclose(O, sdpa64(Q, K, V), rtol=0, atol=1e-12)


def test_prefill_constant_values_give_constant_output():
    rng = np.random.default_rng(3)
    T, d = 40, 8
    Q, K = rand(rng, T, d, scale=3), rand(rng, T, d, scale=3)
    row = rand(rng, d)
    O, _ = prefill(UnitCache(2, 3, d), Q, K, np.tile(row, (T, 1)))
    np.testing.assert_allclose(O, np.tile(row, (T, 1)), rtol=0, atol=1e-12)


def test_prefill_zero_query_column_sums_are_harmonic_tails():
    # Q = 0 makes every causal row uniform: row i gives 1/(i+1) to each j <= i,
    # so c_j = sum_{i=j}^{T-1} 1/(i+1) = H_T - H_j.
    T, d = 50, 4
    rng = np.random.default_rng(5)
    _, c = prefill(UnitCache(5, 5, d), np.zeros((T, d)), rand(rng, T, d), rand(rng, T, d))
    HT = harmonic(T)
    expect = [float(HT - harmonic(j)) for j in range(T)]
    np.testing.assert_allclose(c, expect, rtol=1e-13, atol=0)
    assert abs(c.sum() - T) < 1e-11          # every row carries mass one


def test_prefill_zero_query_output_is_prefix_mean():
    T, d = 30, 6
    rng = np.random.default_rng(8)
    V = rand(rng, T, d)
    O, _ = prefill(UnitCache(3, 3, d), np.zeros((T, d)), rand(rng, T, d), V)
    expect = np.cumsum(V, axis=0) / np.arange(1, T + 1)[:, None]
    np.testing.assert_allclose(O, expect, rtol=0, atol=1e-13)


def test_seed_zero_query_keeps_first_heavy_and_last_local():
    T, d, kh, kl = 50, 4, 5, 7
    rng = np.random.default_rng(9)
    K = rand(rng, T, d)
    cache = UnitCache(kh, kl, d)
    _, c = prefill(cache, np.zeros((T, d)), K, rand(rng, T, d))
    kept = list(range(kh)) + list(range(T - kl, T))
    assert cache.pos.tolist() == kept                       # ascending slots
    np.testing.assert_array_equal(cache.K, K[kept])
    HT = harmonic(T)
    np.testing.assert_array_equal(
        cache.acc, np.array([float(HT - harmonic(j)) for j in kept], dtype=np.float32))


def test_seed_keeps_everything_when_prompt_fits():
    rng = np.random.default_rng(10)
    T, d = 6, 4
    cache = UnitCache(4, 4, d)
    _, c = prefill(cache, rand(rng, T, d), rand(rng, T, d), rand(rng, T, d))
    assert cache.pos.tolist() == [0, 1, 2, 3, 4, 5, -1, -1]
    np.testing.assert_array_equal(cache.acc[:T], c.astype(np.float32))
    assert np.all(cache.acc[T:] == 0)


def _seed_by_repeated_removal(c32, kh, kl):
    T = len(c32)
    keep = set(range(T))
    while len(keep) > kh + kl:
        cand = [p for p in keep if p < T - kl]
        keep.remove(min(cand, key=lambda p: (float(c32[p]), p)))
    return sorted(keep)


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(0, 5), min_size=0, max_size=14), st.integers(0, 4), st.integers(1, 4))
def test_seed_matches_repeated_removal_including_ties(levels, kh, kl):
    # Few distinct levels force many exact ties; both routes must agree.
    c32 = np.array(levels, dtype=np.float32) / 4
    assert seed_positions(c32, kh, kl) == _seed_by_repeated_removal(c32, kh, kl)


def test_seed_tie_drops_the_oldest():
    c32 = np.array([1.0, 2.0, 1.0, 1.0, 0.5, 0.1], dtype=np.float32)
    # T=6, k_local=1 keeps position 5; k_heavy=2 among 0..4: 1 (2.0) then the
    # newest of the three tied at 1.0, which is position 3.
    assert seed_positions(c32, 2, 1) == [1, 3, 5]


# ---------------------------------------------------------------- decode --------

def sequence(rng, N, d, scale=1.0):
    return rand(rng, N, d, scale=scale), rand(rng, N, d, scale=scale), rand(rng, N, d)


def run_sequence(Q, K, V, T, kh, kl):
    return run_unit(kh, kl, Q[:T], K[:T], V[:T], Q[T:], K[T:], V[T:])


@pytest.mark.parametrize("T,n", [(0, 20), (9, 15), (24, 8)])
def test_full_cache_is_full_attention(T, n):
    # Blog §3.1.1 "Full" baseline: with k >= T + n nothing is ever evicted, so every
    # decode output is the causal attention row of the whole sequence and every
    # score is the column sum of the whole causal softmax matrix.
    rng = np.random.default_rng(100 + T)
    d, N = 8, T + n
    Q, K, V = sequence(rng, N, d, scale=1.3)
    cache, _, _, outs, victims = run_sequence(Q, K, V, T, kh=N, kl=3)
    full = sdpa64(Q, K, V)
    np.testing.assert_allclose(outs, full[T:], rtol=0, atol=1e-12)
    assert np.all(victims == -1)
    q, k = torch.from_numpy(Q), torch.from_numpy(K)
    S = (q @ k.T) / math.sqrt(d)
    S = S.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    colsums = torch.softmax(S, dim=1).sum(0).numpy()
    assert cache.pos[:N].tolist() == list(range(N))
    np.testing.assert_allclose([cache.hist64[p] for p in range(N)], colsums, rtol=1e-12)
    np.testing.assert_allclose(cache.acc[:N], colsums, rtol=2e-6)


@pytest.mark.parametrize("T,kl", [(0, 5), (3, 5), (30, 5), (30, 1)])
def test_zero_heavy_budget_is_sliding_window(T, kl):
    # Blog §3.1.1 "Local" baseline: with k_heavy = 0 the token at t attends exactly
    # to positions max(0, t - kl) .. t, and the cache holds the last kl positions.
    rng = np.random.default_rng(200 + T + kl)
    d, n = 8, 25
    N = T + n
    Q, K, V = sequence(rng, N, d, scale=1.3)
    cache, _, _, outs, _ = run_sequence(Q, K, V, T, kh=0, kl=kl)
    for i, t in enumerate(range(T, N)):
        lo = max(0, t - kl)
        s = K[lo:t + 1] @ Q[t] / math.sqrt(d)
        p = np.exp(s - s.max())
        p /= p.sum()
        np.testing.assert_allclose(outs[i], p @ V[lo:t + 1], rtol=0, atol=1e-12)
    assert cache.kept_positions() == list(range(N - kl, N))


@pytest.mark.parametrize("seed", range(4))
def test_attention_mass_is_conserved(seed):
    # Every attention row sums to one, and evicted tokens keep the score they had,
    # so the scores of all tokens ever seen add up to the number of rows.
    rng = np.random.default_rng(300 + seed)
    d, T, n, kh, kl = 16, 40, 60, 6, 5
    Q, K, V = sequence(rng, T + n, d, scale=2.0)
    cache, _, _, _, _ = run_sequence(Q, K, V, T, kh, kl)
    assert len(cache.hist64) == T + n and cache.rows == T + n
    assert abs(sum(cache.hist64.values()) - (T + n)) <= 1e-9 * (T + n)
    assert abs(sum(float(x) for x in cache.hist32.values()) - (T + n)) <= 1e-5 * (T + n)


@pytest.mark.parametrize("seed", range(3))
def test_greedy_state_invariants_every_step(seed):
    rng = np.random.default_rng(400 + seed)
    d, T, n, kh, kl = 8, 12, 50, 4, 3
    Q, K, V = sequence(rng, T + n, d, scale=2.0)
    cache = UnitCache(kh, kl, d)
    prefill(cache, Q[:T], K[:T], V[:T])
    present = {p: T - p for p in range(T)}          # rows each token was present for
    for t in range(T, T + n):
        before = {int(p): float(a) for p, a in zip(cache.pos, cache.acc) if p >= 0}
        _, victim = decode(cache, t, Q[t], K[t], V[t])
        after = {int(p): float(a) for p, a in zip(cache.pos, cache.acc) if p >= 0}
        assert len(after) == min(cache.k, t + 1)
        assert set(range(max(0, t - kl + 1), t + 1)) <= set(after)     # window kept
        for p in before:
            present[p] = present.get(p, 0) + 1
        present[t] = 1
        if victim >= 0:
            gone = set(before) - set(after)
            assert len(gone) == 1
            g = gone.pop()
            assert g <= t - kl
            score_g = cache.hist32[g]
            for p, a in after.items():
                if p <= t - kl:
                    assert (float(score_g), g) < (a, p)                # greedy minimum
        for p, a in after.items():
            if p in before:
                assert a >= before[p]                                  # never decreases
            assert a <= present[p] + 1e-6                              # <= rows present


def test_zero_query_decode_closed_form():
    # Q = 0 everywhere: prompt scores are harmonic tails, every decode row is uniform
    # over the k + 1 keys, so the kept set is {0..kh-1} plus the window at every
    # step, the output is the mean of V over the keys, and each score is a rational
    # closed form.
    T, n, kh, kl, d = 20, 15, 3, 4, 5
    k = kh + kl
    rng = np.random.default_rng(11)
    K = rand(rng, T + n, d)
    V = rand(rng, T + n, d)
    Z = np.zeros((T + n, d))
    cache = UnitCache(kh, kl, d)
    prefill(cache, Z[:T], K[:T], V[:T])
    HT = harmonic(T)
    exact = {j: HT - harmonic(j) for j in range(T)}
    for t in range(T, T + n):
        keys = sorted(int(p) for p in cache.pos) + [t]
        out, _ = decode(cache, t, Z[t], K[t], V[t])
        np.testing.assert_allclose(out, V[keys].mean(axis=0), rtol=0, atol=1e-13)
        for p in keys[:-1]:
            exact[p] += Fraction(1, k + 1)
        exact[t] = Fraction(1, k + 1)
        assert cache.kept_positions() == list(range(kh)) + list(range(t - kl + 1, t + 1))
    for p in cache.kept_positions():
        assert abs(cache.hist64[p] - float(exact[p])) < 1e-13
        assert abs(float(cache.hist32[p]) - float(exact[p])) <= 1e-6 * float(exact[p])


def test_decode_tie_evicts_the_oldest():
    d = 4
    cache = UnitCache(2, 2, d)
    cache.pos[:] = [3, 1, 5, 6]
    cache.acc[:] = 1.0
    cache.K[:] = 0.25
    for p in (3, 1, 5, 6):
        cache.hist32[p], cache.hist64[p] = np.float32(1.0), 1.0
    _, victim = decode(cache, 7, np.ones(d), np.full(d, 0.25), np.ones(d))
    # Candidates are positions <= 7 - 2 = 5, i.e. {3, 1, 5}, all tied: oldest (1) goes.
    assert victim == 1 and cache.pos.tolist() == [3, 7, 5, 6]


def test_near_tie_adoption_accepts_ties_and_rejects_the_rest():
    d = 4
    def fresh():
        c = UnitCache(2, 2, d)
        c.pos[:] = [3, 1, 5, 6]
        c.acc[:] = [1.0, 1.0000001, 2.0, 3.0]
        c.K[:] = 0.25
        for p, a in zip(c.pos, c.acc):
            c.hist32[int(p)], c.hist64[int(p)] = a, float(a)
        return c
    c = fresh()
    _, v = decode(c, 7, np.ones(d), np.full(d, 0.25), np.ones(d), adopt_victim=1)
    assert v == 1 and len(c.ties) == 1
    with pytest.raises(ParityError):
        decode(fresh(), 7, np.ones(d), np.full(d, 0.25), np.ones(d), adopt_victim=2)
    with pytest.raises(ParityError):   # position 6 is inside the window
        decode(fresh(), 7, np.ones(d), np.full(d, 0.25), np.ones(d), adopt_victim=3)


# Prefill near-tie adoption: another implementation's kept set replaces the oracle's only
# when it is a set of the same size that holds the window and differs by swaps whose fp32
# scores lie within the tolerance (the tolerance rule applied at the heavy cutoff).

def _cutoff_scores():
    # Candidates 0..7 (T = 10, k_local = 2), k_heavy = 3. The oracle keeps 5, 6, 1 (scores
    # 9, 8, 7); position 3 is 1e-6 relative below 1 (a near tie), position 4 is 1e-4 below.
    s = np.array([1.0, 7.0, 0.5, 7.0 * (1 - 1e-6), 7.0 * (1 - 1e-4), 9.0, 8.0, 0.25, 0.1, 0.1],
                 dtype=np.float32)
    kept = seed_positions(s, 3, 2)
    assert kept == [1, 5, 6, 8, 9]
    return s, kept


def test_prefill_adoption_accepts_a_near_tie_swap():
    s, kept = _cutoff_scores()
    theirs, ours = adopt_prefill_kept(kept, [3, 5, 6, 8, 9], s, 10, 2)
    assert theirs == [3] and ours == [1]


@pytest.mark.parametrize("other,why", [
    ([4, 5, 6, 8, 9], "not within the tolerance"),      # swap at 1e-4 relative
    ([0, 5, 6, 8, 9], "not within the tolerance"),      # a low score
    ([5, 5, 6, 8, 9], "kept twice"),                    # a duplicated position
    ([1, 1, 5, 6, 8, 9], "kept twice"),
    ([1, 3, 5, 6, 8, 9], "instead of 5"),               # one too many
    ([5, 6, 8, 9], "instead of 5"),                     # one too few
    ([1, 3, 5, 6, 9], "recent-window position is missing"),
    ([1, 5, 6, 9, 10], "outside the prompt"),           # position T
    ([-1, 5, 6, 8, 9], "outside the prompt"),
])
def test_prefill_adoption_rejects_the_rest(other, why):
    s, kept = _cutoff_scores()
    with pytest.raises(ParityError, match=why):
        adopt_prefill_kept(kept, other, s, 10, 2)


def test_prefill_adoption_through_the_prompt():
    # Top-K with Q = 0: the last prompt row is uniform, so every candidate ties exactly and
    # any swap among candidates is a tie; malformed sets are still refused.
    T, d, kh, kl = 12, 4, 3, 2
    rng = np.random.default_rng(3)
    Q, K, V = np.zeros((T, d)), rng.standard_normal((T, d)), rng.standard_normal((T, d))
    ref = UnitCache(kh, kl, d, policy="topk")
    prefill(ref, Q, K, V)
    assert ref.kept_positions() == [7, 8, 9, 10, 11] and not ref.ties
    c = UnitCache(kh, kl, d, policy="topk")
    prefill(c, Q, K, V, adopt_kept=[0, 1, 2, 10, 11])
    assert c.kept_positions() == [0, 1, 2, 10, 11]
    assert c.ties == [("prefill", T, [0, 1, 2], [7, 8, 9])]
    for bad in ([0, 0, 2, 10, 11], [0, 1, 10, 11], [0, 1, 2, 9, 11], [0, 1, 2, 11, 12]):
        with pytest.raises(ParityError):
            prefill(UnitCache(kh, kl, d, policy="topk"), Q, K, V, adopt_kept=bad)
    # under H2O the same prompt's column sums are strictly decreasing (harmonic tails), so
    # no swap is a tie
    with pytest.raises(ParityError):
        prefill(UnitCache(kh, kl, d), Q, K, V, adopt_kept=[0, 1, 3, 10, 11])


# ------------------------------------------------------------ brute force -------

def _oracle_victim_positions(cache):
    return [(t, p) for (t, slot, p, _) in cache.evictions if slot != -1]


@settings(max_examples=120, deadline=None)
@given(T=st.integers(0, 8), n=st.integers(0, 12), kh=st.integers(0, 3), kl=st.integers(1, 3),
       d=st.integers(1, 4), seed=st.integers(0, 10_000))
def test_brute_force_replay_random(T, n, kh, kl, d, seed):
    rng = np.random.default_rng(seed)
    N = T + n
    Q, K, V = sequence(rng, N, d, scale=1.5)
    bf = replay(Q.tolist(), K.tolist(), V.tolist(), T, kh, kl)
    if any(g < 1e-5 for g in bf["gaps"]):
        return                         # near tie: either choice is valid
    c32 = None
    cache, _, c64, outs, _ = run_sequence(Q, K, V, T, kh, kl)
    if T > 0:
        c32 = c64.astype(np.float32)
        srt = sorted(c32[: max(0, T - kl)])
        if any(abs(a - b) <= 1e-5 * max(a, b) for a, b in zip(srt, srt[1:])):
            return
    assert [int(p) for p in sorted(cache.pos) if p >= 0] == bf["kept"]
    assert _oracle_victim_positions(cache) == bf["victims"]
    if n:
        np.testing.assert_allclose(outs, np.array(bf["outs"]), rtol=0, atol=1e-12)
    for p in range(N):
        assert abs(cache.hist64[p] - bf["scores"][p]) <= 1e-12 * max(1.0, bf["scores"][p])


@pytest.mark.parametrize("T,n,kh,kl", [(0, 12, 2, 2), (5, 10, 1, 2), (8, 12, 3, 3), (6, 9, 0, 2)])
def test_brute_force_replay_exact_uniform(T, n, kh, kl):
    # Q = 0: every row uniform; the replay runs in exact fractions, so exact ties
    # between equal scores do occur and must resolve the same way.
    d = 3
    rng = np.random.default_rng(T * 100 + n)
    N = T + n
    K, V = rand(rng, N, d), rand(rng, N, d)
    Z = np.zeros((N, d))
    bf = replay([[0.0] * d] * N, K.tolist(), V.tolist(), T, kh, kl, uniform=True)
    cache, _, c64, outs, _ = run_sequence(Z, K, V, T, kh, kl)
    assert [int(p) for p in sorted(cache.pos) if p >= 0] == bf["kept"]
    assert _oracle_victim_positions(cache) == bf["victims"]
    np.testing.assert_allclose(outs, np.array([[float(x) for x in o] for o in bf["outs"]]),
                               rtol=0, atol=1e-12)
    for p in range(N):
        assert abs(cache.hist64[p] - float(bf["scores"][p])) < 1e-12


# ---------------------------------------------------------------------------
# Eviction policies other than H2O ([blog] §3.1.1 baselines, §3.3 Q1 StreamLLM)
# ---------------------------------------------------------------------------

def _policy_run(policy, param, kh, kl, T, n, d=16, seed=0):
    rng = np.random.default_rng(seed)
    N = T + n
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    cache = UnitCache(kh, kl, d, policy=policy, policy_param=param)
    prefill(cache, Q[:T], K[:T], V[:T])
    kept = [cache.kept_positions()]
    for i in range(n):
        decode(cache, T + i, Q[T + i], K[T + i], V[T + i])
        kept.append(cache.kept_positions())
    return kept


@pytest.mark.parametrize("n_sink,kl,T", [(4, 8, 40), (1, 3, 10), (0, 5, 12)])
def test_sinks_policy_keeps_first_tokens_and_window(n_sink, kl, T):
    # StreamLLM's cache: the first n_sink tokens plus the most recent window. With
    # k_heavy = n_sink that is the whole budget, after the prompt and after every step.
    kept = _policy_run("sinks", n_sink, n_sink, kl, T, n=30)
    for i, ks in enumerate(kept):
        last = T - 1 + i
        assert ks == sorted(set(range(n_sink)) | set(range(last - kl + 1, last + 1)))


@pytest.mark.parametrize("s,kh,kl,T", [(4, 5, 6, 60), (3, 2, 1, 20), (7, 3, 4, 90)])
def test_strided_policy_keeps_window_and_latest_multiples(s, kh, kl, T):
    # Strided retention: the window plus the k_heavy most recent multiples of the stride
    # among the older positions (enough of them exist in these cases).
    kept = _policy_run("strided", s, kh, kl, T, n=40)
    for i, ks in enumerate(kept):
        last = T - 1 + i
        older = [p for p in range(last - kl + 1) if p % s == 0]
        assert ks == sorted(set(older[-kh:]) | set(range(last - kl + 1, last + 1)))


def test_position_policies_ignore_the_values():
    # Under a position-only ranking the kept sets cannot depend on Q/K/V.
    for policy, param in (("sinks", 3), ("strided", 5)):
        a = _policy_run(policy, param, 3, 4, 30, 20, seed=1)
        b = _policy_run(policy, param, 3, 4, 30, 20, seed=2)
        assert a == b


def test_topk_policy_evicts_the_least_attended_now():
    # Keys along the query: logit_j = a_j / sqrt(d), so this step's attention order is the
    # order of a_j by construction (no softmax needed). Slots hold positions 0..4 with
    # a = [3, 1, 4, 1, 5]; k_local = 2 protects positions 4 and the new token 5. The
    # candidates are positions 0..3; the least attended have a = 1 (positions 1 and 3),
    # and the tie goes to the older one: position 1 leaves, whatever the running scores.
    d = 8
    q = np.zeros(d)
    q[0] = 1.0
    a = [3.0, 1.0, 4.0, 1.0, 5.0]
    cache = UnitCache(3, 2, d, policy="topk")
    for slot, (pos, ai) in enumerate(zip(range(5), a)):
        cache.pos[slot] = pos
        cache.K[slot] = ai * q
        cache.V[slot] = 0.0
        cache.acc[slot] = np.float32([0.1, 9.0, 0.2, 9.0, 0.3][slot])   # H2O would pick pos 0
        cache.hist32[pos], cache.hist64[pos] = cache.acc[slot], float(cache.acc[slot])
    _, victim = decode(cache, 5, q, 2.0 * q, np.zeros(d))
    assert victim == 1 and cache.kept_positions() == [0, 2, 3, 4, 5]
    # the same state under H2O evicts the lowest running score instead (position 0)
    cache2 = UnitCache(3, 2, d)
    for slot in range(5):
        cache2.pos[slot], cache2.K[slot], cache2.acc[slot] = cache.pos[slot], a[slot] * q, \
            np.float32([0.1, 9.0, 0.2, 9.0, 0.3][slot])
        cache2.pos[slot] = slot
        cache2.hist32[slot], cache2.hist64[slot] = cache2.acc[slot], float(cache2.acc[slot])
    _, v2 = decode(cache2, 5, q, 2.0 * q, np.zeros(d))
    assert v2 == 0


def test_topk_seed_zero_query_keeps_the_newest():
    # Q = 0: the prompt's last attention row is exactly uniform, so every candidate ties
    # and the newest k_heavy candidates are kept. (Ranking by the column sums instead would
    # keep the oldest: c_j = H_T - H_j decreases in j.)
    T, d, kh, kl = 40, 8, 6, 5
    rng = np.random.default_rng(0)
    K, V = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    c = UnitCache(kh, kl, d, policy="topk")
    prefill(c, np.zeros((T, d)), K, V)
    assert c.kept_positions() == list(range(T - kl - kh, T))
    h = UnitCache(kh, kl, d)
    prefill(h, np.zeros((T, d)), K, V)
    assert h.kept_positions() == list(range(kh)) + list(range(T - kl, T))
    # the running scores still start from the column sums: acc_j = H_T - H_j
    for s_, p in enumerate(c.pos):
        exact = sum(Fraction(1, i + 1) for i in range(int(p), T))
        assert abs(float(c.acc[s_]) - float(exact)) <= 1e-6 * float(exact)


def test_topk_seed_follows_the_last_row_not_the_column_sums():
    # Two key directions: keys at the positions in M point along e0, the others along e1.
    # Every query but the last points along e1 (so the column sums favour positions outside
    # M), the last one along e0 with a large norm (so its attention sits on M). Top-K keeps M
    # (the highest current attention); H2O keeps the highest column sums, outside M.
    T, d, kh, kl = 30, 4, 4, 3
    M = [2, 9, 15, 21]
    e0, e1 = np.eye(d)[0], np.eye(d)[1]
    K = np.array([e0 if j in M else e1 for j in range(T)], dtype=np.float64)
    Q = np.array([6.0 * e1] * (T - 1) + [6.0 * e0])
    V = np.random.default_rng(1).standard_normal((T, d))
    c = UnitCache(kh, kl, d, policy="topk")
    prefill(c, Q, K, V)
    assert c.kept_positions() == sorted(M + list(range(T - kl, T)))
    h = UnitCache(kh, kl, d)
    prefill(h, Q, K, V)
    assert not set(M) & set(h.kept_positions())


def test_policy_parameters_are_checked():
    with pytest.raises(ValueError):
        UnitCache(2, 2, 8, policy="strided", policy_param=0)
    with pytest.raises(ValueError):
        UnitCache(2, 2, 8, policy="sinks", policy_param=-1)
    with pytest.raises(ValueError):
        UnitCache(2, 2, 8, policy="lru")


# ---------------------------------------------------------------------------
# E4M3 slots ([blog] §3.3 Q3: H2O with KV quantisation; the format is the OCP FP8 E4M3
# of the oracle's reading R14)
# ---------------------------------------------------------------------------

from oracle import e4m3_decode, e4m3_encode, e4m3_round, quantize_row  # noqa: E402


def _torch_e4m3(x32):
    """torch's own float32 -> float8_e4m3fn conversion (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy(), t.view(torch.uint8).numpy()


def _all_finite(dtype):
    bits = np.arange(1 << 16, dtype=np.uint32)
    if dtype == "f16":
        x = bits.astype(np.uint16).view(np.float16).astype(np.float32)
    else:
        x = (bits << 16).view(np.float32)
    return x[np.isfinite(x)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_e4m3_matches_the_library_conversion_on_every_half_value(dtype):
    # Every finite fp16 / bf16 value inside the E4M3 range, plus random fp32 values
    # spread over all binades, against torch's float8_e4m3fn cast.
    x = _all_finite(dtype)
    rng = np.random.default_rng(0)
    r32 = (rng.choice([-1.0, 1.0], 20000) * np.exp2(rng.uniform(-14, 8.8, 20000))).astype(np.float32)
    x = np.concatenate([x[np.abs(x) <= 448.0], r32[np.abs(r32) <= 448.0]])
    want, codes = _torch_e4m3(x)
    got = e4m3_round(x)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))
    assert np.array_equal(e4m3_encode(got), codes)


def test_e4m3_closed_forms():
    cases = {  # value -> (rounded value, code), from the E4M3 layout by hand
        448.0: (448.0, 0x7E), -448.0: (-448.0, 0xFE),
        1000.0: (448.0, 0x7E), -1e9: (-448.0, 0xFE),           # saturation
        1.0: (1.0, 0x38), 1.0625: (1.0, 0x38),                 # tie 1 + 1/16 goes to even
        1.1875: (1.25, 0x3A), 1.125: (1.125, 0x39),            # tie 1 + 3/16 goes up to even
        2.0 ** -6: (2.0 ** -6, 0x08),                          # smallest normal
        2.0 ** -9: (2.0 ** -9, 0x01),                          # smallest subnormal
        2.0 ** -10: (0.0, 0x00), 3 * 2.0 ** -10: (2 * 2.0 ** -9, 0x02),
        7 * 2.0 ** -9: (7 * 2.0 ** -9, 0x07), 0.0: (0.0, 0x00),
        240.0: (240.0, 0x77), 232.0: (224.0, 0x76), 248.0: (256.0, 0x78),
    }
    for x, (r, code) in cases.items():
        got = e4m3_round(np.float32(x))
        assert float(got) == r, x
        assert int(e4m3_encode(got)) == code, x
        assert float(e4m3_decode(code)) == r, x


def test_e4m3_codes_round_trip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3_decode(codes)
    assert np.array_equal(e4m3_round(vals), vals)
    assert np.array_equal(e4m3_encode(vals), codes)
    assert np.isnan(e4m3_decode(np.array([0x7F, 0xFF]))).all()
    assert float(np.nanmax(np.abs(vals))) == 448.0


def test_quantize_row_scale_by_hand():
    # scale 3: 1/3 in fp32 is 0x3EAAAAAB = 0.3333333432674408; 1.0 times it is the same;
    # E4M3 steps of 2^-5 in [0.25, 0.5): 0.33333 / 0.03125 = 10.67 -> 11 -> 0.34375,
    # code 0 0101 011 = 0x2B; read back 0.34375 * 3 = 1.03125.
    codes, vals = quantize_row(np.array([1.0, -1.0, 0.0, 2000.0]), 3.0)
    assert list(codes) == [0x2B, 0xAB, 0x00, 0x7E]
    assert list(vals) == [1.03125, -1.03125, 0.0, 448.0 * 3]


def _e4m3_exact(rng, shape, scale):
    """Values that E4M3 holds exactly, times scale: integers in [-15, 15] / 4."""
    return rng.integers(-15, 16, size=shape) / 4.0 * scale


@pytest.mark.parametrize("scale", [1.0, 2.0, 0.125])
def test_e4m3_slots_reduce_to_plain_slots_on_representable_rows(scale):
    # When every K/V row is a representable value times a power-of-two scale, quantising
    # changes nothing: the E4M3 cache must then match the unquantised one step for step.
    rng = np.random.default_rng(3)
    T, n, d, kh, kl = 20, 15, 8, 3, 4
    Q = rng.standard_normal((T + n, d))
    K, V = _e4m3_exact(rng, (T + n, d), scale), _e4m3_exact(rng, (T + n, d), scale)
    a = run_unit(kh, kl, Q[:T], K[:T], V[:T], Q[T:], K[T:], V[T:])
    b = run_unit(kh, kl, Q[:T], K[:T], V[:T], Q[T:], K[T:], V[T:],
                 slot_format="e4m3", k_scale=scale, v_scale=scale)
    assert np.array_equal(a[3], b[3]) and np.array_equal(a[4], b[4])
    assert np.array_equal(a[0].K, b[0].K) and np.array_equal(a[0].pos, b[0].pos)


def test_e4m3_step_attends_to_what_the_cache_then_holds():
    # While the cache fills nothing leaves, so after each step the valid slots are exactly
    # the keys the step attended to: its output must be attention over the stored rows,
    # and the stored codes must decode to the stored values.
    rng = np.random.default_rng(4)
    d = 16
    cache = UnitCache(6, 4, d, slot_format="e4m3", k_scale=0.37, v_scale=1.9)
    for t in range(9):
        q, k, v = (rng.standard_normal(d) * 3 for _ in range(3))
        out, victim = decode(cache, t, q, k, v)
        assert victim == -1
        n = t + 1
        s = cache.K[:n] @ q / math.sqrt(d)
        p = np.exp(s - s.max())
        np.testing.assert_allclose(out, (p / p.sum()) @ cache.V[:n], rtol=1e-12, atol=1e-12)
        assert np.array_equal(e4m3_decode(cache.Kc[:n]) * float(np.float32(0.37)), cache.K[:n])
        assert np.array_equal(e4m3_decode(cache.Vc[:n]) * float(np.float32(1.9)), cache.V[:n])


def test_e4m3_slot_parameters_are_checked():
    with pytest.raises(ValueError):
        UnitCache(2, 2, 8, slot_format="e5m2")
    with pytest.raises(ValueError):
        UnitCache(2, 2, 8, slot_format="e4m3", k_scale=0.0)
    with pytest.raises(ValueError):
        UnitCache(2, 2, 8, slot_format="e4m3", v_scale=float("inf"))
