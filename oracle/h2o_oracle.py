"""Plain CPU oracle for the H2O (Heavy-Hitter Oracle) KV-cache eviction hot path.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check in __graft_entry__ and
the CPU-baseline leg of bench.py may import this module. The product path (the
HIP library and its Python binding) never imports or calls it, and this module
imports nothing from the product path.

It is slow and obviously correct on purpose: float64 NumPy, one unit
(layer, sequence, head) at a time, no blocking, no fusion.

Pages cited (by title and section):
  [blog]     The H2O summary post at ttsmallhot.github.io/posts/8adb0d1a.html.
             §2.1.1 attention sparsity (the scaled softmax of Q K^T / sqrt(d)),
             §2.1.2 heavy hitters (accumulated attention score of a token),
             §2.2 method (budget split into k_local recent + k_heavy heavy
             hitters; the running score ledger; greedy eviction of the lowest
             score outside the recent tokens),
             §2.3 system implementation (evicted slot is marked free and the new
             token's K/V is written at that address; no compaction),
             §3.1.1 baselines (Full KV cache, Local sliding window).
  [analysis] "H2O Heavy-Hitter Oracle 分析" (liuhc.cn).
             §3.1 heavy-hitter identification (per head, cumulative attention
             over the token axis, then the top-k of it),
             §3.2 core eviction logic (score of a token = sum of its attention
             over all steps; victim = argmin of the score; the new token always
             joins the cache).

Readings taken where the pages are silent or disagree (each is listed with its
justification in the design notes of the repository):
  R1  Logits are scaled by 1/sqrt(d) ([blog] §2.1.1 says the paper drops the
      factor only for brevity).
  R2  The recent window protects positions (t - k_local, t], the new token
      included; eviction candidates are cached tokens with pos <= t - k_local.
      [blog] §2.2 protects the recent tokens; [analysis] §3.2 (no window) is not
      followed except for "the new token always joins".
  R3  Within a decode step the new token's probabilities are added first, then
      the victim is chosen on the updated scores; the new token's own score is
      its own probability.
  R4  While fewer than k slots are valid the new token is appended to the next
      free slot and nothing is evicted; free slots take no part in attention.
  R5  The prefill output is full causal attention over the prompt; eviction only
      decides which K/V rows persist.
  R6  Prefill column sums run over every causal row of the prompt.
  R7  At prefill, heavy hitters are chosen only outside the last k_local
      positions, ranked by (score desc, position desc): on equal score the
      older token is dropped, matching the decode tie rule.
  R8  After prefill the kept positions fill slots 0.. in ascending position order.
  R9  Decode ties on score evict the oldest position.
  R10 Scores live in fp32: prefill seeds each slot with fl32(c_j); each decode
      step adds fl32(p) with one fp32 add. Decisions are taken on these fp32
      values. A float64 shadow of every score is kept for the invariants.
  R11 Eviction is per head and per layer (the analysis page's §4 notes that each
      layer decides independently).
  R12 k_local >= 1, so the new token is never a candidate.

Eviction policies. The baselines and comparisons the pages name ([blog] §3.1.1:
Local, Strided sparse attention, Top-K by current attention; §3.3 Q1: StreamLLM's
sinks plus window; §3.3 Q4: heavy-only and local-only) run on the same slots with
a different ranking. Seeding keeps the last k_local positions plus the top k_heavy
of the rest by (seed score desc, position desc); a decode step evicts, among the
candidates (pos <= t - k_local), the minimum of (key, position):
  "h2o"      seed score c_j (the column sum), key = acc (the running score);
  "sinks"    seed score [j < n_sink], key = [pos < n_sink]: with k_heavy = n_sink
             the cache holds the first n_sink tokens and the most recent window;
  "strided"  seed score [j % s == 0], key = [pos % s == 0]: the window plus the
             most recent multiples of the stride s;
  "topk"     key = this step's probability p of the slot (the token with the
             least attention now goes); seed score = the prompt's last row of
             attention, P[T-1, j] (R13).
Local is "h2o" with k_heavy = 0, heavy-only is k_local = 1. The running score acc
is kept under every policy.
  R13 [blog] §3.1.1 defines Top-K as keeping the tokens with the highest current
      attention score. At a decode step the current attention is that step's
      softmax row; at the end of the prompt it is the last prompt row, P[T-1, :],
      so Top-K seeds by fl32(P[T-1, j]). (The running score acc still starts
      from the column sums under every policy.)

Quantised slots. [blog] §3.3 Q3 reports that H2O combines with KV quantisation
but names no scheme. With slot_format "e4m3" every K/V row that enters a slot
is stored as OCP FP8 E4M3 codes (R14); prefill attention still reads the
prompt's own K/V.
  R14 One scale per cache for K and one for V (k_scale, v_scale > 0). A row x is
      stored as codes e4m3(fl32(x * fl32(1 / scale))), rounded to nearest, ties
      to even, saturated at +-448; it is read back as code value * scale. The new
      token's K/V are quantised when they join, before the step's attention, so
      the step attends to exactly what the cache then holds.

Near-tie adoption (the tolerance rule): when an accelerator implementation made
a different choice whose score lies within `rel_tol` (relative) of the oracle's
own choice, the oracle may adopt that choice so that the two states stay
comparable; each adoption is logged on the unit. Any other disagreement raises
ParityError.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

FREE = -1


class ParityError(AssertionError):
    """The other implementation's discrete choice is not a near tie."""


# ---------------------------------------------------------------------------
# Attention over the prompt ([blog] §2.1.1; R1, R5, R6)
# ---------------------------------------------------------------------------

def causal_softmax(Q: np.ndarray, K: np.ndarray) -> np.ndarray:
    """P = row-softmax(Q K^T / sqrt(d)) with P_ij = 0 for j > i, in float64."""
    T, d = Q.shape
    S = (Q @ K.T) / math.sqrt(d)
    future = np.triu(np.ones((T, T), dtype=bool), k=1)
    S = np.where(future, -np.inf, S)
    E = np.exp(S - S.max(axis=1, keepdims=True))
    return E / E.sum(axis=1, keepdims=True)


def column_sums(P: np.ndarray) -> np.ndarray:
    """c_j = sum over rows i of P_ij; the causal mask makes this sum over i >= j.

    This is the cumulative attention each prompt token received
    ([analysis] §3.1: accumulate the attention scores of each token, per head).
    """
    return P.sum(axis=0)


POLICIES = ("h2o", "sinks", "strided", "topk")
SLOT_FORMATS = ("input", "e4m3")


# ---------------------------------------------------------------------------
# OCP FP8 E4M3 slot codes (R14). E4M3: a sign bit, 4 exponent bits with bias 7
# and 3 mantissa bits. Exponent field 0 holds the subnormals m * 2^-9; exponent
# field 15 with mantissa 7 is NaN (no infinities), so the largest finite value
# is 1.75 * 2^8 = 448.
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_round(y) -> np.ndarray:
    """The E4M3 value nearest each y (ties to even), saturated at +-448, as float64."""
    y = np.clip(np.asarray(y, dtype=np.float64), -E4M3_MAX, E4M3_MAX)
    a = np.abs(y)
    _, e = np.frexp(a)                   # a = f * 2^e with f in [0.5, 1)
    lead = np.maximum(e - 1, -6)         # exponent of the leading bit; subnormals share -6
    quantum = np.ldexp(1.0, lead - 3)    # 3 mantissa bits below the leading bit
    return np.copysign(np.rint(a / quantum) * quantum, y)


def e4m3_encode(r) -> np.ndarray:
    """Codes (uint8) of E4M3 values r (as e4m3_round returns them)."""
    r = np.asarray(r, dtype=np.float64)
    a = np.abs(r)
    _, e = np.frexp(a)
    normal = a >= 2.0 ** -6
    lead = np.where(normal, e - 1, -6)
    mant = np.where(normal, a / np.ldexp(1.0, lead - 3) - 8, a / 2.0 ** -9)
    field = np.where(normal, lead + 7, 0)
    code = (np.signbit(r).astype(np.int64) << 7) | (field.astype(np.int64) << 3) | \
        mant.astype(np.int64)
    return code.astype(np.uint8)


def e4m3_decode(code) -> np.ndarray:
    """float64 value of each E4M3 code (NaN for the two NaN codes)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    field, mant = (c >> 3) & 15, c & 7
    mag = np.where(field == 0, mant * 2.0 ** -9, np.ldexp(1.0 + mant / 8.0, field - 7))
    return np.where((field == 15) & (mant == 7), np.nan, sign * mag)


def quantize_row(x, scale):
    """Codes and read-back values of a K or V row stored in an E4M3 slot (R14)."""
    s32 = np.float32(scale)
    with np.errstate(over="ignore"):   # a product past the fp32 range is +-inf, then saturates
        y = np.asarray(x, dtype=np.float32) * (np.float32(1.0) / s32)   # one fp32 rounding
    r = e4m3_round(y)
    return e4m3_encode(r), r * float(s32)


def policy_seed_scores(policy: str, param: int, c32: np.ndarray,
                       last_row: np.ndarray | None = None) -> np.ndarray:
    """The fp32 score each prompt position is ranked by at seeding (see the header).

    c32: the fp32 column sums; last_row: the prompt's last attention row P[T-1, :]
    in float64 (used by "topk", R13)."""
    j = np.arange(len(c32))
    if policy == "h2o":
        return np.asarray(c32, dtype=np.float32)
    if policy == "topk":
        return np.asarray(last_row, dtype=np.float64).astype(np.float32)
    if policy == "sinks":
        return (j < param).astype(np.float32)
    if policy == "strided":
        return (j % param == 0).astype(np.float32)
    raise ValueError(f"unknown policy {policy!r}")


def seed_positions(c32: np.ndarray, k_heavy: int, k_local: int) -> list[int]:
    """Positions kept after a prompt of length T = len(c32).

    If T <= k every position is kept. Otherwise the last k_local positions are
    kept ([blog] §2.2 recent tokens) plus the k_heavy highest-scoring of the
    remaining ones ([analysis] §3.1 top-k of cumulative attention), ranked by
    (score desc, position desc) on the fp32 scores (R7, R10). Under another
    policy c32 holds that policy's seed scores.
    """
    T = len(c32)
    k = k_heavy + k_local
    if T <= k:
        return list(range(T))
    candidates = range(0, T - k_local)
    ranked = sorted(candidates, key=lambda j: (-float(c32[j]), -j))
    heavy = ranked[:k_heavy]
    return sorted(heavy + list(range(T - k_local, T)))


# ---------------------------------------------------------------------------
# One unit's cache state ([blog] §2.2 budget of k slots; §2.3 slots overwritten
# in place)
# ---------------------------------------------------------------------------

@dataclass
class UnitCache:
    k_heavy: int
    k_local: int
    head_dim: int
    policy: str = "h2o"                      # eviction ranking (see the header)
    policy_param: int = 0                    # n_sink ("sinks") or the stride ("strided")
    slot_format: str = "input"               # "input" or "e4m3" (R14)
    k_scale: float = 1.0                     # E4M3 scales of K and V (R14)
    v_scale: float = 1.0
    pos: np.ndarray = field(init=False)      # [k] int64, FREE = -1
    K: np.ndarray = field(init=False)        # [k, d] float64 (exact stored values)
    V: np.ndarray = field(init=False)
    Kc: np.ndarray = field(init=False)       # [k, d] uint8 E4M3 codes ("e4m3" only)
    Vc: np.ndarray = field(init=False)
    acc: np.ndarray = field(init=False)      # [k] float32 accumulated score
    hist32: dict = field(init=False)         # position -> fp32 score (frozen on eviction)
    hist64: dict = field(init=False)         # position -> float64 shadow score
    evictions: list = field(init=False)      # (t, slot, position, fp32 score)
    ties: list = field(init=False)           # near-tie adoptions
    rows: int = field(init=False)            # attention rows accumulated so far

    def __post_init__(self):
        if self.k_local < 1 or self.k_heavy < 0:
            raise ValueError("need k_local >= 1 and k_heavy >= 0 (R12)")
        if self.policy not in POLICIES:
            raise ValueError(f"unknown policy {self.policy!r}")
        if (self.policy == "sinks" and self.policy_param < 0) or \
                (self.policy == "strided" and self.policy_param < 1):
            raise ValueError(f"bad parameter {self.policy_param} for policy {self.policy!r}")
        if self.slot_format not in SLOT_FORMATS:
            raise ValueError(f"unknown slot format {self.slot_format!r}")
        if self.slot_format == "e4m3" and not all(
                math.isfinite(x) and x > 0 for x in (self.k_scale, self.v_scale)):
            raise ValueError("E4M3 scales must be finite and > 0 (R14)")
        k = self.k
        self.pos = np.full(k, FREE, dtype=np.int64)
        self.K = np.zeros((k, self.head_dim))
        self.V = np.zeros((k, self.head_dim))
        self.Kc = np.zeros((k, self.head_dim), dtype=np.uint8)
        self.Vc = np.zeros((k, self.head_dim), dtype=np.uint8)
        self.acc = np.zeros(k, dtype=np.float32)
        self.hist32, self.hist64 = {}, {}
        self.evictions, self.ties = [], []
        self.rows = 0

    @property
    def k(self) -> int:
        return self.k_heavy + self.k_local

    @property
    def n_valid(self) -> int:
        return int((self.pos != FREE).sum())

    def kept_positions(self) -> list[int]:
        return sorted(int(p) for p in self.pos if p != FREE)

    def stored(self, k_row, v_row):
        """What a slot holds for these K/V rows: (k value, v value, k codes, v codes)."""
        if self.slot_format == "e4m3":
            kc, kv = quantize_row(k_row, self.k_scale)
            vc, vv = quantize_row(v_row, self.v_scale)
            return kv, vv, kc, vc
        return np.asarray(k_row, np.float64), np.asarray(v_row, np.float64), None, None

    def write(self, slot, k_row, v_row):
        self.K[slot], self.V[slot], kc, vc = self.stored(k_row, v_row)
        if kc is not None:
            self.Kc[slot], self.Vc[slot] = kc, vc


def _near(a: float, b: float, rel_tol: float) -> bool:
    return abs(a - b) <= rel_tol * max(abs(a), abs(b))


def adopt_prefill_kept(kept, other, score, T, k_local, rel_tol=1e-5):
    """Whether another implementation's kept set `other` may replace the oracle's `kept`.

    The rule (near ties at the heavy cutoff, R10 + the tolerance rule of the header):
    `other` must be a set of distinct prompt positions in [0, T) of the oracle's size
    that holds the whole recent window, and every position it keeps instead of the
    oracle's must score within rel_tol (relative, on the fp32 seed scores) of every
    position the oracle keeps instead of it. Returns (theirs, ours) — the positions
    kept only by `other` and only by the oracle — or raises ParityError.
    """
    other = [int(p) for p in other]
    theirs = sorted(set(other) - set(kept))
    ours = sorted(set(kept) - set(other))
    why = None
    if len(set(other)) != len(other):
        why = "a position is kept twice"
    elif len(other) != len(kept):
        why = f"{len(other)} positions kept instead of {len(kept)}"
    elif any(not 0 <= p < T for p in other):
        why = "a kept position lies outside the prompt"
    elif set(range(max(0, T - k_local), T)) - set(other):
        why = "a recent-window position is missing"
    elif not (len(theirs) == len(ours) > 0):
        why = "the sets differ in size"
    elif not all(_near(float(score[x]), float(score[y]), rel_tol) for x in theirs for y in ours):
        why = "the swapped scores are not within the tolerance"
    if why is not None:
        raise ParityError(f"prefill kept sets differ beyond a near tie ({why}): "
                          f"only theirs {theirs}, only ours {ours}")
    return theirs, ours


def prefill(cache: UnitCache, Q, K, V, adopt_kept=None, rel_tol=1e-5):
    """Run the prompt through one unit and seed its cache.

    Returns (O, c64): O = P V (float64, [T, d]) and the float64 column sums.
    `adopt_kept`, if given, is another implementation's kept positions (a list);
    it is adopted when adopt_prefill_kept accepts it, and the swap is logged.
    """
    Q, K, V = (np.asarray(x, dtype=np.float64) for x in (Q, K, V))
    T = Q.shape[0]
    if T == 0:
        return np.zeros((0, cache.head_dim)), np.zeros(0)
    P = causal_softmax(Q, K)
    O = P @ V
    c64 = column_sums(P)
    c32 = c64.astype(np.float32)
    score = policy_seed_scores(cache.policy, cache.policy_param, c32, last_row=P[T - 1])
    kept = seed_positions(score, cache.k_heavy, cache.k_local)

    if adopt_kept is not None:
        other = [int(p) for p in adopt_kept]
        if sorted(other) != kept:
            theirs, ours = adopt_prefill_kept(kept, other, score, T, cache.k_local, rel_tol)
            cache.ties.append(("prefill", T, theirs, ours))
            kept = sorted(other)

    for j in range(T):
        cache.hist32[j] = c32[j]
        cache.hist64[j] = float(c64[j])
    for s, p in enumerate(kept):
        cache.pos[s] = p
        cache.write(s, K[p], V[p])
        cache.acc[s] = c32[p]
    dropped = sorted(set(range(T)) - set(kept))
    for p in dropped:
        cache.evictions.append((T - 1, FREE, p, c32[p]))
    cache.rows += T
    return O, c64


def _decode_keys(cache: UnitCache, p32: np.ndarray) -> np.ndarray:
    """Per slot, the fp32 value a decode step ranks eviction candidates by (header)."""
    if cache.policy == "h2o":
        return cache.acc.copy()
    if cache.policy == "topk":
        return np.asarray(p32, dtype=np.float32)
    if cache.policy == "sinks":
        return (cache.pos < cache.policy_param).astype(np.float32)
    return (cache.pos % cache.policy_param == 0).astype(np.float32)


def decode(cache: UnitCache, t: int, q, k_new, v_new, adopt_victim=None,
           rel_tol=1e-5):
    """One decode step for the token at position t (t = tokens seen before it).

    Attention runs over the valid slots plus the new token ([blog] §2.1.1 scaled
    softmax); each probability is added to its token's running score ([blog]
    §2.2 score ledger; [analysis] §3.2 score = sum over steps; R3, R10). If the
    cache is full, the candidate with the lowest (score, position) outside the
    recent window is evicted ([blog] §2.2 greedy step; [analysis] §3.2 argmin;
    R2, R9) and the new token's K/V overwrites that slot ([blog] §2.3). If it
    is not full, the new token takes the next free slot (R4).

    Returns (out, victim_slot): out is float64 [d]; victim_slot is the evicted
    slot or -1 when the token was appended.
    """
    q, k_new, v_new = (np.asarray(x, dtype=np.float64) for x in (q, k_new, v_new))
    k_in, v_in = k_new, v_new
    k_new, v_new, _, _ = cache.stored(k_in, v_in)    # what the new token's slot will hold (R14)
    n = cache.n_valid
    assert np.all(cache.pos[:n] != FREE) and np.all(cache.pos[n:] == FREE), \
        "valid slots must be a prefix"
    if n > 0:
        assert int(cache.pos[:n].max()) < t, "decode positions must increase"
    keys = np.vstack([cache.K[:n], k_new[None, :]])
    vals = np.vstack([cache.V[:n], v_new[None, :]])
    s = (keys @ q) / math.sqrt(cache.head_dim)
    e = np.exp(s - s.max())
    p = e / e.sum()
    out = p @ vals

    p32 = p.astype(np.float32)
    for slot in range(n):
        cache.acc[slot] = np.float32(cache.acc[slot] + p32[slot])
        pos = int(cache.pos[slot])
        cache.hist32[pos] = cache.acc[slot]
        cache.hist64[pos] += float(p[slot])
    acc_new = p32[n]
    cache.hist32[t] = acc_new
    cache.hist64[t] = float(p[n])
    cache.rows += 1

    if n < cache.k:
        slot, victim = n, -1
    else:
        limit = t - cache.k_local
        cand = [s_ for s_ in range(cache.k) if cache.pos[s_] <= limit]
        key = _decode_keys(cache, p32[:n])
        victim = min(cand, key=lambda s_: (float(key[s_]), int(cache.pos[s_])))
        if adopt_victim is not None and int(adopt_victim) != victim:
            g = int(adopt_victim)
            if g not in cand or not _near(float(key[g]), float(key[victim]), rel_tol):
                raise ParityError(
                    f"t={t}: victim slot {g} (pos {int(cache.pos[g]) if 0 <= g < cache.k else None}) "
                    f"is not a near tie with the oracle's slot {victim} "
                    f"(pos {int(cache.pos[victim])}, key {float(key[victim])!r})")
            cache.ties.append(("decode", t, int(cache.pos[g]), int(cache.pos[victim]),
                               float(key[g]), float(key[victim])))
            victim = g
        slot = victim
        cache.evictions.append((t, slot, int(cache.pos[slot]), cache.acc[slot]))

    cache.pos[slot] = t
    cache.write(slot, k_in, v_in)
    cache.acc[slot] = acc_new
    return out, victim


# ---------------------------------------------------------------------------
# Convenience: a whole unit, prompt then every decode step
# ---------------------------------------------------------------------------

def run_unit(k_heavy, k_local, Qp, Kp, Vp, qd, kd, vd, t0=None,
             adopt_kept=None, adopt_victims=None, rel_tol=1e-5, **cache_kw):
    """Prefill with Qp/Kp/Vp ([T, d]) then decode rows of qd/kd/vd ([n, d]).

    cache_kw are further UnitCache fields (policy, slot format, scales).
    Returns (cache, O_prefill, c64, outs [n, d], victims [n]).
    """
    d = np.asarray(Qp).shape[-1] if np.asarray(Qp).size else np.asarray(qd).shape[-1]
    cache = UnitCache(k_heavy, k_local, d, **cache_kw)
    O, c64 = prefill(cache, Qp, Kp, Vp, adopt_kept=adopt_kept, rel_tol=rel_tol)
    T = np.asarray(Qp).shape[0] if t0 is None else t0
    n = np.asarray(qd).shape[0]
    outs = np.zeros((n, d))
    victims = np.zeros(n, dtype=np.int64)
    for i in range(n):
        adopt = None if adopt_victims is None else int(adopt_victims[i])
        outs[i], victims[i] = decode(cache, T + i, qd[i], kd[i], vd[i],
                                     adopt_victim=adopt, rel_tol=rel_tol)
    return cache, O, c64, outs, victims
