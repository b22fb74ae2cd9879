"""Regression lock: the oracle still reproduces its budget-3 fixture exactly.

The fixture was written by tests/golden/make_golden.py, which calls only the
oracle (the H2O blog's §2.2 budget-3 illustration has no values in the text).
"""
import json
import os

import numpy as np

from oracle import run_unit

HERE = os.path.dirname(os.path.abspath(__file__))


def test_budget3_fixture_reproduces():
    g = json.load(open(os.path.join(HERE, "golden", "budget3_replay.json")))
    Q, K, V = (np.array(g[x]) for x in ("Q", "K", "V"))
    T = g["prompt"]
    cache, O, c64, outs, victims = run_unit(g["k_heavy"], g["k_local"], Q[:T], K[:T], V[:T],
                                            Q[T:], K[T:], V[T:])
    np.testing.assert_allclose(O, g["prefill_out"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(c64, g["colsum"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(outs, g["decode_out"], rtol=0, atol=1e-15)
    assert victims.tolist() == g["victim_slots"]
    assert [[t, s, p] for (t, s, p, _) in cache.evictions] == g["evicted"]
    assert cache.pos.tolist() == g["final_pos"]
    assert [float(a) for a in cache.acc] == g["final_acc"]
    # Budget 3 with one heavy slot: after every step the window holds the two
    # newest positions and the heavy slot holds the best-scoring older one.
    assert sorted(g["final_pos"])[-2:] == [len(Q) - 2, len(Q) - 1]
