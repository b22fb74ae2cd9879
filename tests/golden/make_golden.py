"""Writes tests/golden/budget3_replay.json by calling only the oracle.

The H2O blog (ttsmallhot.github.io), §2.2, illustrates the method with a cache
budget of 3 in its Figure 3; the figure was an image and its values are not in
the text, so no page value exists to store. This fixture uses the same budget
(k_heavy = 1, k_local = 2) on a tiny input of multiples of 1/8 (exact in text)
and records what the oracle computes. It is a regression lock on the oracle,
not an independent pin: the independent pins are in test_oracle_pins.py.

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle import run_unit  # noqa: E402

T, N, D, KH, KL = 4, 10, 2, 1, 2


def inputs():
    rng = np.random.default_rng(2023)
    x = np.round(rng.standard_normal((3, N, D)) * 8) / 8
    return x[0], x[1], x[2]


def compute():
    Q, K, V = inputs()
    cache, O, c64, outs, victims = run_unit(KH, KL, Q[:T], K[:T], V[:T], Q[T:], K[T:], V[T:])
    return {
        "k_heavy": KH, "k_local": KL, "prompt": T, "steps": N - T,
        "Q": Q.tolist(), "K": K.tolist(), "V": V.tolist(),
        "prefill_out": O.tolist(), "colsum": c64.tolist(),
        "decode_out": outs.tolist(), "victim_slots": victims.tolist(),
        "evicted": [[int(t), int(s), int(p)] for (t, s, p, _) in cache.evictions],
        "final_pos": cache.pos.tolist(), "final_acc": [float(a) for a in cache.acc],
    }


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "budget3_replay.json")
    data = compute()
    with open(out, "w") as f:
        f.write("{\n" + ",\n".join(f" {json.dumps(k)}: {json.dumps(v)}" for k, v in data.items())
                + "\n}\n")
    print("wrote", out)
