"""GPU parity over a seeded sweep of small random configurations.

The fixed cases elsewhere each aim at one code path; this sweep draws shapes,
budgets, dtypes, policies and slot formats together from one seeded generator,
so that combinations nobody wrote down by hand (a prompt that ends one row into
a tile, a budget split with k_heavy = 0, a sinks count above k_heavy, E4M3 slots
on a cache that only ever appends, a split decode under a position policy) meet
the oracle too. Every unit of every
configuration is compared, prefill outputs, column sums, slots and every decode
step, with the same tolerances as the fixed cases.
"""
import sys

import numpy as np
import pytest

from tests.parity import check_units, run_gpu
from workloads import Workload, generate

N_CONFIGS = 64
N_WIDE = 16
# Input seed of the sweep's workloads: the generator seed is (seed * 100 + id) * 1000 + layer,
# so seeds 7 and 8 keep the sweep's draws apart from the fixed cases' (seeds 0 and 1).
SWEEP_SEED = 7
RAGGED_SEED = 8
WIDE_SEED = 9


def sweep_configs(n=N_CONFIGS, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = str(rng.choice(["f16", "bf16", "f32"], p=[0.4, 0.4, 0.2]))
        d = int(rng.choice([64, 128]))
        k_local = int(rng.integers(1, 65))
        k_heavy = int(rng.choice([0, int(rng.integers(1, 33)), int(rng.integers(33, 321)),
                                  int(rng.integers(321, 1001))], p=[0.15, 0.4, 0.33, 0.12]))
        k = k_heavy + k_local
        shape = rng.random()
        if shape < 0.1:
            T = 0                                   # empty prompt: the decode fills the cache
        elif shape < 0.3:
            T = int(rng.integers(1, k + 1))         # every prompt position kept
        else:
            T = int(rng.integers(k + 1, k + 701))   # the seed selects
        policy = str(rng.choice(["h2o", "sinks", "strided", "topk"], p=[0.55, 0.15, 0.15, 0.15]))
        param = {"h2o": 0, "topk": 0, "sinks": int(rng.integers(0, 9)),
                 "strided": int(rng.integers(1, 17))}[policy]
        e4m3 = dtype != "f32" and rng.random() < 0.25
        kw = dict(heavy_frac=float(rng.choice([0.0, 0.05])), sinks=int(rng.choice([0, 4])),
                  policy=policy, policy_param=param)
        if e4m3:
            kw.update(slot_format="e4m3", k_scale=float(rng.uniform(0.2, 2.0)),
                      v_scale=float(rng.uniform(0.2, 2.0)))
        out.append(Workload(20 + i, f"sweep{i:02d}", int(rng.integers(1, 3)), 1,
                            int(rng.integers(1, 4)), d, dtype, T, int(rng.integers(1, 61)),
                            k_heavy, k_local, **kw))
    return out


CONFIGS = sweep_configs()


def wide_configs(n=N_WIDE, seed=2028):
    """Longer runs than sweep_configs: prompts up to k + 3000 (at most 6000), up to 200
    decode steps, caches up to 4000 heavy slots (the split decode) and heavier key
    injection, the regime where an fp32 running sum over a thousand keys once drifted
    past its bound."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = str(rng.choice(["f16", "bf16", "f32"], p=[0.4, 0.4, 0.2]))
        d = int(rng.choice([64, 128]))
        k_local = int(rng.integers(1, 257))
        k_heavy = int(rng.choice([0, int(rng.integers(1, 200)), int(rng.integers(200, 1200)),
                                  int(rng.integers(1200, 4000))], p=[0.1, 0.35, 0.35, 0.2]))
        k = k_heavy + k_local
        T = int(rng.choice([0, int(rng.integers(1, k + 1)), int(rng.integers(k + 1, k + 3000))],
                           p=[0.05, 0.2, 0.75]))
        policy = str(rng.choice(["h2o", "sinks", "strided", "topk"], p=[0.55, 0.15, 0.15, 0.15]))
        param = {"h2o": 0, "topk": 0, "sinks": int(rng.integers(0, 9)),
                 "strided": int(rng.integers(1, 17))}[policy]
        kw = dict(heavy_frac=float(rng.choice([0.0, 0.05, 0.1])), sinks=int(rng.choice([0, 4])),
                  policy=policy, policy_param=param)
        if dtype != "f32" and rng.random() < 0.25:
            kw.update(slot_format="e4m3", k_scale=float(rng.uniform(0.2, 2.0)),
                      v_scale=float(rng.uniform(0.2, 2.0)))
        out.append(Workload(300 + i, f"wide{i:02d}", int(rng.integers(1, 3)), 1,
                            int(rng.integers(1, 3)), d, dtype, min(T, 6000),
                            int(rng.integers(1, 201)), k_heavy, k_local, **kw))
    return out


WIDE = wide_configs()


def test_sweep_is_fixed_and_valid():
    """The sweep is a pure function of its seed and stays inside the library's limits."""
    again = sweep_configs()
    assert again == CONFIGS
    for w in CONFIGS:
        assert w.k_local >= 1 and 1 <= w.k <= 8192
        assert w.slot_format == "input" or w.dtype != "f32"
    # the draw reaches the paths it is meant to mix
    assert any(w.prompt == 0 for w in CONFIGS)
    assert any(0 < w.prompt <= w.k for w in CONFIGS)
    assert any(w.k_heavy == 0 for w in CONFIGS)
    assert any(w.slot_format == "e4m3" for w in CONFIGS)
    assert {w.policy for w in CONFIGS} == {"h2o", "sinks", "strided", "topk"}
    # caches past one workgroup's reach at d = 128 (split decode)
    assert any(w.k + 1 > 511 and w.head_dim == 128 for w in CONFIGS)
    assert wide_configs() == WIDE
    for w in WIDE:
        assert w.k_local >= 1 and 1 <= w.k <= 8192 and w.prompt <= 6000
        assert w.slot_format == "input" or w.dtype != "f32"
    assert any(w.dtype == "f32" and w.prompt > 1000 for w in WIDE)
    assert any(w.k + 1 > 511 and w.head_dim == 128 for w in WIDE)


@pytest.mark.gpu
@pytest.mark.parametrize("w", CONFIGS, ids=[w.name for w in CONFIGS])
def test_random_configuration_every_unit(w):
    print(f"[sweep] {w.name}: B={w.batch} H={w.heads} d={w.head_dim} {w.dtype} T={w.prompt} "
          f"n={w.steps} k={w.k_heavy}+{w.k_local} {w.policy}({w.policy_param}) "
          f"{w.slot_format} heavy_frac={w.heavy_frac} sinks={w.sinks}", flush=True)
    sys.stdout.flush()
    x = generate(w, seed=SWEEP_SEED, device="cuda")
    r = run_gpu(w, x)
    agg = check_units(w, x, r, range(w.units_per_layer))
    print(f"[sweep] {w.name}: prefill {agg['prefill_out']:.2e} decode {agg['decode_out']:.2e} "
          f"ties={len(agg['ties'])}", flush=True)


@pytest.mark.gpu
@pytest.mark.parametrize("w", WIDE, ids=[w.name for w in WIDE])
def test_wide_random_configuration_every_unit(w):
    print(f"[sweep] {w.name}: B={w.batch} H={w.heads} d={w.head_dim} {w.dtype} T={w.prompt} "
          f"n={w.steps} k={w.k_heavy}+{w.k_local} {w.policy}({w.policy_param}) "
          f"{w.slot_format} heavy_frac={w.heavy_frac} sinks={w.sinks}", flush=True)
    sys.stdout.flush()
    x = generate(w, seed=WIDE_SEED, device="cuda")
    r = run_gpu(w, x)
    agg = check_units(w, x, r, range(w.units_per_layer))
    print(f"[sweep] {w.name}: prefill {agg['prefill_out']:.2e} decode {agg['decode_out']:.2e} "
          f"ties={len(agg['ties'])}", flush=True)


def ragged_configs(n=16, seed=2027):
    """Ragged batches: per-sequence prompt lengths in [0, T_max], drawn with the rest."""
    rng = np.random.default_rng(seed)
    out = []
    for i, w in enumerate(sweep_configs(n, seed)):
        B = int(rng.integers(2, 6))
        t_max = max(1, w.prompt)
        lens = [int(v) for v in rng.integers(0, t_max + 1, size=B)]
        lens[int(rng.integers(0, B))] = t_max      # the longest fills the stored rows
        out.append((w.scaled(id=50 + i, name=f"ragged{i:02d}", batch=B, prompt=t_max), lens))
    return out


RAGGED = ragged_configs()


@pytest.mark.gpu
@pytest.mark.parametrize("w,lens", RAGGED, ids=[w.name for w, _ in RAGGED])
def test_random_ragged_batch_every_unit(w, lens):
    from tests.parity import run_gpu_ragged
    print(f"[sweep] {w.name}: lens={lens} H={w.heads} d={w.head_dim} {w.dtype} n={w.steps} "
          f"k={w.k_heavy}+{w.k_local} {w.policy}({w.policy_param}) {w.slot_format}", flush=True)
    sys.stdout.flush()
    x = generate(w, seed=RAGGED_SEED, device="cuda")
    r = run_gpu_ragged(w, x, lens)
    agg = check_units(w, x, r, range(w.units_per_layer), lens=lens)
    assert r["cache"].t_seq.cpu().tolist() == [L + w.steps for L in lens]
    print(f"[sweep] {w.name}: prefill {agg['prefill_out']:.2e} decode {agg['decode_out']:.2e} "
          f"ties={len(agg['ties'])}", flush=True)
