"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Inputs are the seeded synthetic workloads (fixed-length prompts plus a fixed
number of generated tokens, as in the H2O blog's §3.2.2 throughput runs).
Each test prints what it checks before it touches the GPU.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import UnitCache, decode, prefill
from tests.parity import OUT_ATOL, check_units, run_gpu
from workloads import WORKLOADS, Workload, generate, sample_units

pytestmark = pytest.mark.gpu


def announce(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gen(w, seed=0, layer=0):
    return generate(w, seed=seed, layer=layer, device="cuda")


@pytest.mark.parametrize("seed", [0, 1])
def test_tiny_fp32_every_unit(seed):
    w = WORKLOADS[1]
    announce(f"[parity] {w.name} seed={seed} all units")
    x = gen(w, seed)
    r = run_gpu(w, x)
    agg = check_units(w, x, r, range(w.units_per_layer))
    announce(f"[parity] {w.name}: {agg['prefill_out']:.2e} {agg['decode_out']:.2e} ties={len(agg['ties'])}")


@pytest.mark.parametrize("seed", [0, 1])
def test_opt67_layer_fp16_every_unit(seed):
    w = WORKLOADS[2]
    announce(f"[parity] {w.name} seed={seed} all 256 units")
    x = gen(w, seed)
    r = run_gpu(w, x)
    agg = check_units(w, x, r, range(w.units_per_layer))
    announce(f"[parity] {w.name}: prefill {agg['prefill_out']:.2e} decode {agg['decode_out']:.2e} "
             f"colsum {agg['colsum_rel']:.2e} acc {agg['acc_rel']:.2e} ties={len(agg['ties'])}")


SMALL = [
    # ragged prompt (not a multiple of the 64-row tiles), eviction every step
    Workload(90, "ragged-f16", 2, 1, 3, 128, "f16", 100, 40, 10, 7),
    # local window only, d = 64, bf16, heavy keys
    Workload(91, "local-bf16-d64", 1, 1, 5, 64, "bf16", 130, 30, 0, 16, heavy_frac=0.05),
    # cache larger than the prompt: append first, then evict
    Workload(92, "append-f16-d64", 2, 1, 2, 64, "f16", 20, 50, 30, 20),
    # fp32 with d = 128
    Workload(93, "f32-d128", 1, 1, 3, 128, "f32", 33, 20, 5, 3),
    # no prompt, k + 1 > one load batch (general decode loop), streaming fill then evict
    Workload(94, "stream-bf16-k200", 1, 1, 2, 128, "bf16", 0, 300, 100, 100, heavy_frac=0.02),
    # large k with radix-select seeding over several histogram passes, sinks
    Workload(95, "bigk-f16", 1, 1, 2, 128, "f16", 700, 12, 300, 300, heavy_frac=0.05, sinks=4),
    # one-token prompt
    Workload(96, "t1-f32-d64", 1, 1, 1, 64, "f32", 1, 6, 1, 1),
    # prompt of exactly two tiles, bf16 d=128, several heavy hitters
    Workload(97, "tiles-bf16", 1, 1, 4, 128, "bf16", 128, 16, 20, 12, heavy_frac=0.05, sinks=4),
    # fp32 d=128 with k = 300: the split decode (six 56-slot chunks, then the combine)
    Workload(88, "split-f32-d128", 1, 1, 2, 128, "f32", 280, 40, 150, 150),
    # bf16 d=64 with k = 1500: seven 224-slot chunks, then the 512-thread combine
    Workload(89, "split-bf16-d64", 1, 1, 2, 64, "bf16", 1400, 150, 750, 750, heavy_frac=0.05),
    # 256-thread resident decode with eight slots per row group (k + 1 above the 112 or 224
    # slots that seven cover at d = 128 or d = 64)
    Workload(66, "eight-slots-f16-d128", 2, 1, 2, 128, "f16", 180, 30, 60, 60, heavy_frac=0.05),
    Workload(65, "eight-slots-bf16-d64", 1, 1, 2, 64, "bf16", 300, 30, 120, 120, heavy_frac=0.05),
    # 1024-thread resident decode with eight slots per row group (k + 1 > 448), fp16
    Workload(63, "eight-slots-f16-k480", 1, 1, 2, 128, "f16", 540, 30, 240, 240, heavy_frac=0.05),
    # heavy hitters only (k_local = 1: the window holds just the new token), fp16 d=128
    Workload(68, "heavy-only-f16", 2, 1, 2, 128, "f16", 90, 30, 20, 1, heavy_frac=0.05),
    # k = 8192 (the maximum), fp32 d=128: 147 split workgroups per unit (the combine's
    # partial-out loop past its first 64 splits) and 8192 slots (its score loop past 4096)
    Workload(86, "maxk-f32-d128", 1, 1, 1, 128, "f32", 8400, 4, 8000, 192),
    # T + k = 15900 words: the seed keeps the column sums in global memory, not LDS
    # (63 partial column-sum rows; 7700 heavy rows gathered after the selection)
    Workload(87, "unstaged-seed-f16-d64", 1, 1, 1, 64, "f16", 8000, 3, 7700, 200),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_shapes_every_unit(w):
    announce(f"[parity] {w.name}: B={w.batch} H={w.heads} d={w.head_dim} {w.dtype} "
             f"T={w.prompt} n={w.steps} k={w.k_heavy}+{w.k_local}")
    x = gen(w)
    r = run_gpu(w, x)
    agg = check_units(w, x, r, range(w.units_per_layer))
    announce(f"[parity] {w.name}: {agg['prefill_out']:.2e} {agg['decode_out']:.2e} ties={len(agg['ties'])}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_early_keys_dominate(dtype):
    # Keys 0..3 get a large component along a direction every query shares, so each row's
    # largest logits (about 10 above the rest) sit in its first key tile, far from the
    # diagonal: the row max found on the diagonal tile must be raised late in the row.
    w = Workload(98, f"early-dominant-{dtype}", 1, 1, 3, 128, dtype, 300, 8, 20, 20)
    announce(f"[parity] {w.name}: T={w.prompt}, keys 0..3 dominate every row")
    x = gen(w)
    x["q_prompt"][..., 0] += 3.0
    x["k_prompt"][:, :, 0:4, 0] = 40.0
    r = run_gpu(w, x)
    agg = check_units(w, x, r, range(w.units_per_layer))
    announce(f"[parity] {w.name}: prefill {agg['prefill_out']:.2e} colsum {agg['colsum_rel']:.2e}")


BOUNDARY_T = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 191, 255, 256, 257]


@pytest.mark.parametrize("dtype,d", [("f16", 128), ("bf16", 64)])
def test_prefill_tile_boundaries(dtype, d):
    # Prompt lengths around the 32-key (pass 2) and 64-key (pass 1) tiles and the 128-row
    # query blocks of the prefill kernel, each followed by a few decode steps.
    for T in BOUNDARY_T:
        w = Workload(85, f"boundary-{dtype}-d{d}-T{T}", 1, 1, 2, d, dtype, T, 3, 8, 8)
        announce(f"[parity] {w.name}")
        x = gen(w)
        r = run_gpu(w, x)
        check_units(w, x, r, range(w.units_per_layer))


@pytest.mark.parametrize("dtype,d", [("f16", 128), ("bf16", 64), ("f32", 128)])
def test_ragged_batch(dtype, d):
    # Sequences with their own prompt lengths (an empty prompt, one at k, one below it and
    # two longer ones, the longest filling the stored rows), then 24 decode steps, each
    # sequence at its own position.
    from tests.parity import run_gpu_ragged
    lens = [300, 0, 64, 37, 157]
    w = Workload(84, f"ragged-batch-{dtype}-d{d}", len(lens), 1, 3, d, dtype, max(lens), 24,
                 40, 24, heavy_frac=0.05)
    announce(f"[parity] {w.name}: prompt lengths {lens}, k = {w.k}")
    x = gen(w)
    r = run_gpu_ragged(w, x, lens)
    agg = check_units(w, x, r, range(w.units_per_layer), lens=lens)
    assert r["cache"].t_seq.cpu().tolist() == [L + w.steps for L in lens]
    announce(f"[parity] {w.name}: prefill {agg['prefill_out']:.2e} decode {agg['decode_out']:.2e} "
             f"ties={len(agg['ties'])}")


POLICY_CASES = [
    # sinks + window (k_heavy = n_sink = 4), resident decode
    Workload(83, "policy-sinks-f16", 2, 1, 3, 128, "f16", 200, 40, 4, 28, heavy_frac=0.05,
             policy="sinks", policy_param=4),
    # strided (stride 8), resident decode
    Workload(82, "policy-strided-f16", 2, 1, 3, 128, "f16", 200, 40, 12, 20, policy="strided",
             policy_param=8),
    # Top-K by this step's attention, bf16 d=64
    Workload(81, "policy-topk-bf16-d64", 2, 1, 3, 64, "bf16", 200, 40, 24, 16,
             heavy_frac=0.05, policy="topk"),
    # the split decode (k = 300, fp32 d=128) under Top-K and under sinks
    Workload(80, "policy-topk-split-f32", 1, 1, 2, 128, "f32", 280, 30, 150, 150, policy="topk"),
    Workload(79, "policy-sinks-split-bf16", 1, 1, 2, 128, "bf16", 400, 30, 8, 292,
             policy="sinks", policy_param=8),
]


@pytest.mark.parametrize("w", POLICY_CASES, ids=[w.name for w in POLICY_CASES])
def test_eviction_policies(w):
    announce(f"[parity] {w.name}: policy {w.policy}({w.policy_param}), k = {w.k_heavy}+{w.k_local}")
    x = gen(w)
    r = run_gpu(w, x)
    agg = check_units(w, x, r, range(w.units_per_layer))
    announce(f"[parity] {w.name}: prefill {agg['prefill_out']:.2e} decode {agg['decode_out']:.2e} "
             f"ties={len(agg['ties'])}")


@pytest.mark.parametrize("layer", [0, 31])
def test_llama7b_layer_bf16_sampled_units(layer):
    w = WORKLOADS[3]
    announce(f"[parity] {w.name} layer {layer}: full shape, 32 sampled units")
    x = gen(w, layer=layer)
    r = run_gpu(w, x)
    agg = check_units(w, x, r, sample_units(w.units_per_layer, 32, seed=layer))
    announce(f"[parity] layer {layer}: prefill {agg['prefill_out']:.2e} decode "
             f"{agg['decode_out']:.2e} ties={len(agg['ties'])}")
    del x, r
    torch.cuda.empty_cache()


@pytest.mark.parametrize("seed", [0, 1])
def test_opt30b_layer_fp16_sampled_units(seed):
    w = WORKLOADS[4]
    announce(f"[parity] {w.name} seed={seed}: full shape, 32 sampled units")
    x = gen(w, seed)
    r = run_gpu(w, x)
    agg = check_units(w, x, r, sample_units(w.units_per_layer, 32, seed=seed))
    announce(f"[parity] {w.name}: prefill {agg['prefill_out']:.2e} decode {agg['decode_out']:.2e} "
             f"ties={len(agg['ties'])}")


@pytest.mark.parametrize("wid,n_units", [(3, 8), (4, 6)])
def test_e4m3_full_layer_shapes_sampled_units(wid, n_units):
    # The LLaMA-7B and OPT-30B layer shapes with E4M3 slots, in the launch configurations
    # the E4M3 decode timings use (256-thread and 1024-thread resident decode).
    w = WORKLOADS[wid].scaled(slot_format="e4m3")
    announce(f"[parity] {w.name} e4m3 slots: full shape, {n_units} sampled units")
    x = gen(w)
    r = run_gpu(w, x)
    assert r["cache"].k_slots.dtype == torch.float8_e4m3fn
    agg = check_units(w, x, r, sample_units(w.units_per_layer, n_units, seed=wid))
    announce(f"[parity] {w.name} e4m3: prefill {agg['prefill_out']:.2e} decode "
             f"{agg['decode_out']:.2e} ties={len(agg['ties'])}")
    del x, r
    torch.cuda.empty_cache()


def test_determinism_bitwise():
    w = WORKLOADS[2]
    announce(f"[determinism] {w.name} twice")
    x = gen(w)
    a, b = run_gpu(w, x), run_gpu(w, x)
    for key in ("prefill_out", "colsum", "pos0", "acc0", "outs", "victims", "ev_pos", "ev_acc"):
        assert torch.equal(a[key], b[key]), key
    for key in ("k_slots", "v_slots", "slot_pos", "acc_score"):
        assert torch.equal(getattr(a["cache"], key), getattr(b["cache"], key)), key


def test_resume_from_state_is_bitwise_identical():
    from kv_cache_eviction_03_amd import H2OCache
    w = WORKLOADS[2]
    announce(f"[resume] {w.name}: snapshot at step 16, restore into a fresh cache")
    x = gen(w)
    full = run_gpu(w, x)
    c1 = H2OCache(w.batch, w.heads, w.head_dim, w.k_heavy, w.k_local, w.torch_dtype, "cuda",
                  max_prompt=w.prompt)
    c1.reset()
    c1.prefill(x["q_prompt"], x["k_prompt"], x["v_prompt"])
    for i in range(16):
        c1.decode(x["q_dec"][i], x["k_dec"][i], x["v_dec"][i])
    snap = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in c1.state().items()}
    del c1
    c2 = H2OCache(w.batch, w.heads, w.head_dim, w.k_heavy, w.k_local, w.torch_dtype, "cuda")
    c2.load_state(snap)
    for i in range(16, w.steps):
        o = c2.decode(x["q_dec"][i], x["k_dec"][i], x["v_dec"][i])
        assert torch.equal(o, full["outs"][i])
    for key in ("k_slots", "v_slots", "slot_pos", "acc_score"):
        assert torch.equal(getattr(c2, key), getattr(full["cache"], key)), key


def test_resume_ragged_from_state_is_bitwise_identical():
    # A ragged cache's checkpoint carries each sequence's own position (t_seq): a fresh
    # cache restored from it continues the steps exactly as the original run does.
    from kv_cache_eviction_03_amd import H2OCache
    from tests.parity import run_gpu_ragged
    lens = [200, 0, 64, 37, 150]
    w = Workload(53, "resume-ragged-f16", len(lens), 1, 2, 128, "f16", max(lens), 24, 30, 20,
                 heavy_frac=0.05)
    announce(f"[resume] {w.name}: ragged snapshot at step 10, restore into a fresh cache")
    x = gen(w)
    full = run_gpu_ragged(w, x, lens)
    lens_d = torch.tensor(lens, dtype=torch.int32, device="cuda")
    c1 = H2OCache(w.batch, w.heads, w.head_dim, w.k_heavy, w.k_local, w.torch_dtype, "cuda",
                  max_prompt=w.prompt)
    c1.reset()
    c1.prefill_ragged(x["q_prompt"], x["k_prompt"], x["v_prompt"], lens_d)
    for i in range(10):
        c1.decode_ragged(x["q_dec"][i], x["k_dec"][i], x["v_dec"][i])
    snap = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in c1.state().items()}
    assert snap["t_seq"].cpu().tolist() == [L + 10 for L in lens]
    del c1
    c2 = H2OCache(w.batch, w.heads, w.head_dim, w.k_heavy, w.k_local, w.torch_dtype, "cuda")
    c2.load_state(snap)
    for i in range(10, w.steps):
        o = c2.decode_ragged(x["q_dec"][i], x["k_dec"][i], x["v_dec"][i])
        assert torch.equal(o, full["outs"][i]), i
    for key in ("k_slots", "v_slots", "slot_pos", "acc_score"):
        assert torch.equal(getattr(c2, key), getattr(full["cache"], key)), key
    assert c2.t_seq.cpu().tolist() == [L + w.steps for L in lens]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_injected_exact_tie_evicts_the_oldest(dtype):
    from kv_cache_eviction_03_amd import H2OCache
    announce(f"[tie] injected equal scores, {dtype}")
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    d = 64
    c = H2OCache(1, 1, d, 2, 2, tdt, "cuda")
    c.slot_pos.copy_(torch.tensor([[[3, 1, 5, 6]]], dtype=torch.int32))
    c.acc_score.fill_(1.0)
    c.k_slots.fill_(0.25)
    c.v_slots.normal_()
    c.t = 7
    q = torch.randn(1, 1, d, device="cuda").to(tdt)
    kn = torch.full((1, 1, d), 0.25, device="cuda").to(tdt)
    vn = torch.randn(1, 1, d, device="cuda").to(tdt)
    victim = torch.empty(1, 1, dtype=torch.int32, device="cuda")
    evp = torch.empty_like(victim)
    c.decode(q, kn, vn, victim_slot=victim, evicted_pos=evp)
    torch.cuda.synchronize()
    # candidates are positions <= 7 - 2 = 5: {3, 1, 5}, all with equal scores -> oldest (1)
    assert int(victim) == 1 and int(evp) == 1
    assert c.slot_pos.flatten().tolist() == [3, 7, 5, 6]
    # the oracle takes the same decision from the same state
    u = UnitCache(2, 2, d)
    u.pos[:] = [3, 1, 5, 6]
    u.acc[:] = 1.0
    u.K[:] = 0.25
    for p in (3, 1, 5, 6):
        u.hist32[p], u.hist64[p] = np.float32(1.0), 1.0
    _, v = decode(u, 7, q.double().cpu().numpy()[0, 0], kn.double().cpu().numpy()[0, 0],
                  vn.double().cpu().numpy()[0, 0])
    assert v == 1


def test_decode_alone_on_oracle_seeded_cache():
    """Decode kernel by itself: the cache is seeded by uploading the oracle's prefill state."""
    from kv_cache_eviction_03_amd import H2OCache
    w = WORKLOADS[2].scaled(batch=1, heads=8)
    announce(f"[decode-alone] {w.name} 8 heads, oracle-seeded cache")
    x = gen(w)
    dt = w.torch_dtype
    c = H2OCache(1, w.heads, w.head_dim, w.k_heavy, w.k_local, dt, "cuda")
    units = []
    for h in range(w.heads):
        u = UnitCache(w.k_heavy, w.k_local, w.head_dim)
        prefill(u, x["q_prompt"][0, h].double().cpu().numpy(),
                x["k_prompt"][0, h].double().cpu().numpy(), x["v_prompt"][0, h].double().cpu().numpy())
        c.k_slots[0, h].copy_(torch.from_numpy(u.K).to(dt))
        c.v_slots[0, h].copy_(torch.from_numpy(u.V).to(dt))
        c.slot_pos[0, h].copy_(torch.from_numpy(u.pos.astype(np.int32)))
        c.acc_score[0, h].copy_(torch.from_numpy(u.acc))
        units.append(u)
    c.t = w.prompt
    victim = torch.empty(1, w.heads, dtype=torch.int32, device="cuda")
    for i in range(w.steps):
        o = c.decode(x["q_dec"][i], x["k_dec"][i], x["v_dec"][i], victim_slot=victim)
        o, vg = o.double().cpu().numpy(), victim.cpu().numpy()
        for h, u in enumerate(units):
            ref, v = decode(u, w.prompt + i, x["q_dec"][i, 0, h].double().cpu().numpy(),
                            x["k_dec"][i, 0, h].double().cpu().numpy(),
                            x["v_dec"][i, 0, h].double().cpu().numpy(), adopt_victim=int(vg[0, h]))
            assert np.abs(o[0, h] - ref).max() <= OUT_ATOL[w.dtype]
            assert v == vg[0, h]
    for h, u in enumerate(units):
        assert c.slot_pos[0, h].cpu().tolist() == u.pos.tolist()


def test_stream_bf16_fill_then_evict_sampled_heads():
    # The long-streaming shape (4096 slots, no prompt) over the first 6000 steps: 4096
    # fill steps, then an eviction every step, through the split decode.
    w = WORKLOADS[5].scaled(steps=6000)
    announce(f"[parity] {w.name}: k={w.k}, {w.steps} steps, 4 sampled heads")
    x = gen(w)
    r = run_gpu(w, x)
    agg = check_units(w, x, r, [0, 9, 22, 31])
    announce(f"[parity] {w.name}: decode {agg['decode_out']:.2e} acc {agg['acc_rel']:.2e} "
             f"ties={len(agg['ties'])}")


def test_stream_late_window_from_gpu_snapshot():
    # The long-streaming workload in full: the GPU runs the first 995,904 steps, its cache
    # state of three heads is loaded into the oracle, and the next 1024 steps run on both
    # (positions near 2^20, every step an eviction).
    from kv_cache_eviction_03_amd import H2OCache
    from tests.parity import advance_gpu
    w = WORKLOADS[5]
    t0, n = 995_904, 1024
    heads = (0, 13, 31)
    announce(f"[parity] {w.name}: GPU to t = {t0}, then {n} steps on GPU and oracle, heads {heads}")
    x = gen(w)
    c = H2OCache(w.batch, w.heads, w.head_dim, w.k_heavy, w.k_local, w.torch_dtype, "cuda")
    c.reset()
    advance_gpu(c, x, t0)
    torch.cuda.synchronize()
    announce(f"[parity] {w.name}: reached t = {c.t}")
    units = {}
    for h in heads:
        u = UnitCache(w.k_heavy, w.k_local, w.head_dim)
        u.K[:] = c.k_slots[0, h].double().cpu().numpy()
        u.V[:] = c.v_slots[0, h].double().cpu().numpy()
        u.pos[:] = c.slot_pos[0, h].cpu().numpy()
        u.acc[:] = c.acc_score[0, h].cpu().numpy()
        for p_, a in zip(u.pos.tolist(), u.acc.tolist()):
            u.hist32[p_], u.hist64[p_] = np.float32(a), float(a)
        assert int(u.pos.max()) == t0 - 1 and int(u.pos.min()) >= 0
        units[h] = u
    victim = torch.empty(1, w.heads, dtype=torch.int32, device="cuda")
    worst = 0.0
    for t in range(t0, t0 + n):
        o = c.decode(x["q_dec"][t], x["k_dec"][t], x["v_dec"][t], victim_slot=victim)
        o, vg = o.double().cpu().numpy(), victim.cpu().numpy()
        for h, u in units.items():
            ref, v = decode(u, t, x["q_dec"][t, 0, h].double().cpu().numpy(),
                            x["k_dec"][t, 0, h].double().cpu().numpy(),
                            x["v_dec"][t, 0, h].double().cpu().numpy(), adopt_victim=int(vg[0, h]))
            err = float(np.abs(o[0, h] - ref).max())
            assert err <= OUT_ATOL[w.dtype], (t, h, err)
            assert v == vg[0, h]
            worst = max(worst, err)
    for h, u in units.items():
        assert c.slot_pos[0, h].cpu().tolist() == u.pos.tolist()
        ga = c.acc_score[0, h].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(ga - u.acc) <= 1e-4 * np.maximum(np.abs(ga), np.abs(u.acc)) + 1e-30)
    ties = sum(len(u.ties) for u in units.values())
    announce(f"[parity] {w.name}: late window decode {worst:.2e} ties={ties}")
    del x, c
    torch.cuda.empty_cache()


# More than 1024 units with 16-bit slots and k + 1 <= 7 row groups' worth take the
# two-phase decode, whose 256-thread form decides (scores, argmin, bookkeeping) while the
# V rows are in flight: filling from an empty cache (the append path), short prompts,
# every policy, d = 64, k_local = 1 with all 112 slots used, and a ragged batch.
TWO_PHASE = [
    (Workload(900, "tp-fill-f16", 33, 1, 32, 128, "f16", 0, 150, 52, 52), None),
    (Workload(901, "tp-short-bf16", 33, 1, 32, 128, "bf16", 40, 120, 52, 52), None),
    (Workload(902, "tp-sinks-f16", 33, 1, 32, 128, "f16", 300, 60, 52, 52, policy="sinks",
              policy_param=4, sinks=4), None),
    (Workload(903, "tp-strided-bf16", 33, 1, 32, 128, "bf16", 300, 60, 52, 52,
              policy="strided", policy_param=3), None),
    (Workload(904, "tp-topk-f16", 33, 1, 32, 128, "f16", 300, 60, 52, 52, policy="topk"), None),
    (Workload(905, "tp-d64-bf16", 65, 1, 16, 64, "bf16", 400, 80, 150, 60, heavy_frac=0.05), None),
    (Workload(906, "tp-k1-f16", 33, 1, 32, 128, "f16", 200, 40, 110, 1), None),
    (Workload(907, "tp-ragged-bf16", 40, 1, 32, 128, "bf16", 300, 60, 52, 52),
     [300] + [int(v) for v in np.random.default_rng(5).integers(0, 301, size=39)]),
]


@pytest.mark.parametrize("w,lens", TWO_PHASE, ids=[w.name for w, _ in TWO_PHASE])
def test_two_phase_decode_over_1024_units(w, lens):
    from tests.parity import run_gpu_ragged
    assert w.batch * w.heads > 1024
    announce(f"[parity] {w.name}: units={w.batch * w.heads} k={w.k_heavy}+{w.k_local} "
             f"T={w.prompt} n={w.steps} {w.policy} lens={'ragged' if lens else 'padded'}")
    x = generate(w, seed=3, device="cuda")
    r = run_gpu(w, x) if lens is None else run_gpu_ragged(w, x, lens)
    agg = check_units(w, x, r, sample_units(w.units_per_layer, 24, seed=w.id), lens=lens)
    announce(f"[parity] {w.name}: prefill {agg['prefill_out']:.2e} decode {agg['decode_out']:.2e} "
             f"ties={len(agg['ties'])}")


def test_fp32_long_prompts_with_sink_keys():
    # fp32 inputs, prompts of 1029 and up to 1218 keys with four sink keys each: over that
    # many keys, with a few dominating, an fp32 running sum of the prefill's softmax drifts
    # past the 1e-5 output bound (1.3e-5 and 1.7e-5 were seen on these two cases); the
    # fp64 running sum holds it. One padded case and one ragged batch, both every unit.
    from tests.parity import run_gpu_ragged
    w = Workload(1211, "f32-long-sinks", 1, 1, 1, 64, "f32", 1029, 37, 294, 57, sinks=4,
                 policy="sinks", policy_param=0)
    announce(f"[parity] {w.name}: T={w.prompt} d={w.head_dim} k={w.k_heavy}+{w.k_local}")
    x = generate(w, seed=11, device="cuda")
    r = run_gpu(w, x)
    agg = check_units(w, x, r, range(w.units_per_layer))
    announce(f"[parity] {w.name}: prefill {agg['prefill_out']:.2e} decode {agg['decode_out']:.2e}")
    w = Workload(201, "f32-long-ragged", 3, 1, 2, 128, "f32", 1218, 42, 973, 60, sinks=4)
    lens = [1218, 1045, 708]
    announce(f"[parity] {w.name}: lens={lens} d={w.head_dim} k={w.k_heavy}+{w.k_local}")
    x = generate(w, seed=12, device="cuda")
    r = run_gpu_ragged(w, x, lens)
    agg = check_units(w, x, r, range(w.units_per_layer), lens=lens)
    announce(f"[parity] {w.name}: prefill {agg['prefill_out']:.2e} decode {agg['decode_out']:.2e}")


def test_prefill_exact_ties_keep_the_newest():
    # Dead keys point against every query, so their column sums underflow to exactly 0
    # on both sides; k_heavy exceeds the live candidates, so the heavy cutoff falls
    # among exact ties and the newest dead positions must be the ones kept.
    w = Workload(98, "ties-f16", 1, 1, 2, 128, "f16", 64, 8, 20, 4)
    announce(f"[parity] {w.name}: exact zero column sums at the heavy cutoff")
    g = torch.Generator(device="cpu").manual_seed(98)
    N = w.prompt + w.steps
    qrow = torch.full((w.head_dim,), 0.5)
    Q = qrow.expand(N, w.batch, w.heads, w.head_dim).clone()
    K = torch.randn(N, w.batch, w.heads, w.head_dim, generator=g) * 0.5
    V = torch.randn(N, w.batch, w.heads, w.head_dim, generator=g)
    live = {0, 3, 7, 12, 20, 21, 33, 40, 47, 55}          # all other prompt candidates die
    for j in range(w.prompt - w.k_local):
        if j not in live:
            K[j] = -100.0 * qrow
    x = {}
    for name, full in (("q", Q), ("k", K), ("v", V)):
        full = full.to(w.torch_dtype).cuda()
        x[f"{name}_prompt"] = full[:w.prompt].permute(1, 2, 0, 3).contiguous()
        x[f"{name}_dec"] = full[w.prompt:].contiguous()
    r = run_gpu(w, x)
    cs = r["colsum"][0, 0].cpu()
    dead = [j for j in range(w.prompt - w.k_local) if j not in live]
    assert bool((cs[dead] == 0).all())
    kept = sorted(int(p) for p in r["pos0"][0, 0].cpu() if p >= 0)
    assert kept == sorted(sorted(live) + dead[-10:] + list(range(w.prompt - w.k_local, w.prompt)))
    check_units(w, x, r, range(w.units_per_layer))


# E4M3 slots (the oracle's reading R14): every row that enters a slot is stored as FP8 E4M3
# codes; the codes must match the oracle's byte for byte and the outputs its attention over
# the read-back values.
E4M3_CASES = [
    # resident decode (256 threads), unit scales
    Workload(78, "e4m3-f16-d128", 2, 1, 3, 128, "f16", 200, 40, 24, 16, heavy_frac=0.05,
             slot_format="e4m3"),
    # bf16 d=64, scales that are not powers of two
    Workload(77, "e4m3-bf16-d64-scaled", 2, 1, 3, 64, "bf16", 200, 40, 24, 16, heavy_frac=0.05,
             slot_format="e4m3", k_scale=0.37, v_scale=1.9),
    # scales so small that a few percent of the elements saturate at +-448
    Workload(76, "e4m3-f16-saturating", 2, 1, 2, 128, "f16", 150, 30, 20, 12,
             heavy_frac=0.05, slot_format="e4m3", k_scale=0.004, v_scale=0.003),
    # a prompt shorter than k (every position kept) that the decode steps then fill and
    # overflow, and an empty prompt
    Workload(75, "e4m3-bf16-fill", 2, 1, 2, 128, "bf16", 10, 50, 20, 20, slot_format="e4m3",
             k_scale=0.5, v_scale=0.25),
    Workload(74, "e4m3-f16-empty-prompt", 1, 1, 3, 64, "f16", 0, 40, 12, 12,
             slot_format="e4m3"),
    # the 1024-thread resident decode with seven slots per row group (k = 300), and the
    # split decode (k = 600), with Top-K
    Workload(73, "e4m3-f16-k300", 1, 1, 2, 128, "f16", 360, 30, 150, 150, heavy_frac=0.05,
             slot_format="e4m3", k_scale=0.75, v_scale=0.6),
    # the 256-thread resident decode with eight slots per row group (k + 1 > 112)
    Workload(64, "e4m3-f16-k120", 2, 1, 2, 128, "f16", 180, 30, 60, 60, heavy_frac=0.05,
             slot_format="e4m3"),
    # the 1024-thread resident decode with eight slots per row group (k + 1 > 448)
    Workload(67, "e4m3-f16-k480", 1, 1, 2, 128, "f16", 540, 30, 240, 240, heavy_frac=0.05,
             slot_format="e4m3"),
    Workload(72, "e4m3-bf16-split", 1, 1, 2, 128, "bf16", 700, 30, 300, 300, heavy_frac=0.05,
             slot_format="e4m3", k_scale=1.3),
    Workload(71, "e4m3-f16-split-topk", 1, 1, 2, 128, "f16", 650, 24, 320, 280,
             slot_format="e4m3", policy="topk"),
]


@pytest.mark.parametrize("w", E4M3_CASES, ids=[w.name for w in E4M3_CASES])
def test_e4m3_slots(w):
    announce(f"[parity] {w.name}: E4M3 slots, scales {w.k_scale}/{w.v_scale}, "
             f"k = {w.k_heavy}+{w.k_local}")
    x = gen(w)
    r = run_gpu(w, x)
    assert r["cache"].k_slots.dtype == torch.float8_e4m3fn
    agg = check_units(w, x, r, range(w.units_per_layer))
    announce(f"[parity] {w.name}: prefill {agg['prefill_out']:.2e} decode {agg['decode_out']:.2e} "
             f"ties={len(agg['ties'])}")


def test_e4m3_ragged_batch():
    from tests.parity import run_gpu_ragged
    lens = [120, 0, 33, 64]
    w = Workload(70, "e4m3-ragged-f16", len(lens), 1, 2, 128, "f16", max(lens), 20, 24, 16,
                 heavy_frac=0.05, slot_format="e4m3", k_scale=0.8, v_scale=1.1)
    announce(f"[parity] {w.name}: prompt lengths {lens}")
    x = gen(w)
    r = run_gpu_ragged(w, x, lens)
    check_units(w, x, r, range(w.units_per_layer), lens=lens)


def _all_finite_half(dtype):
    bits = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16)
    x = bits.view(torch.float16 if dtype == "f16" else torch.bfloat16)
    return x[torch.isfinite(x)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 0.37])
def test_e4m3_quantisation_of_every_half_value(dtype, scale):
    # Every finite fp16 / bf16 value enters a slot once, as the new token of a decode step
    # on an empty cache (it takes slot 0): the codes must equal the oracle's.
    from kv_cache_eviction_03_amd import H2OCache
    from oracle import quantize_row
    vals = _all_finite_half(dtype)
    d = 128
    units = (vals.numel() + d - 1) // d
    pad = units * d - vals.numel()
    row = torch.cat([vals, torch.zeros(pad, dtype=vals.dtype)]).reshape(1, units, d)
    announce(f"[parity] e4m3 quantisation: {vals.numel()} finite {dtype} values, scale {scale}")
    dev = "cuda"
    tdt = row.dtype
    c = H2OCache(1, units, d, 2, 2, tdt, dev, slot_format="e4m3", k_scale=scale,
                 v_scale=scale)
    c.reset()
    kn = row.to(dev)
    vn = row.flip(-1).contiguous().to(dev)
    q = torch.zeros_like(kn)
    c.decode(q, kn, vn)
    torch.cuda.synchronize()
    gk = c.k_slots[0, :, 0].view(torch.uint8).cpu().numpy()
    gv = c.v_slots[0, :, 0].view(torch.uint8).cpu().numpy()
    ek, _ = quantize_row(row.double().numpy().reshape(-1), scale)
    ev, _ = quantize_row(row.flip(-1).double().numpy().reshape(-1), scale)
    assert np.array_equal(gk.reshape(-1), ek), \
        f"{int((gk.reshape(-1) != ek).sum())} K codes differ"
    assert np.array_equal(gv.reshape(-1), ev), \
        f"{int((gv.reshape(-1) != ev).sum())} V codes differ"
    assert c.slot_pos[0, :, 0].cpu().tolist() == [0] * units
