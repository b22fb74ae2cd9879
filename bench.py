"""Throughput of the H2O hot path on one MI355X, as one JSON line.

Workload (the headline): the LLaMA-7B-shaped stack — 32 layers, batch 64, 32 heads,
head_dim 128, bf16 K/V, a 512-token padded prompt plus 1024 generated tokens, k = 52
heavy + 52 local slots per (layer, sequence, head) (20% of the prompt). Inputs are
seeded synthetic draws (5% heavy-hitter keys), generated on the device before timing.

One step = one pass of the whole hot path over the batch: every layer's reset and
prefill (causal attention + column sums + cache seeding), then 1024 model decode
steps of 32 layer launches each (fused attention + score accumulation + masked argmin
+ in-place overwrite). `value` is generated tokens per second of the whole step
(64 * 1024 / step time), the end-to-end token throughput the H2O blog's §3.1.3
defines; the decode-phase and prefill-phase rates are reported beside it.

Timing:
  * each step replays one HIP graph of the 32 layers' reset + prefill, then the decode
    phase as graphs of G model steps each (positions are host arguments, so each graph
    holds its own); HIP events on torch's stream around the timed loop and around each
    phase;
  * roofline: the decode kernel's mean device duration = decode phase time / its 32 * 1024
    launches (graph gaps included: conservative), against its algorithmic bytes;
  * graph replays are checked bit for bit against an eager run of the same step;
  * cpu_baseline: the CPU oracle on 64 sampled (layer, sequence, head) units of the same
    inputs (prefill + 1024 decode steps each), extrapolated to the whole step;
  * opt67_layer: the OPT-6.7B-shaped layer (batch 8, fp16, prompt 512 + 32), whole step
    as one graph, and its decode launch MALL-warm and MALL-cold;
  * prefill_mfma_opt30b: the prefill of the OPT-30B-shaped layer (T = 2048), where
    prefill is MFMA-bound, against the 2.5 PFLOP/s dense fp16 peak;
  * decode_by_workload (+ _e4m3, + cold): the decode kernel at each workload's layer shape;
  * hbm_measured_ceiling / mfma_measured_ceiling: the streaming-read and MFMA-loop probes
    (libh2o_probes.so), plus plain PyTorch read and copy rates;
  * dense_comparator, launch_floor, ragged_step, decode_by_policy: context figures;
  * stream_sustained: the long-streaming workload in full (4096 slots, 2^20 decode steps
    from an empty cache), and its first 4096 + 4 x 65,536 steps again as replays of one
    256-step HIP graph, checked bit for bit against the direct run.
Every timed figure is the median of its repetitions, with the min beside it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published
METRIC = "H2O decode tokens/s at 20% KV budget + % of HBM roofline (prefill % MFMA peak)"

# HBM bytes per decode launch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of this
# script, scaled by the same counters on a plain 512 MiB copy (`--copy-probe`), per
# workload. They describe one build of the decode kernel: the hash of its sources is
# recorded with them, and a figure is reported only while the sources still match.
DECODE_SOURCES = ("kv_cache_eviction_03_amd/csrc/decode.hip",
                  "kv_cache_eviction_03_amd/csrc/h2o_device.hpp")
DECODE_TRAFFIC = {
    "opt-6.7b-layer-fp16": {"sha256": "a35bb581cf7bcdd20fbf300cb44b9fb7afe961bb168e44be80e2bfc2d0e04c1d",
                            "read_bytes": 14175279, "write_bytes": 376832},
    "llama-7b-stack-bf16": {"sha256": "a35bb581cf7bcdd20fbf300cb44b9fb7afe961bb168e44be80e2bfc2d0e04c1d",
                            "read_bytes": 113000816, "write_bytes": 3015295},
}


def decode_sources_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def decode_traffic(workload: str):
    t = DECODE_TRAFFIC.get(workload)
    if t is None or t["sha256"] is None or t["sha256"] != decode_sources_hash():
        return None
    return t["read_bytes"] + t["write_bytes"]


def stats(times):
    """Median and min of a list of per-call times (the figure is the median)."""
    import statistics
    return statistics.median(times), min(times)


def replay_times(g, reps, per, before=None):
    """Per-call times (us) of `reps` replays of graph g, each divided by `per` calls, with
    HIP events on torch's current stream; `before` runs (untimed) ahead of each replay."""
    import torch
    out = []
    for _ in range(reps):
        if before is not None:
            before()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        out.append(1e3 * a.elapsed_time(b) / per)
    return out


def decode_bytes_per_unit(w) -> int:
    """Algorithmic HBM bytes of one decode step of one unit (slots of one byte per element
    when they hold E4M3 codes; q, k_new and v_new always in the input dtype)."""
    k, d, s = w.k, w.head_dim, w.elem_bytes
    ss = 1 if w.slot_format == "e4m3" else s
    return 2 * k * d * ss + 12 * k + 3 * d * s + 4 * d + 2 * d * ss + 8


def prefill_flops_per_unit(w) -> int:
    """Causal QK^T and PV, diagonal included: 2 * T(T+1)/2 * 2d."""
    T, d = w.prompt, w.head_dim
    return 2 * T * (T + 1) * d


def prefill_bytes_per_unit(w) -> int:
    T, d, s, k = w.prompt, w.head_dim, w.elem_bytes, w.k
    return 3 * T * d * s + 4 * T * d + 4 * T + 2 * k * d * s + 8 * k


def prefill_mfma_probe(reps=10, warmup=3):
    """Prefill of the OPT-30B-shaped layer (T = 2048, MFMA-bound) timed with HIP events,
    one event pair per h2o_prefill call (median and min over `reps`)."""
    import torch

    from kv_cache_eviction_03_amd import H2OCache
    from workloads import WORKLOADS, generate
    w = WORKLOADS[4].scaled(steps=0)
    x = generate(w, seed=0, device="cuda:0")
    c = H2OCache(w.batch, w.heads, w.head_dim, w.k_heavy, w.k_local, w.torch_dtype, "cuda:0",
                 max_prompt=w.prompt)
    out = torch.empty((w.batch, w.heads, w.prompt, w.head_dim), dtype=torch.float32, device="cuda:0")
    cs = torch.empty((w.batch, w.heads, w.prompt), dtype=torch.float32, device="cuda:0")

    def call():
        c.prefill(x["q_prompt"], x["k_prompt"], x["v_prompt"], out=out, colsum=cs)
    for _ in range(warmup):                     # the shader clock ramps over the first calls
        call()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        torch.cuda.synchronize()
        times.append(1e3 * a.elapsed_time(b))
    us, us_min = stats(times)
    flops = prefill_flops_per_unit(w) * w.units_per_layer
    tflops = flops / (us * 1e-6) / 1e12
    res = {"workload": f"{w.name}: batch {w.batch}, {w.heads} heads, d {w.head_dim}, fp16, "
                       f"prompt {w.prompt}, k = {w.k_heavy}+{w.k_local}",
           "bound": "mfma (arithmetic intensity %.0f flop/B > ridge 312.5)" % (
               prefill_flops_per_unit(w) / prefill_bytes_per_unit(w)),
           "prefill_us": us, "prefill_us_min": us_min, "achieved_tflops": tflops,
           "peak_tflops": MFMA_F16_PEAK_TFLOPS, "frac": tflops / MFMA_F16_PEAK_TFLOPS,
           "frac_at_min": flops / (us_min * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS,
           "prompt_tokens_per_s": w.batch * w.prompt / (us * 1e-6),
           "note": "algorithmic flops 2T(T+1)d per unit over one h2o_prefill call "
                   "(attention + column sums + seeding); median of %d calls" % reps}
    del x, c, out, cs
    torch.cuda.empty_cache()
    return res


def decode_by_policy(n=32, reps=5):
    """The bench layer's decode launch under each eviction ranking (H2O, sinks + window,
    strided, Top-K by current attention), graph-replayed like decode_by_workload; context:
    the ranking changes one fp32 value per candidate, not the bytes moved."""
    import torch

    from kv_cache_eviction_03_amd import H2OCache
    from workloads import WORKLOADS, generate
    dev = "cuda:0"
    w = WORKLOADS[2].scaled(steps=n)
    x = generate(w, seed=0, device=dev)
    out = torch.empty((n, w.batch, w.heads, w.head_dim), dtype=torch.float32, device=dev)
    res = []
    for policy, param in (("h2o", 0), ("sinks", 4), ("strided", 8), ("topk", 0)):
        c = H2OCache(w.batch, w.heads, w.head_dim, w.k_heavy, w.k_local, w.torch_dtype, dev,
                     max_prompt=w.prompt, policy=policy, policy_param=param)
        c.reset()
        c.prefill(x["q_prompt"], x["k_prompt"], x["v_prompt"])
        torch.cuda.synchronize()
        side = torch.cuda.Stream(dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for i in range(n):
                    c.decode(x["q_dec"][i], x["k_dec"][i], x["v_dec"][i], out=out[i])
        torch.cuda.synchronize()

        def refill():
            c.reset()
            c.prefill(x["q_prompt"], x["k_prompt"], x["v_prompt"])
        us, us_min = stats(replay_times(g, reps, n, before=refill))
        res.append({"policy": policy, "policy_param": param, "us_per_launch": us,
                    "us_per_launch_min": us_min})
        del c, g
    del x, out
    torch.cuda.empty_cache()
    return res


def decode_by_workload(ids=(2, 3, 4, 5), n=64, reps=5, slot_format="input"):
    """Decode launches of each workload's layer shape, graph-replayed, timed with HIP events.

    The cache is filled by a prefill of k + 64 tokens (so every step evicts), then n
    decode steps are captured once and replayed; the median (and min) replay's mean per
    launch is reported with the algorithmic bytes of one launch. slot_format "e4m3" runs the same
    shapes with FP8 E4M3 slots (scales 1: the synthetic K/V, heavy-hitter keys included,
    stay far inside the E4M3 range of +-448).
    """
    import torch

    from kv_cache_eviction_03_amd import H2OCache
    from workloads import WORKLOADS, generate
    dev = "cuda:0"
    res = []
    for wid in ids:
        w = WORKLOADS[wid].scaled(prompt=WORKLOADS[wid].k + 64, steps=n, layers=1,
                                  slot_format=slot_format)
        x = generate(w, seed=0, device=dev)
        c = H2OCache(w.batch, w.heads, w.head_dim, w.k_heavy, w.k_local, w.torch_dtype, dev,
                     max_prompt=w.prompt, **w.cache_kw)
        out = torch.empty((n, w.batch, w.heads, w.head_dim), dtype=torch.float32, device=dev)
        c.reset()
        c.prefill(x["q_prompt"], x["k_prompt"], x["v_prompt"])
        torch.cuda.synchronize()
        side = torch.cuda.Stream(dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for i in range(n):
                    c.decode(x["q_dec"][i], x["k_dec"][i], x["v_dec"][i], out=out[i])
        torch.cuda.synchronize()

        def refill():
            c.reset()
            c.prefill(x["q_prompt"], x["k_prompt"], x["v_prompt"])
        us, us_min = stats(replay_times(g, reps, n, before=refill))
        byt = decode_bytes_per_unit(w) * w.units_per_layer
        slots = "e4m3 slots" if slot_format == "e4m3" else f"{w.dtype} slots"
        res.append({"workload": f"{w.name} layer: B {w.batch}, H {w.heads}, d {w.head_dim}, "
                                f"{w.dtype} inputs, {slots}, k = {w.k_heavy}+{w.k_local}",
                    "us_per_launch": us, "us_per_launch_min": us_min,
                    "algorithmic_MB": byt / 1e6, "GBps": byt / (us * 1e-6) / 1e9,
                    "hbm_frac": byt / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                    "hbm_frac_at_min": byt / (us_min * 1e-6) / 1e9 / HBM_PEAK_GBS,
                    "decode_tokens_per_s": w.batch / (us * 1e-6)})
        del x, c, out, g
        torch.cuda.empty_cache()
    return res


def ragged_step(reps=20, seed=7):
    """The bench layer shape with a ragged batch: the 8 sequences' prompt lengths are seeded
    uniform draws in [256, 512] (stored padded to 512 rows, as a summarisation batch would
    be), then 32 generated tokens per sequence, each at its own position. One step = reset +
    h2o_prefill_ragged + 32 h2o_decode_step_ragged (each step's position array precomputed
    on the device), replayed as one HIP graph; compared with the same step padded to 512
    for every sequence (h2o_prefill + h2o_decode_step)."""
    import numpy as np
    import torch

    from kv_cache_eviction_03_amd import H2OCache
    from workloads import WORKLOADS, generate
    dev = "cuda:0"
    w = WORKLOADS[2]
    B, H, d, T, n = w.batch, w.heads, w.head_dim, w.prompt, w.steps
    lens = np.random.default_rng(seed).integers(256, T + 1, size=B).astype(np.int32)
    x = generate(w, seed=0, device=dev)
    lens_d = torch.from_numpy(lens).to(dev)
    t_all = torch.stack([lens_d + i for i in range(n)]).contiguous()   # [n][B]
    out_p = torch.empty((B, H, T, d), dtype=torch.float32, device=dev)
    cs = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    outs = torch.empty((n, B, H, d), dtype=torch.float32, device=dev)
    res = {}
    for mode in ("ragged", "padded"):
        c = H2OCache(B, H, d, w.k_heavy, w.k_local, w.torch_dtype, dev, max_prompt=T)

        def step():
            c.reset()
            if mode == "ragged":
                c.prefill_ragged(x["q_prompt"], x["k_prompt"], x["v_prompt"], lens_d,
                                 out=out_p, colsum=cs)
                for i in range(n):
                    c.decode_ragged(x["q_dec"][i], x["k_dec"][i], x["v_dec"][i], out=outs[i],
                                    t=t_all[i])
            else:
                c.prefill(x["q_prompt"], x["k_prompt"], x["v_prompt"], out=out_p, colsum=cs)
                for i in range(n):
                    c.decode(x["q_dec"][i], x["k_dec"][i], x["v_dec"][i], out=outs[i])
        step()
        torch.cuda.synchronize()
        side = torch.cuda.Stream(dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                step()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        us, us_min = stats(replay_times(g, reps, 1))
        res[mode] = {"us_per_step": us, "us_per_step_min": us_min,
                     "generated_tokens_per_s": B * n / (us * 1e-6)}
        del c, g
    res["workload"] = (f"{w.name} shape with prompt lengths {lens.tolist()} (seeded uniform in "
                       f"[256, {T}], stored padded to {T}), {n} generated tokens each")
    res["prompt_tokens"] = int(lens.sum())
    res["ragged_speedup"] = res["padded"]["us_per_step"] / res["ragged"]["us_per_step"]
    del x, out_p, cs, outs
    torch.cuda.empty_cache()
    return res


def decode_cold(w, replicas=36, reps=5, min_launches=64):
    """A workload's decode step with the Infinity Cache (MALL) out of play.

    `replicas` independent caches, each prefilled from the same prompt, are visited in turn,
    round after round, by one graph of at least `min_launches` decode steps, so consecutive
    steps touch disjoint slot arrays and between two visits of one replica the others sweep
    (replicas - 1) x the step's bytes, more than the 256 MB MALL. Enough launches per graph
    that the replay's own start-up cost is spread as thinly as in a model's decode graph.
    The same launch shape as the warm figure; median and best replay, per step. Each visit
    repeats its replica's position t; that leaves the work per step unchanged.
    """
    import torch

    from kv_cache_eviction_03_amd import H2OCache
    from workloads import generate
    dev = "cuda:0"
    x = generate(w, seed=0, device=dev)
    caches = []
    for _ in range(replicas):
        c = H2OCache(w.batch, w.heads, w.head_dim, w.k_heavy, w.k_local, w.torch_dtype, dev,
                     max_prompt=w.prompt, **w.cache_kw)
        c.reset()
        c.prefill(x["q_prompt"], x["k_prompt"], x["v_prompt"])
        caches.append(c)
    out = torch.empty((w.batch, w.heads, w.head_dim), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(dev)
    g = torch.cuda.CUDAGraph()
    rounds = -(-min_launches // replicas)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(rounds):
                for c in caches:
                    c.decode(x["q_dec"][0], x["k_dec"][0], x["v_dec"][0], out=out)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    med, best = stats(replay_times(g, reps, rounds * replicas))
    byt = decode_bytes_per_unit(w) * w.units_per_layer
    del x, caches, out, g
    torch.cuda.empty_cache()
    slots = "e4m3 slots" if w.slot_format == "e4m3" else f"{w.dtype} slots"
    return {"workload": f"{w.name} layer: B {w.batch}, H {w.heads}, d {w.head_dim}, {w.dtype}, "
                        f"{slots}, k = {w.k_heavy}+{w.k_local}",
            "bound": "hbm", "kernel": "decode step, MALL-cold",
            "achieved": byt / (med * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": byt / (med * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "frac_at_min": byt / (best * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "avg_launch_us": med, "best_launch_us": best,
            "algorithmic_bytes_per_launch": byt, "replicas": replicas,
            "launches_per_replay": rounds * replicas,
            "swept_between_visits_MB": (replicas - 1) * byt / 1e6,
            "duration_from": "HIP events around graph replays of every replica in turn, round "
                             "after round (median replay over its launches)"}


def launch_floor(w, n=32, reps=10):
    """Context: the per-launch time of graph-replayed kernels that do almost nothing (a
    one-element torch fill, one workgroup; the library's h2o_reset of the bench layer,
    104 workgroups writing 0.2 MB), i.e. the dispatch cost any kernel in a graph pays."""
    import torch

    from kv_cache_eviction_03_amd import H2OCache
    dev = "cuda:0"
    x = torch.empty(1, device=dev)
    c = H2OCache(w.batch, w.heads, w.head_dim, w.k_heavy, w.k_local, w.torch_dtype, dev)
    res = {}
    for name, fn in (("fill_1_workgroup_us", x.zero_), ("h2o_reset_us", c.reset)):
        fn()
        torch.cuda.synchronize()
        side = torch.cuda.Stream(dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for _ in range(n):
                    fn()
        torch.cuda.synchronize()
        res[name], res[name.replace("_us", "_us_min")] = stats(replay_times(g, reps, n))
        del g
    del x, c
    return res


def _probe_lib():
    import ctypes
    from kv_cache_eviction_03_amd.build import PROBE_LIB
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is not built; run `python -m kv_cache_eviction_03_amd.build`")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.hbm_read_probe.restype = ctypes.c_int
    lib.mfma_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.mfma_probe.restype = ctypes.c_int
    lib.mfma_probe_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.mfma_probe_flops.restype = ctypes.c_double
    lib.lds_bank_probe.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.lds_bank_probe.restype = ctypes.c_int
    lib.issue_overlap_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.issue_overlap_probe.restype = ctypes.c_int
    return lib


def _lds_patterns():
    """(name, mode, 64 per-lane byte offsets or -1) for the LDS probe; mode 0 ds_read_b128,
    1 ds_write_b64, 2 ds_read_b64, 3 ds_read_b64_tr_b16."""
    L = range(64)

    def pair(a, b, addr_b=256):
        o = [-1] * 64
        o[a], o[b] = 0, addr_b
        return o
    pats = [("b128 read, lane*16", 0, [l * 16 for l in L]),
            ("b128 read, lane*256 (one bank quad)", 0, [l * 256 for l in L]),
            ("b128 read, prefill K operand (16 rows of 256 B, chunk ^ row)", 0,
             [(l % 16) * 256 + (((l // 16) ^ (l % 16)) & 15) * 16 for l in L])]
    for x in (128, 192, 256, 272, 4096):
        pats.append((f"b128 read, lane 0 at 0 and lane 1 at {x}", 0, pair(0, 1, x)))
    for k in (2, 3, 4, 8, 12, 15, 16, 20, 24, 28, 32):
        pats.append((f"b128 read, lane 0 at 0 and lane {k} at 256", 0, pair(0, k)))
    pats += [("b64 write, lane*8", 1, [l * 8 for l in L]),
             ("b64 write, lane*256", 1, [l * 256 for l in L])]
    for x in (64, 128):
        pats.append((f"b64 write, lane 0 at 0 and lane 1 at {x}", 1, pair(0, 1, x)))
    for k in (8, 15, 16, 31, 32):
        pats.append((f"b64 write, lane 0 at 0 and lane {k} at 256", 1, pair(0, k)))
    pats += [("b64 read, lane*8", 2, [l * 8 for l in L]),
             ("b64 transposing read, lane*8", 3, [l * 8 for l in L])]
    return pats


OVERLAP_MODES = {
    0: "16 MFMA 16x16x32",
    1: "16 v_exp_f32",
    2: "16 MFMA + 16 v_exp_f32, interleaved",
    3: "16 MFMA, then 16 v_exp_f32",
    4: "waves 0-3: 16 v_exp_f32; waves 4-7: 16 MFMA",
    5: "16 v_fma_f32",
    6: "16 MFMA + 16 v_fma_f32, interleaved",
    7: "8 MFMA 32x32x16",
    8: "8 MFMA 32x32x16 + 16 v_exp_f32, interleaved",
}


def overlap_probe(iters=2000, blocks=256):
    """s_memtime ticks per iteration of each instruction mix of the issue-overlap probe, one
    workgroup per CU, with one and with two waves per SIMD; waves 0-3 and 4-7 of a
    workgroup are averaged apart (a SIMD's older wave issues first)."""
    import torch
    lib = _probe_lib()
    sink = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    ticks = torch.zeros(blocks * 8, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    rows = []
    for wps in (1, 2):
        for mode, name in OVERLAP_MODES.items():
            ticks.zero_()
            rc = lib.issue_overlap_probe(mode, wps, blocks, iters, sink.data_ptr(),
                                         ticks.data_ptr(), stream)
            if rc != 0:
                raise RuntimeError(f"issue_overlap_probe(mode {mode}) failed: {rc}")
            torch.cuda.synchronize()
            t = ticks[:blocks * 4 * wps].view(blocks, 4 * wps).double() / iters   # one per wave
            row = {"mix": name, "mode": mode, "waves_per_simd": wps,
                   "ticks_waves_0_3": round(float(t[:, :4].mean()), 1)}
            if wps == 2:
                row["ticks_waves_4_7"] = round(float(t[:, 4:].mean()), 1)
            rows.append(row)
    return rows


def lds_probe(iters=100):
    """One dispatch per pattern of _lds_patterns(), in order (the LDS cycle and conflict
    counters come from rocprofv3 --pmc)."""
    import ctypes
    import torch
    lib = _probe_lib()
    offs_dev = torch.empty(64, dtype=torch.int32, device="cuda")
    sink = torch.empty(256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    rows = []
    for name, mode, offs in _lds_patterns():
        arr = (ctypes.c_int * 64)(*offs)
        rc = lib.lds_bank_probe(arr, offs_dev.data_ptr(), mode, iters, sink.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"lds_bank_probe({name!r}) failed: {rc}")
        torch.cuda.synchronize()
        rows.append({"lds_pattern": name, "mode": mode, "wave_instructions": 4 * 4 * iters,
                     "active_lanes": sum(o >= 0 for o in offs)})
    return rows


# Whole 32 KB tiles per workgroup, nontemporal loads, 512 workgroups: the fastest of the
# layouts and grid sizes measured (7.1 TB/s, against 6.2 with ordinary loads and 5.3-5.8
# with grid-stride addressing).
PROBE_LAYOUT = 2
PROBE_BLOCKS = 512


def hbm_ceiling(reps=10):
    """What this HBM delivers to a plain streaming read, MALL-cold (2 GiB, 8x the MALL):
    the hand-written probe of libh2o_probes.so (16-byte nontemporal loads, eight in flight
    per thread, whole 32 KB tiles per workgroup, 512 workgroups of 256 threads), and
    PyTorch's sum (read) and copy (read + write) as context. Median and min of `reps`
    calls, HIP events per call."""
    import torch
    lib = _probe_lib()
    nbytes = 2 << 30
    blocks = PROBE_BLOCKS
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream

    def probe():
        if lib.hbm_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, PROBE_LAYOUT,
                              stream):
            raise RuntimeError("hbm_read_probe refused its sizes or failed to launch")
    half = buf[: nbytes // 8]                   # 1 GiB: a copy reads it and writes 1 GiB
    dst = torch.empty_like(half)
    out = {}
    for name, fn, moved in (("read_probe_GBps", probe, nbytes),
                            ("torch_sum_GBps", lambda: buf.sum(), nbytes),
                            ("torch_copy_GBps", lambda: dst.copy_(half), nbytes)):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        med, mn = stats(ts)
        out[name] = moved / med / 1e9
        out[name.replace("_GBps", "_GBps_max")] = moved / mn / 1e9
    out["read_probe_frac_of_nominal"] = out["read_probe_GBps"] / HBM_PEAK_GBS
    out["note"] = ("2 GiB read by the streaming-read probe and by torch sum; torch copy of "
                   "1 GiB (2 GiB moved); medians (and best) of %d calls" % reps)
    del buf, sink, half, dst
    torch.cuda.empty_cache()
    return out


def read_at_launch_size(nbytes=115_294_208, regions=32, per_replay=64, reps=5):
    """The streaming-read probe at one decode launch's size (default: the LLaMA-7B-shaped
    layer's 115.3 MB; the OPT-6.7B-shaped layer's is 14.4 MB), launched as the stack's decode launches are: back to back in a HIP
    graph, each launch reading one of `regions` distinct regions, so that a region has
    been swept out of the MALL when it is read again. Tried at 1, 2, 4 and 8 passes of
    whole 32 KB tiles per workgroup; the per-launch time includes the launch's start-up
    and tail, the cost any kernel of this size pays."""
    import torch
    lib = _probe_lib()
    tile = 16 * 8 * 256                          # bytes per workgroup per pass
    rows = []
    for passes in (1, 2, 4, 8):
        blocks = max(1, round(nbytes / (passes * tile)))
        size = blocks * passes * tile
        buf = torch.ones(regions * size // 4, dtype=torch.float32, device="cuda:0")
        sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda:0")

        def launch(i):
            base = buf.data_ptr() + (i % regions) * size
            if lib.hbm_read_probe(base, size, sink.data_ptr(), blocks, PROBE_LAYOUT,
                                  torch.cuda.current_stream().cuda_stream):
                raise RuntimeError("hbm_read_probe refused its sizes or failed to launch")
        for i in range(regions):
            launch(i)
        torch.cuda.synchronize()
        side = torch.cuda.Stream("cuda:0")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side), torch.cuda.graph(g, stream=side):
            for i in range(per_replay):
                launch(i)
        torch.cuda.synchronize()
        med, mn = stats(replay_times(g, reps, per_replay))
        rows.append({"workgroups": blocks, "passes": passes, "bytes_per_launch": size,
                     "us_per_launch": med, "us_per_launch_min": mn,
                     "GBps": size / med / 1e3, "frac_of_nominal": size / med / 1e3 / HBM_PEAK_GBS})
        del g, buf, sink
        torch.cuda.empty_cache()
    best = min(rows, key=lambda r: r["us_per_launch"] * nbytes / r["bytes_per_launch"])
    return {"best_GBps": best["GBps"], "best_frac_of_nominal": best["frac_of_nominal"],
            "best_us_at_bytes": best["us_per_launch"] * nbytes / best["bytes_per_launch"],
            "bytes": nbytes, "regions": regions, "launches_per_replay": per_replay,
            "by_shape": rows}


def mfma_ceiling(reps=5, iters=4096):
    """The dense fp16 MFMA rate of a register-only loop (libh2o_probes.so: eight
    independent 16x16x32 accumulation chains per wave, 256-thread workgroups, 8 per CU)."""
    import torch
    lib = _probe_lib()
    blocks = 256 * 8
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream

    def probe():
        if lib.mfma_probe(blocks, iters, out.data_ptr(), stream):
            raise RuntimeError("mfma_probe failed to launch")
    probe()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        probe()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    med, mn = stats(ts)
    flops = lib.mfma_probe_flops(blocks, iters)
    del out
    return {"fp16_TFLOPs": flops / med / 1e12, "fp16_TFLOPs_max": flops / mn / 1e12,
            "frac_of_nominal": flops / med / 1e12 / MFMA_F16_PEAK_TFLOPS,
            "note": f"{blocks} workgroups x 4 waves x {iters} rounds x 8 chains of "
                    f"v_mfma_f32_16x16x32_f16; median (and best) of {reps} launches"}


def decode_cold_by_workload(ids_replicas=((3, 5), (4, 4), (5, 8)), slot_format="input"):
    """MALL-cold decode at the other workloads' layer shapes (cache filled by a k + 64 prompt,
    so every step evicts); between two visits of a replica the others sweep >= 356 MB."""
    from workloads import WORKLOADS
    res = []
    for wid, r in ids_replicas:
        w = WORKLOADS[wid].scaled(prompt=WORKLOADS[wid].k + 64, steps=1, layers=1,
                                  slot_format=slot_format)
        d = decode_cold(w, replicas=r)
        res.append({k: d[k] for k in ("workload", "avg_launch_us", "best_launch_us", "achieved",
                                      "frac", "frac_at_min", "replicas", "launches_per_replay",
                                      "swept_between_visits_MB")})
    return res


def dense_comparator(w, reps=5):
    """Context, not a target: the same decode steps with k = T + n, so nothing is evicted
    (every prompt and generated token stays cached), against the H2O budget k."""
    import torch

    from kv_cache_eviction_03_amd import H2OCache
    from workloads import generate
    dev = "cuda:0"
    n = w.steps
    kd = w.prompt + n
    x = generate(w, seed=0, device=dev)
    c = H2OCache(w.batch, w.heads, w.head_dim, kd - w.k_local, w.k_local, w.torch_dtype, dev,
                 max_prompt=w.prompt)
    out = torch.empty((n, w.batch, w.heads, w.head_dim), dtype=torch.float32, device=dev)
    c.reset()
    c.prefill(x["q_prompt"], x["k_prompt"], x["v_prompt"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(n):
                c.decode(x["q_dec"][i], x["k_dec"][i], x["v_dec"][i], out=out[i])
    torch.cuda.synchronize()

    def refill():
        c.reset()
        c.prefill(x["q_prompt"], x["k_prompt"], x["v_prompt"])
    us, us_min = stats(replay_times(g, reps, n, before=refill))
    del x, c, out, g
    torch.cuda.empty_cache()
    return {"workload": f"{w.name} layer with k = T + n = {kd} (no eviction)",
            "decode_us_per_step": us, "decode_us_per_step_min": us_min,
            "decode_tokens_per_s": w.batch / (us * 1e-6)}


def stream_sustained(window=65536, graph_windows=4, G=256):
    """The long-streaming workload in full: 32 heads, 4096 slots, 2^20 decode steps of
    seeded inputs (2% heavy-hitter keys), one h2o_decode_step call per step through the C
    ABI (t is a host argument, so the steps cannot be one replayed graph). HIP events at
    window boundaries give the device time of the 4096 fill steps and of each 65,536-step
    window after them; the host's own time per enqueued step is reported beside it, to
    show the loop is bound by the GPU, not by the enqueueing.

    Then the same stream through graphs: the ragged entry point takes each step's position
    from device memory, so one HIP graph holds G steps (a gather of the G steps' inputs by
    position, G decode launches, and an add that advances the positions by G) and is
    replayed with no host work per step. It runs the fill and `graph_windows` windows from
    an empty cache, and its final cache state is compared bit for bit with the direct
    run's state at the same step."""
    import ctypes
    import torch
    from kv_cache_eviction_03_amd import H2OCache
    from kv_cache_eviction_03_amd._abi import library
    from workloads import WORKLOADS, generate
    w = WORKLOADS[5]
    dev = "cuda:0"
    x = generate(w, seed=0, device=dev)
    B, H, d, n, k = w.batch, w.heads, w.head_dim, w.steps, w.k
    c = H2OCache(B, H, d, w.k_heavy, w.k_local, w.torch_dtype, dev)
    c.reset()
    out = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    lib = library()
    desc = c.desc()
    dref = ctypes.byref(desc)
    fn = lib.h2o_decode_step
    sb = B * H * d * w.elem_bytes
    q0, k0, v0 = x["q_dec"].data_ptr(), x["k_dec"].data_ptr(), x["v_dec"].data_ptr()
    op, wp, wn = out.data_ptr(), c.workspace.data_ptr(), c.workspace.numel()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    marks = [0, k] + list(range(k + window, n + 1, window))
    if marks[-1] < n:
        marks.append(n)                         # a last, shorter window
    events = {}
    snap_at = k + graph_windows * window
    names = ("k_slots", "v_slots", "slot_pos", "acc_score")
    snap = None
    torch.cuda.synchronize()
    host0 = time.perf_counter()
    t = 0
    for a, b in zip(marks[:-1], marks[1:]):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        events[a] = e
        for t in range(a, b):
            st = fn(dref, t, q0 + t * sb, k0 + t * sb, v0 + t * sb, op, None, wp, wn, sp)
            if st:
                raise RuntimeError(f"h2o_decode_step failed at t = {t}: {lib.h2o_last_error()}")
        if b == snap_at:
            snap = {nm: getattr(c, nm).clone() for nm in names}
    e = torch.cuda.Event(enable_timing=True)
    e.record(stream)
    events[marks[-1]] = e
    host_s = time.perf_counter() - host0
    torch.cuda.synchronize()
    ms = [events[a].elapsed_time(events[b]) for a, b in zip(marks[:-1], marks[1:])]
    step_bytes = decode_bytes_per_unit(w) * w.units_per_layer
    win = [(b - a) * B / (m * 1e-3) for a, b, m in zip(marks[1:-1], marks[2:], ms[1:])]
    us_step = [m * 1e3 / (b - a) for a, b, m in zip(marks[1:-1], marks[2:], ms[1:])]
    steady_steps = marks[-1] - k
    steady_ms = sum(ms[1:])
    full = [r for r, a, b in zip(win, marks[1:-1], marks[2:]) if b - a == window]
    us_full = [u for u, a, b in zip(us_step, marks[1:-1], marks[2:]) if b - a == window]
    res = {
        "workload": f"{w.name}: batch {B}, {H} heads, d {d}, bf16, k = {w.k_heavy}+{w.k_local}, "
                    f"{n} decode steps from an empty cache, 2% heavy-hitter keys",
        "steps_timed": marks[-1],
        "fill_steps": k, "fill_ms": ms[0],
        "windows": len(win), "window_steps": window, "full_windows": len(full),
        "tokens_per_s_sustained": steady_steps * B / (steady_ms * 1e-3),
        "tokens_per_s_window_min": min(full), "tokens_per_s_window_max": max(full),
        "us_per_step_window_min": min(us_full), "us_per_step_window_max": max(us_full),
        "GBps_sustained": step_bytes * steady_steps / (steady_ms * 1e-3) / 1e9,
        "hbm_frac_sustained": step_bytes * steady_steps / (steady_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "host_us_per_step_enqueue": host_s * 1e6 / marks[-1],
        "note": "device time from HIP events at window boundaries (min/max over the full "
                "windows; the sustained rate covers every step after the fill); per step: both "
                "decode launches (partial + combine); algorithmic bytes 2kd·s + 12k + 5d·s + 4d "
                "+ 8 per unit; the host waits on a full launch queue, so its time per step "
                "matches the device's",
    }
    if snap is not None and snap_at % G == 0 and window % G == 0 and k % G == 0:
        res["graph_replayed"] = stream_graph(w, x, snap, snap_at, k, window, G)
    del x, c, out, snap
    torch.cuda.empty_cache()
    return res


def stream_graph(w, x, snap, steps, fill, window, G):
    """The stream's first `steps` decode steps as replays of one G-step HIP graph (see
    stream_sustained), timed per window with HIP events; checked bit for bit against the
    direct run's cache state at the same step."""
    import torch
    from kv_cache_eviction_03_amd import H2OCache
    dev = "cuda:0"
    B, H, d = w.batch, w.heads, w.head_dim
    c = H2OCache(B, H, d, w.k_heavy, w.k_local, w.torch_dtype, dev)
    c.reset()
    tp = torch.arange(G, dtype=torch.int32, device=dev)        # positions of the G steps
    qs, ks, vs = (torch.empty((G, B, H, d), dtype=w.torch_dtype, device=dev) for _ in range(3))
    out = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            torch.index_select(x["q_dec"], 0, tp, out=qs)
            torch.index_select(x["k_dec"], 0, tp, out=ks)
            torch.index_select(x["v_dec"], 0, tp, out=vs)
            for i in range(G):
                c.decode_ragged(qs[i], ks[i], vs[i], out=out, t=tp[i:i + 1])
            tp.add_(G)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    marks = [0, fill] + list(range(fill + window, steps + 1, window))
    ev = []
    for a, b in zip(marks[:-1], marks[1:]):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range((b - a) // G):
            g.replay()
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    for nm in ("k_slots", "v_slots", "slot_pos", "acc_score"):
        if not torch.equal(getattr(c, nm), snap[nm]):
            raise RuntimeError(f"graph-replayed stream diverged from the direct run in {nm}")
    us = [m * 1e3 / window for m in ms[1:]]
    step_bytes = decode_bytes_per_unit(w) * w.units_per_layer
    res = {"steps": steps, "graph_steps": G, "replays": steps // G,
           "fill_ms": ms[0], "windows": len(us),
           "us_per_step_window_min": min(us), "us_per_step_window_max": max(us),
           "tokens_per_s_sustained": (steps - fill) * B / (sum(ms[1:]) * 1e-3),
           "hbm_frac_sustained": step_bytes * (steps - fill) / (sum(ms[1:]) * 1e-3) / 1e9
           / HBM_PEAK_GBS,
           "matches_direct_run": True}
    del g, c, qs, ks, vs, out, tp
    return res


def cpu_baseline(w, units_inputs, total_units, min_seconds=10.0, single_core_units=8):
    """The CPU oracle (as it stands) on sampled units of the headline workload: each unit is
    a prompt plus every decode step of that (layer, sequence, head), independent of all
    others, so the whole step's oracle time is the mean unit time times the number of units
    (extrapolated linearly). units_inputs: host float64 inputs of the sampled units."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import run_unit

    def timed(min_s, sample):
        # Whole passes over the sampled units until about min_s of CPU work has been timed.
        t0 = time.perf_counter()
        passes = 0
        while True:
            for u in sample:
                run_unit(w.k_heavy, w.k_local, u["Qp"], u["Kp"], u["Vp"], u["qd"], u["kd"],
                         u["vd"])
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= min_s or passes >= 50:
                return dt, passes

    def rate(dt, passes, n_units):
        return w.batch * w.steps / (dt / (passes * n_units) * total_units)

    dt, passes = timed(min_seconds, units_inputs)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    few = units_inputs[:single_core_units]
    with threadpool_limits(limits=1):           # the same oracle on one core
        dt1, passes1 = timed(min_seconds / 4, few)
    return {"value": rate(dt, passes, len(units_inputs)), "unit": "tokens/s",
            "cores": int(threads), "kind": "oracle",
            "sample": f"{passes} pass(es) over {len(units_inputs)} sampled (layer, sequence, head) "
                      f"units of {total_units} (prompt {w.prompt} + {w.steps} decode steps each) "
                      f"in {dt:.1f} s, extrapolated linearly to the whole step",
            "extrapolated": True,
            "value_1_core": rate(dt1, passes1, len(few)),
            "sample_1_core": f"{passes1} pass(es) over {len(few)} of those units in {dt1:.1f} s, "
                             f"one BLAS thread, extrapolated to the whole step"}


def opt67_layer(steps, warmup, seed=0, with_cold=True):
    """The OPT-6.7B-shaped layer (batch 8, 32 heads, d 128, fp16, prompt 512 + 32, k = 52 +
    52): one step (reset + prefill + 32 decode steps) replayed as one HIP graph, then the
    same step as two graphs for the phase split; the decode phase's mean per launch is the
    decode kernel's duration (MALL-warm: the 14 MB layer state stays in the Infinity
    Cache), and with_cold adds the MALL-cold launch (36 replicas)."""
    import torch

    from kv_cache_eviction_03_amd import H2OCache
    from workloads import WORKLOADS, generate
    dev = torch.device("cuda:0")
    w = WORKLOADS[2]
    x = generate(w, seed=seed, device=dev)
    B, H, d, T, n = w.batch, w.heads, w.head_dim, w.prompt, w.steps
    units = w.units_per_layer
    cache = H2OCache(B, H, d, w.k_heavy, w.k_local, w.torch_dtype, dev, max_prompt=T)
    out_p = torch.empty((B, H, T, d), dtype=torch.float32, device=dev)
    colsum = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    outs = torch.empty((n, B, H, d), dtype=torch.float32, device=dev)

    def run_prefill():
        cache.reset()
        cache.prefill(x["q_prompt"], x["k_prompt"], x["v_prompt"], out=out_p, colsum=colsum)

    def run_decode():
        for i in range(n):
            cache.decode(x["q_dec"][i], x["k_dec"][i], x["v_dec"][i], out=outs[i])

    run_prefill()
    run_decode()
    torch.cuda.synchronize()
    ref_state = {k: v.clone() for k, v in cache.state().items() if torch.is_tensor(v)}
    ref_outs = outs.clone()
    side = torch.cuda.Stream(dev)
    g_step, g_pre, g_dec = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g_step, stream=side):
            run_prefill()
            run_decode()
        with torch.cuda.graph(g_pre, stream=side):
            run_prefill()
        cache.t = T
        with torch.cuda.graph(g_dec, stream=side):
            run_decode()
    torch.cuda.synchronize()
    for _ in range(warmup):
        g_step.replay()
    torch.cuda.synchronize()
    step_us, step_us_min = stats(replay_times(g_step, steps, 1))

    def check_replay(what):
        for k, v in ref_state.items():
            if not torch.equal(getattr(cache, k), v):
                raise RuntimeError(f"{what} replay diverged from the eager run in {k}")
        if not torch.equal(outs, ref_outs):
            raise RuntimeError(f"{what} replay diverged from the eager run in decode outputs")
    check_replay("opt67 step graph")
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1, e2 in ev:
        e0.record(stream)
        g_pre.replay()
        e1.record(stream)
        g_dec.replay()
        e2.record(stream)
    torch.cuda.synchronize()
    pre_us, pre_us_min = stats([1e3 * a.elapsed_time(b) for a, b, _ in ev])
    dec_us, dec_us_min = stats([1e3 * b.elapsed_time(c) / n for _, b, c in ev])
    check_replay("opt67 phase graph")
    dec_bytes = decode_bytes_per_unit(w) * units
    res = {"workload": f"{w.name}: batch {B}, {H} heads, head_dim {d}, fp16 K/V, prompt {T} + "
                       f"{n} generated, k = {w.k_heavy} heavy + {w.k_local} local slots",
           "us_per_step": step_us, "us_per_step_min": step_us_min,
           "generated_tokens_per_s": B * n / (step_us * 1e-6),
           "prefill_phase_us": pre_us, "prefill_phase_us_min": pre_us_min,
           "prefill_tokens_per_s": B * T / (pre_us * 1e-6),
           "decode_launch_us": dec_us, "decode_launch_us_min": dec_us_min,
           "decode_tokens_per_s": B / (dec_us * 1e-6),
           "roofline_warm": {"bound": "hbm",
                             "kernel": "decode_resident_kernel<_Float16,128,256,false,7,false>",
                             "achieved": dec_bytes / (dec_us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                             "unit": "GB/s",
                             "frac": dec_bytes / (dec_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                             "traffic": decode_traffic(w.name),
                             "algorithmic_bytes_per_launch": dec_bytes,
                             "note": "MALL-warm: the layer's 14 MB decode state stays in the "
                                     "256 MB Infinity Cache between launches"},
           "roofline_prefill": {
               "bound": "hbm (arithmetic intensity %.1f flop/B < ridge 312.5)" % (
                   prefill_flops_per_unit(w) / prefill_bytes_per_unit(w)),
               "mfma_frac": prefill_flops_per_unit(w) * units / (pre_us * 1e-6) / 1e12
               / MFMA_F16_PEAK_TFLOPS,
               "hbm_frac": prefill_bytes_per_unit(w) * units / (pre_us * 1e-6) / 1e9
               / HBM_PEAK_GBS}}
    floor = launch_floor(w)
    above = dec_us - floor["h2o_reset_us"]
    floor["decode_us_above_floor"] = above
    floor["decode_GBps_above_floor"] = dec_bytes / (above * 1e-6) / 1e9 if above > 0 else None
    res["launch_floor"] = floor
    del g_step, g_pre, g_dec, cache, x, out_p, colsum, outs
    torch.cuda.empty_cache()
    if with_cold:
        res["roofline_cold"] = decode_cold(w)
        res["roofline_cold"]["kernel"] = ("decode_resident_kernel<_Float16,128,256,false,7,false>, "
                                          "MALL-cold")
        dense = dense_comparator(w)
        dense["h2o_decode_speedup"] = dense["decode_us_per_step"] / dec_us
        res["dense_comparator"] = dense
    return res


HEADLINE_KERNEL = "decode_resident_kernel<__bf16,128,256,false,7,true>"


def headline_stack(steps, warmup, seed=0, per_graph=64, cpu_units=64, decode_steps=None):
    """The LLaMA-7B-shaped stack end to end (see the module docstring). Returns the result
    fields of the JSON line that describe the headline. decode_steps (profiling runs only)
    shortens the decode phase; every launch is still a cold launch of the same kernel on
    the same layer shape, so per-dispatch counters are those of the full step."""
    import torch

    from kv_cache_eviction_03_amd import H2OStack
    from workloads import WORKLOADS, generate, sample_units
    dev = torch.device("cuda:0")
    w = WORKLOADS[3]
    if decode_steps is not None:
        w = w.scaled(steps=decode_steps)
    B, H, d, T, n, L = w.batch, w.heads, w.head_dim, w.prompt, w.steps, w.layers
    units = w.units_per_layer
    print(f"[bench] headline {w.name}: generating {L} layers' inputs", file=sys.stderr, flush=True)
    xs = [generate(w, seed=seed, layer=l, device=dev) for l in range(L)]
    prompts = [(x["q_prompt"], x["k_prompt"], x["v_prompt"]) for x in xs]
    dec = [(x["q_dec"], x["k_dec"], x["v_dec"]) for x in xs]
    st = H2OStack(L, B, H, d, w.k_heavy, w.k_local, w.torch_dtype, dev, max_prompt=T)
    out_p = torch.empty((B, H, T, d), dtype=torch.float32, device=dev)
    outs = [torch.empty((B, H, d), dtype=torch.float32, device=dev) for _ in range(L)]

    # Eager reference run of one whole step (also warms the kernels up).
    print("[bench] headline: eager reference step", file=sys.stderr, flush=True)
    st.prefill(prompts, out_p)
    for i in range(n):
        st.decode_step(dec, i, outs)
    torch.cuda.synchronize()
    names = ("k_slots", "v_slots", "slot_pos", "acc_score")
    ref = [{nm: getattr(c, nm).clone() for nm in names} for c in st.caches]
    ref_outs = [o.clone() for o in outs]
    ref_prefill = out_p.clone()

    print("[bench] headline: capturing graphs", file=sys.stderr, flush=True)
    g_pre = st.capture_prefill(prompts, out_p)
    g_dec = st.capture_decode_run(dec, T, n, per_graph, outs)
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        g_pre.replay()
        for g in g_dec:
            g.replay()
    torch.cuda.synchronize()

    # Timed loop: exactly `steps` whole steps, events around the loop and each phase.
    print(f"[bench] headline: timing {steps} steps", file=sys.stderr, flush=True)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for e0, e1, e2 in ev:
        e0.record(stream)
        g_pre.replay()
        e1.record(stream)
        for g in g_dec:
            g.replay()
        e2.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_per_step = start.elapsed_time(end) / steps
    pre_ms = [a.elapsed_time(b) for a, b, _ in ev]
    dec_ms = [b.elapsed_time(c) for _, b, c in ev]

    # The replays must reproduce the eager run bit for bit.
    for l, c in enumerate(st.caches):
        for nm in names:
            if not torch.equal(getattr(c, nm), ref[l][nm]):
                raise RuntimeError(f"graph replay diverged from the eager run: layer {l} {nm}")
        if not torch.equal(outs[l], ref_outs[l]):
            raise RuntimeError(f"graph replay diverged from the eager run: layer {l} outputs")
    if not torch.equal(out_p, ref_prefill):
        raise RuntimeError("graph replay diverged from the eager run: prefill output")

    launches = n * L
    dec_launch_us, dec_launch_us_min = stats([1e3 * m / launches for m in dec_ms])
    pre_med, pre_min = stats(pre_ms)
    dec_med, dec_min = stats(dec_ms)
    dec_bytes = decode_bytes_per_unit(w) * units
    dec_gbs = dec_bytes / (dec_launch_us * 1e-6) / 1e9
    pre_flops = prefill_flops_per_unit(w) * units * L
    pre_bytes = prefill_bytes_per_unit(w) * units * L
    res = {
        "value": B * n / (ms_per_step * 1e-3),
        "ms_per_step": ms_per_step,
        "config": {
            "workload": f"{w.name}: {L} layers, batch {B}, {H} heads, head_dim {d}, bf16 K/V, "
                        f"prompt {T} + {n} generated, k = {w.k_heavy} heavy + {w.k_local} local "
                        f"slots per (layer, sequence, head), 5% heavy-hitter keys",
            "step": f"reset + prefill of all {L} layers (one graph), then {n} model decode steps "
                    f"x {L} layer launches ({len(g_dec)} graphs of {per_graph} model steps)",
            "value_is": "generated tokens / step time (prefill + decode)",
            "global_batch": B, "seq_len": T + n, "parallelism": "single GPU",
        },
        "decode_tokens_per_s": B * n / (dec_med * 1e-3),
        "prefill_tokens_per_s": B * T / (pre_med * 1e-3),
        "phase_ms": {"prefill": pre_med, "prefill_min": pre_min,
                     "decode": dec_med, "decode_min": dec_min},
        "roofline": {
            "bound": "hbm", "kernel": HEADLINE_KERNEL,
            "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": dec_gbs / HBM_PEAK_GBS,
            "frac_at_min": dec_bytes / (dec_launch_us_min * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "traffic": decode_traffic(w.name),
            "avg_launch_us": dec_launch_us, "avg_launch_us_min": dec_launch_us_min,
            "algorithmic_bytes_per_launch": dec_bytes,
            "duration_from": f"HIP events around each step's decode phase ({launches} "
                             f"graph-replayed launches), median over the timed steps",
            "note": "every launch reads its layer's slots from HBM: a model step sweeps "
                    f"{decode_bytes_per_unit(w) * units * L / 1e9:.2f} GB, 14x the 256 MB MALL",
        },
        "roofline_prefill": {
            "bound": "hbm (arithmetic intensity %.1f flop/B < ridge 312.5)" % (
                prefill_flops_per_unit(w) / prefill_bytes_per_unit(w)),
            "achieved_tflops": pre_flops / (pre_med * 1e-3) / 1e12,
            "mfma_peak_tflops": MFMA_F16_PEAK_TFLOPS,
            "mfma_frac": pre_flops / (pre_med * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
            "achieved_gbs": pre_bytes / (pre_med * 1e-3) / 1e9,
            "hbm_frac": pre_bytes / (pre_med * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "note": f"prefill phase = {L} x (reset + attention with column sums + seed), "
                    "algorithmic flops 2T(T+1)d and bytes per unit",
        },
        "wall_s_timed_loop": wall,
    }
    # Host copies of the sampled units for the oracle (64 of the L * B * H units, the first
    # and the last always among them).
    flat = sample_units(L * units, cpu_units, seed=seed)
    f = lambda t: t.double().cpu().numpy()
    sample = []
    for u in flat:
        l, r = divmod(u, units)
        b, h = divmod(r, H)
        x = xs[l]
        sample.append({"Qp": f(x["q_prompt"][b, h]), "Kp": f(x["k_prompt"][b, h]),
                       "Vp": f(x["v_prompt"][b, h]), "qd": f(x["q_dec"][:, b, h]),
                       "kd": f(x["k_dec"][:, b, h]), "vd": f(x["v_dec"][:, b, h])})
    del xs, prompts, dec, st, out_p, outs, ref, ref_outs, ref_prefill, g_pre, g_dec
    torch.cuda.empty_cache()
    return res, w, sample, L * units


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--graph-steps", type=int, default=64,
                    help="model decode steps per captured graph of the headline")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the headline step (no extras, no CPU baseline): for profiling")
    ap.add_argument("--profile-decode-steps", type=int, default=None,
                    help="profiling runs only: model decode steps of the headline step (the "
                         "counter runs, which cannot hold 130k profiled dispatches)")
    ap.add_argument("--cpu-units", type=int, default=64,
                    help="sampled units the CPU oracle runs for cpu_baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mfma-probe", action="store_true")
    ap.add_argument("--decode-shapes", action="store_true",
                    help="only time the decode kernel at each workload's layer shape")
    ap.add_argument("--no-decode-shapes", action="store_true")
    ap.add_argument("--decode-cold", action="store_true",
                    help="only the MALL-cold decode launches of every layer shape")
    ap.add_argument("--no-cold", action="store_true")
    ap.add_argument("--no-stream", action="store_true",
                    help="skip the 2^20-step long-streaming run")
    ap.add_argument("--no-ragged", action="store_true",
                    help="skip the ragged-batch step and the policy launches")
    ap.add_argument("--opt67-only", action="store_true",
                    help="only the OPT-6.7B-shaped layer step; print its figures")
    ap.add_argument("--ragged-only", action="store_true",
                    help="only the ragged-batch step and the policy launches")
    ap.add_argument("--stream-only", action="store_true",
                    help="only the 2^20-step long-streaming run; print its figures")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the OPT-30B-shaped prefill; print its figures")
    ap.add_argument("--ceilings-only", action="store_true",
                    help="only the HBM and MFMA probes; print their figures")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 512 MiB device copy (calibrates HBM byte counters)")
    ap.add_argument("--lds-probe", action="store_true",
                    help="only run the LDS access-pattern probe (one dispatch per pattern)")
    ap.add_argument("--overlap-probe", action="store_true",
                    help="only run the MFMA / vector ALU issue-overlap probe")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the H2O path has no cross-GPU exchange; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe:
        n = 512 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 3}))
        return
    if args.lds_probe:
        for r in lds_probe():
            print(json.dumps(r), flush=True)
        return
    if args.overlap_probe:
        for r in overlap_probe():
            print(json.dumps(r), flush=True)
        return
    if args.decode_shapes:
        for r in decode_by_workload():
            print(json.dumps(r), flush=True)
        for r in decode_by_workload(slot_format="e4m3"):
            print(json.dumps(r), flush=True)
        return
    if args.decode_cold:
        from workloads import WORKLOADS
        print(json.dumps(decode_cold(WORKLOADS[2])), flush=True)
        for r in decode_cold_by_workload():
            print(json.dumps(r), flush=True)
        return
    if args.stream_only:
        print(json.dumps(stream_sustained()), flush=True)
        return
    if args.ragged_only:
        print(json.dumps(ragged_step()), flush=True)
        print(json.dumps(decode_by_policy()), flush=True)
        return
    if args.opt67_only:
        print(json.dumps(opt67_layer(max(args.steps, 5), args.warmup)), flush=True)
        return
    if args.prefill_only:
        print(json.dumps(prefill_mfma_probe()), flush=True)
        return
    if args.ceilings_only:
        print(json.dumps({"hbm": hbm_ceiling(), "mfma": mfma_ceiling(),
                          "hbm_read_at_decode_launch_size": read_at_launch_size(),
                          "hbm_read_at_opt67_launch_size": read_at_launch_size(
                              nbytes=14_411_776, regions=36)}), flush=True)
        return

    torch.cuda.set_device(0)
    if args.profile_decode_steps is not None and not args.headline_only:
        raise SystemExit("--profile-decode-steps is for --headline-only profiling runs")
    head, w, sample, total_units = headline_stack(args.steps, args.warmup, seed=args.seed,
                                                  per_graph=args.graph_steps,
                                                  cpu_units=args.cpu_units,
                                                  decode_steps=args.profile_decode_steps)
    result = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
    }
    result.update({k: v for k, v in head.items() if k not in result})
    if not args.headline_only:
        print("[bench] extras", file=sys.stderr, flush=True)
        result["opt67_layer"] = opt67_layer(20, 3, with_cold=not args.no_cold)
        if not args.no_mfma_probe:
            result["prefill_mfma_opt30b"] = prefill_mfma_probe()
        result["hbm_measured_ceiling"] = hbm_ceiling()
        result["hbm_read_at_decode_launch_size"] = read_at_launch_size()
        result["hbm_read_at_opt67_launch_size"] = read_at_launch_size(nbytes=14_411_776,
                                                                      regions=36)
        result["mfma_measured_ceiling"] = mfma_ceiling()
        if not args.no_decode_shapes:
            result["decode_by_workload"] = decode_by_workload()
            result["decode_by_workload_e4m3"] = decode_by_workload(slot_format="e4m3")
            if not args.no_cold:
                result["decode_cold_by_workload"] = decode_cold_by_workload()
                result["decode_cold_by_workload_e4m3"] = decode_cold_by_workload(
                    ((3, 9), (4, 6), (5, 15)), slot_format="e4m3")
        if not args.no_ragged:
            result["ragged_step"] = ragged_step()
            result["decode_by_policy"] = decode_by_policy()
        if not args.no_stream:
            result["stream_sustained"] = stream_sustained()
        if not args.no_cpu_baseline:
            print("[bench] cpu baseline", file=sys.stderr, flush=True)
            result["cpu_baseline"] = cpu_baseline(w, sample, total_units,
                                                  min_seconds=args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
