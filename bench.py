"""Throughput of the H2O hot path on one MI355X, as one JSON line.

Workload: the OPT-6.7B-shaped layer — batch 8, 32 heads, head_dim 128, fp16
K/V, a 512-token padded prompt plus 32 generated tokens, k = 52 heavy + 52
local slots (20% of the prompt). Inputs are seeded synthetic draws, generated
on the device before timing.

One step = one pass of the whole hot path over the batch: reset, prefill
(causal attention + column sums + cache seeding) and 32 decode steps (fused
attention + score accumulation + masked argmin + in-place overwrite). `value`
is generated tokens per second of the whole step (batch * 32 / step time), the
end-to-end token throughput the H2O blog's §3.1.3 defines; the decode-phase
and prefill-phase rates are reported beside it.

Timing:
  * timed loop: each step replays one HIP graph (reset, prefill, the 32 decode
    launches), with HIP events around the loop, on torch's stream;
  * phase split: a second loop replays the step as two graphs (reset+prefill, then
    the 32 decode launches) with HIP events around each phase; the decode phase
    divided by its 32 launches is the decode kernel's mean device duration used for
    the roofline (it agrees with rocprofv3's kernel trace);
  * graph replays are checked bit for bit against an eager run;
  * cpu_baseline: the CPU oracle on the same inputs (all 256 units of one step);
  * prefill_mfma_opt30b: the prefill of the OPT-30B-shaped layer (T = 2048), where
    prefill is MFMA-bound, against the 2.5 PFLOP/s dense fp16 peak;
  * decode_by_workload: the decode kernel at each workload's layer shape (the
    LLaMA-7B layer, the OPT-30B layer, the 4096-slot stream), graph-replayed;
  * roofline_cold: the bench workload's decode launch with the 256 MB Infinity Cache
    out of play (36 replicas of the cache state visited in turn, 519 MB per sweep);
  * dense_comparator: context only, the same decode steps with k = T + n (nothing
    evicted) against the H2O budget;
  * hbm_measured_ceiling: context only, plain PyTorch streaming read and copy rates;
  * launch_floor: context only, the per-launch time of graph-replayed trivial kernels,
    and the decode launch's bandwidth over the time it spends above that floor;
  * ragged_step: the bench layer with seeded prompt lengths in [256, 512] through the
    ragged entry points, against the same batch padded to 512;
  * decode_by_workload_e4m3: the same shapes with FP8 E4M3 slots (half the slot bytes);
  * decode_by_policy: the bench layer's decode launch under each eviction ranking;
  * llama_stack_decode: the LLaMA-7B-shaped model's decode step, 32 layers each with
    its own prefilled cache (3.69 GB of slots per step, far beyond the MALL);
  * stream_sustained: the long-streaming workload in full (4096 slots, 2^20 decode
    steps from an empty cache), device time per 65,536-step window after the fill; then
    (graph_replayed) its first 4096 + 4 x 65,536 steps again as replays of one 256-step
    HIP graph that advances its own positions, checked bit for bit against the direct run.
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

# HBM bytes per decode launch on this workload from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
# runs of this script, scaled by the same counters on a plain 512 MiB copy
# (`--copy-probe`). They describe one build of the decode kernel: the hash of its sources
# is recorded with them, and the figure is reported only while the sources still match.
DECODE_SOURCES = ("kv_cache_eviction_03_amd/csrc/decode.hip",
                  "kv_cache_eviction_03_amd/csrc/h2o_device.hpp")
DECODE_TRAFFIC = {"sha256": "be2177095510c15d554060f1d93eb213918d04261518bacd574c49931b7fd80c",
                  "read_bytes": 14174610, "write_bytes": 376832}


def decode_sources_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def decode_traffic():
    t = DECODE_TRAFFIC
    if t["sha256"] is None or t["sha256"] != decode_sources_hash():
        return None
    return t["read_bytes"] + t["write_bytes"]


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
    """Prefill of the OPT-30B-shaped layer (T = 2048, MFMA-bound) timed with HIP events."""
    import torch

    from kv_cache_eviction_03_amd import H2OCache
    from workloads import WORKLOADS, generate
    w = WORKLOADS[4].scaled(steps=0)
    x = generate(w, seed=0, device="cuda:0")
    c = H2OCache(w.batch, w.heads, w.head_dim, w.k_heavy, w.k_local, w.torch_dtype, "cuda:0",
                 max_prompt=w.prompt)
    out = torch.empty((w.batch, w.heads, w.prompt, w.head_dim), dtype=torch.float32, device="cuda:0")
    cs = torch.empty((w.batch, w.heads, w.prompt), dtype=torch.float32, device="cuda:0")
    for _ in range(warmup):                     # the shader clock ramps over the first calls
        c.prefill(x["q_prompt"], x["k_prompt"], x["v_prompt"], out=out, colsum=cs)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        c.prefill(x["q_prompt"], x["k_prompt"], x["v_prompt"], out=out, colsum=cs)
    b.record()
    torch.cuda.synchronize()
    us = 1e3 * a.elapsed_time(b) / reps
    flops = prefill_flops_per_unit(w) * w.units_per_layer
    tflops = flops / (us * 1e-6) / 1e12
    res = {"workload": f"{w.name}: batch {w.batch}, {w.heads} heads, d {w.head_dim}, fp16, "
                       f"prompt {w.prompt}, k = {w.k_heavy}+{w.k_local}",
           "bound": "mfma (arithmetic intensity %.0f flop/B > ridge 312.5)" % (
               prefill_flops_per_unit(w) / prefill_bytes_per_unit(w)),
           "prefill_us": us, "achieved_tflops": tflops, "peak_tflops": MFMA_F16_PEAK_TFLOPS,
           "frac": tflops / MFMA_F16_PEAK_TFLOPS,
           "prompt_tokens_per_s": w.batch * w.prompt / (us * 1e-6),
           "note": "algorithmic flops 2T(T+1)d per unit over one h2o_prefill call "
                   "(attention + column sums + seeding)"}
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
        best = None
        for _ in range(reps):
            c.reset()
            c.prefill(x["q_prompt"], x["k_prompt"], x["v_prompt"])
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            us = 1e3 * a.elapsed_time(b) / n
            best = us if best is None else min(best, us)
        res.append({"policy": policy, "policy_param": param, "us_per_launch": best})
        del c, g
    del x, out
    torch.cuda.empty_cache()
    return res


def decode_by_workload(ids=(2, 3, 4, 5), n=32, reps=5, slot_format="input"):
    """Decode launches of each workload's layer shape, graph-replayed, timed with HIP events.

    The cache is filled by a prefill of k + 64 tokens (so every step evicts), then n
    decode steps are captured once and replayed; the best replay's mean per launch is
    reported with the algorithmic bytes of one launch. slot_format "e4m3" runs the same
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
        best = None
        for _ in range(reps):
            c.reset()
            c.prefill(x["q_prompt"], x["k_prompt"], x["v_prompt"])
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            us = 1e3 * a.elapsed_time(b) / n
            best = us if best is None else min(best, us)
        byt = decode_bytes_per_unit(w) * w.units_per_layer
        slots = "e4m3 slots" if slot_format == "e4m3" else f"{w.dtype} slots"
        res.append({"workload": f"{w.name} layer: B {w.batch}, H {w.heads}, d {w.head_dim}, "
                                f"{w.dtype} inputs, {slots}, k = {w.k_heavy}+{w.k_local}",
                    "us_per_launch": best, "algorithmic_MB": byt / 1e6,
                    "GBps": byt / (best * 1e-6) / 1e9, "hbm_frac": byt / (best * 1e-6) / 1e9 / HBM_PEAK_GBS,
                    "decode_tokens_per_s": w.batch / (best * 1e-6)})
        del x, c, out, g
        torch.cuda.empty_cache()
    return res


def llama_stack_decode(steps=16, reps=3):
    """The LLaMA-7B-shaped stack in full: 32 layers (batch 64, 32 heads, d 128, bf16,
    k = 52 + 52), each with its own cache prefilled from its own seeded 512-token prompt.
    One decode step of the model runs the 32 layers' decode launches in turn, 3.69 GB of
    slots per step (14x the MALL), so every launch reads its layer's slots from HBM.
    `steps` such steps are captured as one graph; each timed replay starts from the saved
    post-prefill state of every layer."""
    import torch

    from kv_cache_eviction_03_amd import H2OCache
    from workloads import WORKLOADS, generate
    dev = "cuda:0"
    w = WORKLOADS[3].scaled(steps=steps)
    caches, dec, snaps = [], [], []
    for layer in range(w.layers):
        x = generate(w, seed=0, layer=layer, device=dev)
        c = H2OCache(w.batch, w.heads, w.head_dim, w.k_heavy, w.k_local, w.torch_dtype, dev,
                     max_prompt=w.prompt)
        c.reset()
        c.prefill(x["q_prompt"], x["k_prompt"], x["v_prompt"], want_colsum=False)
        caches.append(c)
        dec.append((x["q_dec"], x["k_dec"], x["v_dec"]))
        snaps.append({k: (v.clone() if torch.is_tensor(v) else v) for k, v in c.state().items()})
        del x
    torch.cuda.synchronize()
    out = torch.empty((w.batch, w.heads, w.head_dim), dtype=torch.float32, device=dev)
    side = torch.cuda.Stream(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(steps):
                for c, (q, k, v) in zip(caches, dec):
                    c.decode(q[i], k[i], v[i], out=out)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        for c, st in zip(caches, snaps):
            c.load_state(st)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(1e3 * a.elapsed_time(b) / steps)
    us = sorted(times)[len(times) // 2]
    byt = decode_bytes_per_unit(w) * w.units_per_layer * w.layers
    res = {"workload": f"{w.name}: {w.layers} layers, batch {w.batch}, {w.heads} heads, "
                       f"d {w.head_dim}, bf16, prompt {w.prompt}, k = {w.k_heavy}+{w.k_local}",
           "us_per_model_step": us, "us_per_model_step_best": min(times),
           "us_per_layer_launch": us / w.layers,
           "decode_tokens_per_s": w.batch / (us * 1e-6),
           "algorithmic_GB_per_step": byt / 1e9,
           "GBps": byt / (us * 1e-6) / 1e9, "hbm_frac": byt / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
           "note": f"{steps} model steps (x {w.layers} layer launches) as one graph, median of "
                   f"{reps} replays from the saved post-prefill state; HIP events"}
    del caches, dec, snaps, out, g
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
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        us = 1e3 * a.elapsed_time(b) / reps
        res[mode] = {"us_per_step": us, "generated_tokens_per_s": B * n / (us * 1e-6)}
        del c, g
    res["workload"] = (f"{w.name} shape with prompt lengths {lens.tolist()} (seeded uniform in "
                       f"[256, {T}], stored padded to {T}), {n} generated tokens each")
    res["prompt_tokens"] = int(lens.sum())
    res["ragged_speedup"] = res["padded"]["us_per_step"] / res["ragged"]["us_per_step"]
    del x, out_p, cs, outs
    torch.cuda.empty_cache()
    return res


def decode_cold(w, replicas=36, reps=5):
    """A workload's decode step with the Infinity Cache (MALL) out of play.

    `replicas` independent caches, each prefilled from the same prompt, are visited in turn
    by one graph of `replicas` decode steps, so consecutive steps touch disjoint slot arrays
    and the state swept per replay (replicas x the step's bytes, >= 512 MB) is at least twice
    the 256 MB MALL. The same launch shape as the warm figure; best and median replay, per
    step. Replays repeat each replica's position t; that leaves the work per step unchanged.
    """
    import statistics

    import torch

    from kv_cache_eviction_03_amd import H2OCache
    from workloads import generate
    dev = "cuda:0"
    x = generate(w, seed=0, device=dev)
    caches = []
    for _ in range(replicas):
        c = H2OCache(w.batch, w.heads, w.head_dim, w.k_heavy, w.k_local, w.torch_dtype, dev,
                     max_prompt=w.prompt)
        c.reset()
        c.prefill(x["q_prompt"], x["k_prompt"], x["v_prompt"])
        caches.append(c)
    out = torch.empty((w.batch, w.heads, w.head_dim), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for c in caches:
                c.decode(x["q_dec"][0], x["k_dec"][0], x["v_dec"][0], out=out)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        per.append(1e3 * a.elapsed_time(b) / replicas)
    byt = decode_bytes_per_unit(w) * w.units_per_layer
    best, med = min(per), statistics.median(per)
    del x, caches, out, g
    torch.cuda.empty_cache()
    return {"workload": f"{w.name} layer: B {w.batch}, H {w.heads}, d {w.head_dim}, {w.dtype}, "
                        f"k = {w.k_heavy}+{w.k_local}",
            "bound": "hbm", "kernel": "decode step, MALL-cold",
            "achieved": byt / (med * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": byt / (med * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "avg_launch_us": med, "best_launch_us": best,
            "algorithmic_bytes_per_launch": byt, "replicas": replicas,
            "state_swept_MB": replicas * byt / 1e6,
            "duration_from": "HIP events around graph replays of one launch per replica (median)"}


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
        best = None
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            us = 1e3 * a.elapsed_time(b) / n
            best = us if best is None else min(best, us)
        res[name] = best
        del g
    del x, c
    return res


def hbm_ceiling(reps=10):
    """Context: what plain PyTorch streaming kernels reach on this HBM (MALL-cold sizes):
    a 1 GiB fp32 sum (read) and a 512 MiB copy (read + write). Median of `reps`."""
    import statistics

    import torch
    n = (1 << 30) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty(n // 2, dtype=torch.float32, device="cuda:0")
    out = {}
    for name, fn, nbytes in (("read_GBps", lambda: x.sum(), 4 * n),
                             ("copy_GBps", lambda: y.copy_(x[: n // 2]), 4 * n)):
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
        out[name] = nbytes / statistics.median(ts) / 1e9
    del x, y
    torch.cuda.empty_cache()
    out["note"] = "torch sum over 1 GiB fp32; torch copy of 512 MiB (1 GiB moved); medians"
    return out


def decode_cold_by_workload(ids_replicas=((3, 5), (4, 3), (5, 8))):
    """MALL-cold decode at the other workloads' layer shapes (cache filled by a k + 64 prompt,
    so every step evicts)."""
    from workloads import WORKLOADS
    res = []
    for wid, r in ids_replicas:
        w = WORKLOADS[wid].scaled(prompt=WORKLOADS[wid].k + 64, steps=1, layers=1)
        d = decode_cold(w, replicas=r)
        res.append({k: d[k] for k in ("workload", "avg_launch_us", "best_launch_us", "achieved",
                                      "frac", "replicas", "state_swept_MB")})
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
    best = None
    for _ in range(reps):
        c.reset()
        c.prefill(x["q_prompt"], x["k_prompt"], x["v_prompt"])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        us = 1e3 * a.elapsed_time(b) / n
        best = us if best is None else min(best, us)
    del x, c, out, g
    torch.cuda.empty_cache()
    return {"workload": f"{w.name} layer with k = T + n = {kd} (no eviction)",
            "decode_us_per_step": best, "decode_tokens_per_s": w.batch / (best * 1e-6)}


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


def cpu_baseline(w, x, units, min_seconds=10.0):
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import run_unit
    host = {k: v.double().cpu().numpy() for k, v in x.items()}

    def timed(min_s, unit_list):
        # Whole passes over the sampled units until about min_s of CPU work has been timed.
        t0 = time.perf_counter()
        passes = 0
        while True:
            for uidx in unit_list:
                b, h = divmod(uidx, w.heads)
                run_unit(w.k_heavy, w.k_local, host["q_prompt"][b, h], host["k_prompt"][b, h],
                         host["v_prompt"][b, h], host["q_dec"][:, b, h], host["k_dec"][:, b, h],
                         host["v_dec"][:, b, h])
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= min_s or passes >= 50:
                return dt, passes

    def rate(dt, passes, n_units):
        return w.batch * w.steps / (dt / (passes * n_units) * w.units_per_layer)

    dt, passes = timed(min_seconds, units)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    with threadpool_limits(limits=1):           # the same oracle on one core
        few = units[: max(1, len(units) // 8)]
        dt1, passes1 = timed(min_seconds / 2, few)
    return {"value": rate(dt, passes, len(units)), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{passes} pass(es) over {len(units)} of {w.units_per_layer} units (prefill + "
                      f"{w.steps} decode steps each) in {dt:.1f} s, scaled to the whole step",
            "value_1_core": rate(dt1, passes1, len(few)),
            "sample_1_core": f"{passes1} pass(es) over {len(few)} units in {dt1:.1f} s, one BLAS "
                             f"thread, scaled to the whole step"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mfma-probe", action="store_true")
    ap.add_argument("--decode-shapes", action="store_true",
                    help="only time the decode kernel at each workload's layer shape")
    ap.add_argument("--no-decode-shapes", action="store_true")
    ap.add_argument("--decode-cold", action="store_true",
                    help="only time the bench workload's decode kernel with the MALL out of play")
    ap.add_argument("--no-cold", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-stream", action="store_true",
                    help="skip the 2^20-step long-streaming run")
    ap.add_argument("--no-ragged", action="store_true",
                    help="skip the ragged-batch step")
    ap.add_argument("--ragged-only", action="store_true",
                    help="only the ragged-batch step; print its figures")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the 32-layer LLaMA-7B-shaped stack decode")
    ap.add_argument("--stack-only", action="store_true",
                    help="only the 32-layer LLaMA-7B-shaped stack decode; print its figures")
    ap.add_argument("--stream-only", action="store_true",
                    help="only the 2^20-step long-streaming run; print its figures")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 512 MiB device copy (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the H2O path has no cross-GPU exchange and this "
              "build runs on a single MI355X; run with --gpus 1", file=sys.stderr)
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

    if args.decode_shapes:
        for r in decode_by_workload():
            print(json.dumps(r), flush=True)
        for r in decode_by_workload(slot_format="e4m3"):
            print(json.dumps(r), flush=True)
        return
    if args.stream_only:
        print(json.dumps(stream_sustained()), flush=True)
        return
    if args.stack_only:
        print(json.dumps(llama_stack_decode()), flush=True)
        return
    if args.ragged_only:
        print(json.dumps(ragged_step()), flush=True)
        print(json.dumps(decode_by_policy()), flush=True)
        return

    from kv_cache_eviction_03_amd import H2OCache
    from workloads import WORKLOADS, generate

    w = WORKLOADS[2]
    if args.decode_cold:
        print(json.dumps(decode_cold(w)), flush=True)
        for r in decode_cold_by_workload():
            print(json.dumps(r), flush=True)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = generate(w, seed=args.seed, device=dev)
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

    # Eager reference run (also warms up the kernels).
    run_prefill()
    run_decode()
    torch.cuda.synchronize()
    ref_state = {k: v.clone() for k, v in cache.state().items() if torch.is_tensor(v)}
    ref_outs = outs.clone()

    # Capture the whole step as one HIP graph (the timed loop), and each phase as a graph
    # of its own (a second loop, for the phase split and the decode kernel's duration).
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

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        g_step.replay()
    torch.cuda.synchronize()

    # Timed loop: exactly `steps` replays of the whole step.
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        g_step.replay()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps

    # Graph replays must reproduce the eager run bit for bit.
    def check_replay(what):
        for k, v in ref_state.items():
            if not torch.equal(getattr(cache, k), v):
                raise RuntimeError(f"{what} replay diverged from the eager run in {k}")
        if not torch.equal(outs, ref_outs):
            raise RuntimeError(f"{what} replay diverged from the eager run in decode outputs")
    check_replay("step graph")

    # Phase split: the same step as two graphs with events between them.
    for _ in range(args.warmup):
        g_pre.replay()
        g_dec.replay()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e0, e1, e2 in ev:
        e0.record(stream)
        g_pre.replay()
        e1.record(stream)
        g_dec.replay()
        e2.record(stream)
    torch.cuda.synchronize()
    pre_ms = sum(a.elapsed_time(b) for a, b, _ in ev) / args.steps
    dec_ms = sum(b.elapsed_time(c) for _, b, c in ev) / args.steps
    check_replay("phase graph")

    # Decode phase = n back-to-back decode launches inside one graph: its mean per launch is
    # the decode kernel's device duration (inter-node gaps included, so conservative).
    dec_kernel_us = 1e3 * dec_ms / n
    pre_call_us = 1e3 * pre_ms

    dec_bytes = decode_bytes_per_unit(w) * units
    dec_gbs = dec_bytes / (dec_kernel_us * 1e-6) / 1e9
    pre_flops = prefill_flops_per_unit(w) * units
    pre_tflops = pre_flops / (pre_call_us * 1e-6) / 1e12
    pre_gbs = prefill_bytes_per_unit(w) * units / (pre_call_us * 1e-6) / 1e9

    tokens = B * n
    value = tokens / (ms_per_step * 1e-3)
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: batch {B}, {H} heads, head_dim {d}, fp16 K/V, prompt {T} + "
                        f"{n} generated, k = {w.k_heavy} heavy + {w.k_local} local slots",
            "step": f"reset + prefill ({T} tokens) + {n} decode steps, replayed as one HIP graph",
            "value_is": "generated tokens / step time (prefill + decode)",
            "global_batch": B, "seq_len": T + n, "parallelism": "single GPU",
        },
        "decode_tokens_per_s": tokens / (dec_ms * 1e-3),
        "prefill_tokens_per_s": B * T / (pre_ms * 1e-3),
        "phase_ms": {"prefill": pre_ms, "decode": dec_ms},
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_resident_kernel<_Float16,128,256,false,7> (one launch per decode step)",
            "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": dec_gbs / HBM_PEAK_GBS, "traffic": decode_traffic(),
            "avg_launch_us": dec_kernel_us, "algorithmic_bytes_per_launch": dec_bytes,
            "duration_from": "HIP events around the graph-replayed decode phase / launches",
        },
        "roofline_prefill": {
            "bound": "hbm (arithmetic intensity %.1f flop/B < ridge 312.5)" % (
                prefill_flops_per_unit(w) / prefill_bytes_per_unit(w)),
            "achieved_tflops": pre_tflops, "mfma_peak_tflops": MFMA_F16_PEAK_TFLOPS,
            "mfma_frac": pre_tflops / MFMA_F16_PEAK_TFLOPS,
            "achieved_gbs": pre_gbs, "hbm_frac": pre_gbs / HBM_PEAK_GBS,
            "avg_phase_us": pre_call_us,
            "note": "prefill phase = reset + attention-with-column-sums + seed kernels",
        },
        "wall_s_timed_loop": wall,
    }
    floor = launch_floor(w)
    above = dec_kernel_us - floor["h2o_reset_us"]
    floor["decode_us_above_floor"] = above
    floor["decode_GBps_above_floor"] = dec_bytes / (above * 1e-6) / 1e9 if above > 0 else None
    result["launch_floor"] = floor
    if not args.no_mfma_probe:
        result["prefill_mfma_opt30b"] = prefill_mfma_probe()
    if not args.no_decode_shapes:
        result["decode_by_workload"] = decode_by_workload()
        result["decode_by_workload_e4m3"] = decode_by_workload(slot_format="e4m3")
    if not args.no_cold:
        result["hbm_measured_ceiling"] = hbm_ceiling()
        result["roofline_cold"] = decode_cold(w)
        result["roofline_cold"]["kernel"] = "decode_resident_kernel<_Float16,128,256,false,7>, MALL-cold"
        if not args.no_decode_shapes:
            result["decode_cold_by_workload"] = decode_cold_by_workload()
    if not args.no_dense:
        dense = dense_comparator(w)
        dense["h2o_decode_speedup"] = dense["decode_us_per_step"] / dec_kernel_us
        result["dense_comparator"] = dense
    if not args.no_ragged:
        result["ragged_step"] = ragged_step()
        result["decode_by_policy"] = decode_by_policy()
    if not args.no_stack:
        result["llama_stack_decode"] = llama_stack_decode()
    if not args.no_stream:
        result["stream_sustained"] = stream_sustained()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, x, list(range(units)))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
