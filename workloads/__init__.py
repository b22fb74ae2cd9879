"""Seeded synthetic workloads for the H2O prefill + decode path.

This module holds input generation only: the table of workload shapes and the
seeded random draws that fill them. It contains none of the method's
arithmetic (no attention, no scores, no eviction), so the oracle side and the
HIP side can both consume what it returns without sharing any method code.

Shapes follow the pages' throughput workloads: fixed-length padded prompts with
a fixed number of generated tokens (512+32, 512+1024, 2048+2048) at about a 20%
cache budget, plus a long streaming run (H2O blog, ttsmallhot.github.io, §3.1.3
metrics and §3.2.2 efficiency experiments). No dataset item is used; every value
is a seeded normal draw.

Recipe (all configurations):
  * One torch.Generator on the target device, seeded with
    (seed * 100 + config_id) * 1000 + layer.
  * Draw order: Q for every position, then K, then V, each as fp32 N(0, 1) in
    position-major chunks of shape [chunk, B, H, d], chunk = min(4096,
    2^24 // (B * H * d)) positions.
  * Heavy-hitter keys (configs with heavy_frac > 0): per sequence, a seeded set of
    round(heavy_frac * (T + n)) positions, shared by every head and layer, plus
    positions 0..sinks-1. For each chosen position j of unit (b, h):
    K[j] <- 4 * ||K[j]||_2 * u, where u is the unit vector along the sum of all
    fp32 queries of that unit. This gives a few keys a large, consistent logit,
    the power-law shape the pages describe for accumulated attention (H2O blog
    §2.1.2; the analysis page's §2.1 heavy-hitter phenomenon).
  * Every tensor is then rounded (round-to-nearest-even) to the storage dtype; the
    rounded bits are the canonical inputs for both sides.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    id: int
    name: str
    batch: int
    layers: int
    heads: int
    head_dim: int
    dtype: str
    prompt: int      # T, tokens in the prompt
    steps: int       # n, decode steps
    k_heavy: int
    k_local: int
    heavy_frac: float = 0.0
    sinks: int = 0
    policy: str = "h2o"       # eviction ranking the cache runs with (h2o, sinks, strided, topk)
    policy_param: int = 0
    slot_format: str = "input"   # K/V slot storage: the input dtype, or "e4m3" codes
    k_scale: float = 1.0         # E4M3 scales of K and V
    v_scale: float = 1.0

    @property
    def cache_kw(self) -> dict:
        """Cache options shared by the library's H2OCache and the oracle's UnitCache."""
        return dict(policy=self.policy, policy_param=self.policy_param,
                    slot_format=self.slot_format, k_scale=self.k_scale, v_scale=self.v_scale)

    @property
    def k(self) -> int:
        return self.k_heavy + self.k_local

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    @property
    def units_per_layer(self) -> int:
        return self.batch * self.heads

    @property
    def elem_bytes(self) -> int:
        return torch.empty(0, dtype=self.torch_dtype).element_size()

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "tiny-fp32", batch=1, layers=1, heads=4, head_dim=64, dtype="f32",
                prompt=64, steps=64, k_heavy=16, k_local=16),
    2: Workload(2, "opt-6.7b-layer-fp16", batch=8, layers=1, heads=32, head_dim=128,
                dtype="f16", prompt=512, steps=32, k_heavy=52, k_local=52),
    3: Workload(3, "llama-7b-stack-bf16", batch=64, layers=32, heads=32, head_dim=128,
                dtype="bf16", prompt=512, steps=1024, k_heavy=52, k_local=52,
                heavy_frac=0.05),
    4: Workload(4, "opt-30b-layer-fp16", batch=16, layers=1, heads=56, head_dim=128,
                dtype="f16", prompt=2048, steps=2048, k_heavy=205, k_local=205,
                heavy_frac=0.05, sinks=4),
    5: Workload(5, "stream-bf16", batch=1, layers=1, heads=32, head_dim=128,
                dtype="bf16", prompt=0, steps=1 << 20, k_heavy=2048, k_local=2048,
                heavy_frac=0.02),
}


def generator_seed(w: Workload, seed: int, layer: int) -> int:
    return (seed * 100 + w.id) * 1000 + layer


@torch.no_grad()
def generate(w: Workload, seed: int = 0, layer: int = 0, device="cpu",
             chunk: int | None = None) -> dict:
    """Return the canonical inputs of one layer of workload `w`.

    Keys:
      q_prompt, k_prompt, v_prompt : [B, H, T, d] storage dtype, contiguous
      q_dec, k_dec, v_dec          : [n, B, H, d] storage dtype, contiguous
                                     (row t-T is the token at position t)
    """
    B, H, d, T, n = w.batch, w.heads, w.head_dim, w.prompt, w.steps
    N = T + n
    dt = w.torch_dtype
    if chunk is None:   # about 16M draws per call
        chunk = max(1, min(4096, (1 << 24) // (B * H * d)))
    g = torch.Generator(device=device)
    g.manual_seed(generator_seed(w, seed, layer))

    def draw_all(transform=None):
        full = torch.empty((N, B, H, d), dtype=dt, device=device)
        acc = torch.zeros((B, H, d), dtype=torch.float64, device=device)
        for p0 in range(0, N, chunk):
            p1 = min(N, p0 + chunk)
            x = torch.randn((p1 - p0, B, H, d), generator=g, device=device,
                            dtype=torch.float32)
            if transform is None:
                acc += x.sum(dim=0, dtype=torch.float64)
            else:
                x = transform(x, p0, p1)
            full[p0:p1] = x.to(dt)
        return full, acc

    q_full, q_sum = draw_all()

    transform = None
    sel = heavy_positions(w, seed)
    if bool(sel.any()):
        sel = sel.to(device)
        u = (q_sum / q_sum.norm(dim=-1, keepdim=True)).to(torch.float32)  # [B, H, d]

        def transform(x, p0, p1):
            m = sel[:, p0:p1].transpose(0, 1)            # [c, B]
            norms = x.norm(dim=-1, keepdim=True)         # [c, B, H, 1]
            heavy = 4.0 * norms * u.unsqueeze(0)         # [c, B, H, d]
            return torch.where(m[:, :, None, None], heavy, x)

    k_full, _ = draw_all(transform)
    v_full, _ = draw_all()

    def prompt_part(x):
        return x[:T].permute(1, 2, 0, 3).contiguous()

    return {
        "q_prompt": prompt_part(q_full), "k_prompt": prompt_part(k_full),
        "v_prompt": prompt_part(v_full),
        "q_dec": q_full[T:].contiguous(), "k_dec": k_full[T:].contiguous(),
        "v_dec": v_full[T:].contiguous(),
    }


def heavy_positions(w: Workload, seed: int = 0) -> torch.Tensor:
    """[B, T+n] bool mask of the positions whose keys the recipe makes heavy."""
    N = w.prompt + w.steps
    count = int(round(w.heavy_frac * N))
    gsel = torch.Generator(device="cpu")
    gsel.manual_seed(generator_seed(w, seed, 999))
    sel = torch.zeros((w.batch, N), dtype=torch.bool)
    if count == 0 and w.sinks == 0:
        return sel
    for b in range(w.batch):
        if count > 0:
            sel[b, torch.randperm(N, generator=gsel)[:count]] = True
        sel[b, :min(w.sinks, N)] = True
    return sel


def sample_units(n_units: int, count: int, seed: int = 0) -> list[int]:
    """A seeded sample of unit indices that always holds the first and the last."""
    if count >= n_units:
        return list(range(n_units))
    g = torch.Generator(device="cpu")
    g.manual_seed(12345 + seed)
    mid = torch.randperm(n_units - 2, generator=g)[: max(0, count - 2)] + 1
    return sorted({0, n_units - 1, *mid.tolist()})
