"""A model's worth of H2O caches stepped together, and their steps as HIP graphs.

A decoder stack evicts per layer (each layer decides on its own: "H2O Heavy-Hitter
Oracle 分析", §4), so a model step is one `h2o_decode_step` per layer, in layer
order, on one stream. `H2OStack` owns one `H2OCache` per layer and records those
calls into HIP graphs, so that a whole run of model steps replays with no host work
per launch (the step-fused decode of a deep model).

Positions are host arguments of `h2o_decode_step`, so a captured graph holds the
positions of the steps it covers; a run of n steps is n / G graphs of G model steps
each, captured once and replayed in order. The layers run in turn on one stream, so
they share one workspace.
"""
from __future__ import annotations

import torch

from .cache import H2OCache


class H2OStack:
    """`layers` caches of the same shape (see H2OCache for the other arguments)."""

    def __init__(self, layers: int, batch: int, heads: int, head_dim: int, k_heavy: int,
                 k_local: int, dtype: torch.dtype, device="cuda", max_prompt: int = 0,
                 **cache_kw):
        self.caches = [H2OCache(batch, heads, head_dim, k_heavy, k_local, dtype, device,
                                **cache_kw) for _ in range(layers)]
        self.device = self.caches[0].device
        self.reserve(max_prompt)

    @property
    def layers(self) -> int:
        return len(self.caches)

    def reserve(self, max_prompt: int) -> None:
        """One workspace, sized for the largest need of any layer, shared by all."""
        c0 = self.caches[0]
        c0.reserve(max_prompt)
        for c in self.caches[1:]:
            c.workspace = c0.workspace

    def reset(self) -> None:
        for c in self.caches:
            c.reset()

    def prefill(self, prompts, out: torch.Tensor) -> None:
        """Reset every layer, then run its prompt: prompts[l] = (q, k, v) [B, H, T, d].
        Every layer writes its attention output to `out` ([B, H, T, d] fp32) in turn; the
        column sums stay in the workspace."""
        self.reserve(prompts[0][0].shape[2])
        for c, (q, k, v) in zip(self.caches, prompts):
            c.reset()
            c.prefill(q, k, v, out=out, want_colsum=False)

    def decode_step(self, dec, i: int, outs, aux=None) -> None:
        """Model step i: layer l decodes dec[l] = (q, k, v) [n, B, H, d] row i into outs[l]
        (fp32, [B, H, d], or [n, B, H, d] to keep every step's output at row i); aux[l], if
        given, is (victim_slot, evicted_pos, evicted_acc), each [n, B, H] or None, written
        at row i."""
        for l, (c, (q, k, v)) in enumerate(zip(self.caches, dec)):
            a = (None, None, None) if aux is None or aux[l] is None else aux[l]
            o = outs[l][i] if outs[l].dim() == 4 else outs[l]
            c.decode(q[i], k[i], v[i], out=o,
                     victim_slot=None if a[0] is None else a[0][i],
                     evicted_pos=None if a[1] is None else a[1][i],
                     evicted_acc=None if a[2] is None else a[2][i])

    def capture_prefill(self, prompts, out: torch.Tensor) -> torch.cuda.CUDAGraph:
        """prefill() recorded as one HIP graph (reset and prefill of every layer)."""
        self.reserve(prompts[0][0].shape[2])
        t_after = prompts[0][0].shape[2]
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(self.device)
        torch.cuda.synchronize(self.device)
        with torch.cuda.stream(side), torch.cuda.graph(g, stream=side):
            self.prefill(prompts, out)
        torch.cuda.synchronize(self.device)
        for c in self.caches:
            c.t = t_after
        return g

    def capture_decode(self, dec, t0: int, first: int, count: int, outs,
                       aux=None) -> torch.cuda.CUDAGraph:
        """Model steps first .. first + count - 1 recorded as one HIP graph; step i decodes
        the token at position t0 + i in every layer. Capturing runs nothing: the graph
        must be replayed after the steps before `first` have run. The layers' host
        positions are left as they were."""
        saved = [c.t for c in self.caches]
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(self.device)
        torch.cuda.synchronize(self.device)
        with torch.cuda.stream(side), torch.cuda.graph(g, stream=side):
            for i in range(first, first + count):
                for c in self.caches:
                    c.t = t0 + i
                self.decode_step(dec, i, outs, aux)
        torch.cuda.synchronize(self.device)
        for c, t in zip(self.caches, saved):
            c.t = t
        return g

    def capture_decode_run(self, dec, t0: int, steps: int, per_graph: int, outs,
                           aux=None) -> list:
        """The graphs of model steps 0 .. steps - 1, per_graph steps each (the last may
        hold fewer): replaying them in order runs the whole decode phase."""
        return [self.capture_decode(dec, t0, f, min(per_graph, steps - f), outs, aux)
                for f in range(0, steps, per_graph)]

    def state(self) -> list:
        return [c.state() for c in self.caches]

    def load_state(self, states) -> None:
        for c, st in zip(self.caches, states):
            c.load_state(st)
