"""Torch-side owner of one layer's H2O cache: device buffers, the host position
counter t, and calls into the C ABI on torch's current HIP stream.

PyTorch supplies device memory and the stream only; every step of the method
runs in the HIP kernels behind the C ABI.
"""
from __future__ import annotations

import torch

from ._abi import (H2O_BF16, H2O_F16, H2O_F32, POLICY_CODES, SLOT_FORMAT_CODES, CacheDesc,
                   DecodeAux, check,
                   h2o_decode_step,
                   h2o_decode_step_ragged, h2o_prefill, h2o_prefill_ragged, h2o_reset,
                   h2o_workspace_bytes)

_DTYPE_CODE = {torch.float32: H2O_F32, torch.float16: H2O_F16, torch.bfloat16: H2O_BF16}


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(x: torch.Tensor | None) -> int:
    return 0 if x is None else x.data_ptr()


class H2OCache:
    """k = k_heavy + k_local slots per (sequence, head) of one layer; `policy` picks the
    eviction ranking (h2o, sinks, strided, topk), `slot_format` the slot storage ("input":
    the input dtype; "e4m3": FP8 E4M3 codes with scales k_scale / v_scale, held as
    torch.float8_e4m3fn tensors). See include/h2o.h."""

    def __init__(self, batch: int, heads: int, head_dim: int, k_heavy: int, k_local: int,
                 dtype: torch.dtype, device="cuda", max_prompt: int = 0, policy: str = "h2o",
                 policy_param: int = 0, slot_format: str = "input", k_scale: float = 1.0,
                 v_scale: float = 1.0):
        if dtype not in _DTYPE_CODE:
            raise ValueError(f"unsupported dtype {dtype}")
        if policy not in POLICY_CODES:
            raise ValueError(f"unknown policy {policy!r}")
        if slot_format not in SLOT_FORMAT_CODES:
            raise ValueError(f"unknown slot format {slot_format!r}")
        self.policy, self.policy_param = policy, policy_param
        self.slot_format, self.k_scale, self.v_scale = slot_format, k_scale, v_scale
        self.batch, self.heads, self.head_dim = batch, heads, head_dim
        self.k_heavy, self.k_local = k_heavy, k_local
        self.k = k_heavy + k_local
        self.dtype = dtype
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        shape = (batch, heads, self.k, head_dim)
        sdt = torch.float8_e4m3fn if slot_format == "e4m3" else dtype
        self.k_slots = torch.zeros(shape, dtype=sdt, device=self.device)
        self.v_slots = torch.zeros(shape, dtype=sdt, device=self.device)
        self.slot_pos = torch.full((batch, heads, self.k), -1, dtype=torch.int32,
                                   device=self.device)
        self.acc_score = torch.zeros((batch, heads, self.k), dtype=torch.float32,
                                     device=self.device)
        self.t = 0
        self.t_seq = None          # per-sequence device positions, set by prefill_ragged
        self.workspace = torch.empty(0, dtype=torch.uint8, device=self.device)
        self.reserve(max_prompt)

    def desc(self) -> CacheDesc:
        return CacheDesc(self.batch, self.heads, self.head_dim, self.k_heavy, self.k_local,
                         _DTYPE_CODE[self.dtype], self.k_slots.data_ptr(),
                         self.v_slots.data_ptr(), self.slot_pos.data_ptr(),
                         self.acc_score.data_ptr(), POLICY_CODES[self.policy],
                         self.policy_param, SLOT_FORMAT_CODES[self.slot_format], self.k_scale,
                         self.v_scale)

    def reserve(self, max_prompt: int) -> None:
        need = h2o_workspace_bytes(self.desc(), max_prompt)
        if need > self.workspace.numel():
            self.workspace = torch.empty(need, dtype=torch.uint8, device=self.device)

    def _check(self, x: torch.Tensor, shape, name: str) -> None:
        if x.dtype != self.dtype or tuple(x.shape) != tuple(shape) or not x.is_contiguous() \
                or x.device != self.device:
            raise ValueError(f"{name}: expected contiguous {self.dtype} {tuple(shape)} on "
                             f"{self.device}, got {x.dtype} {tuple(x.shape)} on {x.device}")

    def reset(self) -> None:
        check(h2o_reset(self.desc(), _stream(self.device)), "h2o_reset")
        self.t = 0

    def prefill(self, q, k, v, out=None, colsum=None, want_colsum=True):
        """q, k, v: [B, H, T, d]. Returns (out [B, H, T, d] fp32, colsum [B, H, T] or None)."""
        T = q.shape[2]
        shape = (self.batch, self.heads, T, self.head_dim)
        for x, name in ((q, "q"), (k, "k"), (v, "v")):
            self._check(x, shape, name)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        if colsum is None and want_colsum:
            colsum = torch.empty(shape[:3], dtype=torch.float32, device=self.device)
        self.reserve(T)
        check(h2o_prefill(self.desc(), q.data_ptr(), k.data_ptr(), v.data_ptr(), T,
                          out.data_ptr(), _ptr(colsum), self.workspace.data_ptr(),
                          self.workspace.numel(), _stream(self.device)), "h2o_prefill")
        self.t = T
        return out, colsum

    def decode(self, q, k_new, v_new, out=None, victim_slot=None, evicted_pos=None,
               evicted_acc=None):
        """q, k_new, v_new: [B, H, d]. Returns out [B, H, d] fp32; advances t by one."""
        shape = (self.batch, self.heads, self.head_dim)
        for x, name in ((q, "q"), (k_new, "k_new"), (v_new, "v_new")):
            self._check(x, shape, name)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        aux = None
        if victim_slot is not None or evicted_pos is not None or evicted_acc is not None:
            aux = DecodeAux(_ptr(victim_slot), _ptr(evicted_pos), _ptr(evicted_acc))
        ws = self.workspace
        check(h2o_decode_step(self.desc(), self.t, q.data_ptr(), k_new.data_ptr(),
                              v_new.data_ptr(), out.data_ptr(), aux, ws.data_ptr(), ws.numel(),
                              _stream(self.device)), "h2o_decode_step")
        self.t += 1
        return out

    def prefill_ragged(self, q, k, v, lens, out=None, colsum=None):
        """q, k, v: [B, H, T_max, d]; lens: int32 [B] on the device, sequence b's prompt
        length. Returns (out, colsum) as prefill does (rows past lens[b] are not written)
        and sets the per-sequence positions `t_seq` to a copy of lens."""
        T = q.shape[2]
        shape = (self.batch, self.heads, T, self.head_dim)
        for x, name in ((q, "q"), (k, "k"), (v, "v")):
            self._check(x, shape, name)
        if lens.dtype != torch.int32 or tuple(lens.shape) != (self.batch,) \
                or not lens.is_contiguous() or lens.device != self.device:
            raise ValueError(f"lens: expected contiguous int32 ({self.batch},) on {self.device}")
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        if colsum is None:
            colsum = torch.empty(shape[:3], dtype=torch.float32, device=self.device)
        self.reserve(T)
        check(h2o_prefill_ragged(self.desc(), q.data_ptr(), k.data_ptr(), v.data_ptr(), T,
                                 lens.data_ptr(), out.data_ptr(), _ptr(colsum),
                                 self.workspace.data_ptr(), self.workspace.numel(),
                                 _stream(self.device)), "h2o_prefill_ragged")
        self.t_seq = lens.clone()
        return out, colsum

    def decode_ragged(self, q, k_new, v_new, out=None, victim_slot=None, evicted_pos=None,
                      evicted_acc=None, t=None):
        """One token per sequence at its own position t_seq[b] (device int32 [B]); advances
        every t_seq[b] by one. With t (device int32 [B]) given, the positions are taken from
        it instead and t_seq is left alone. Returns out [B, H, d] fp32."""
        shape = (self.batch, self.heads, self.head_dim)
        for x, name in ((q, "q"), (k_new, "k_new"), (v_new, "v_new")):
            self._check(x, shape, name)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        aux = None
        if victim_slot is not None or evicted_pos is not None or evicted_acc is not None:
            aux = DecodeAux(_ptr(victim_slot), _ptr(evicted_pos), _ptr(evicted_acc))
        ws = self.workspace
        tp = self.t_seq if t is None else t
        if tp is None:
            raise ValueError("decode_ragged: no positions (run prefill_ragged or pass t)")
        if tp.dtype != torch.int32 or tuple(tp.shape) != (self.batch,) or not tp.is_contiguous() \
                or tp.device != self.device:
            raise ValueError(f"t: expected contiguous int32 ({self.batch},) on {self.device}")
        check(h2o_decode_step_ragged(self.desc(), tp.data_ptr(), q.data_ptr(),
                                     k_new.data_ptr(), v_new.data_ptr(), out.data_ptr(), aux,
                                     ws.data_ptr(), ws.numel(), _stream(self.device)),
              "h2o_decode_step_ragged")
        if t is None:
            self.t_seq += 1
        return out

    def state(self) -> dict:
        """The whole cache state (for checkpoints): tensors, the host counter t and, after a
        ragged prefill, the per-sequence device positions t_seq."""
        st = {"k_slots": self.k_slots, "v_slots": self.v_slots, "slot_pos": self.slot_pos,
              "acc_score": self.acc_score, "t": self.t}
        if getattr(self, "t_seq", None) is not None:
            st["t_seq"] = self.t_seq
        return st

    def load_state(self, st: dict) -> None:
        for name in ("k_slots", "v_slots", "slot_pos", "acc_score"):
            getattr(self, name).copy_(st[name])
        self.t = int(st["t"])
        if st.get("t_seq") is not None:
            self.t_seq = st["t_seq"].to(device=self.device, dtype=torch.int32).clone()
        else:
            self.t_seq = None
