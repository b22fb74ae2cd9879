"""ctypes binding of libh2o.so: the C ABI declared in include/h2o.h, same names.

Argument marshalling only. Every function takes plain integers for device
pointers and the HIP stream, returns the C status code, and does no compute.
The library must have been built (python -m kv_cache_eviction_03_amd.build);
loading fails loudly otherwise. There is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libh2o.so")

H2O_OK, H2O_ERR_INVALID, H2O_ERR_UNSUPPORTED, H2O_ERR_WORKSPACE, H2O_ERR_HIP = range(5)
H2O_F32, H2O_F16, H2O_BF16 = range(3)
H2O_POLICY_H2O, H2O_POLICY_SINKS, H2O_POLICY_STRIDED, H2O_POLICY_TOPK = range(4)
POLICY_CODES = {"h2o": H2O_POLICY_H2O, "sinks": H2O_POLICY_SINKS,
                "strided": H2O_POLICY_STRIDED, "topk": H2O_POLICY_TOPK}
H2O_SLOTS_INPUT, H2O_SLOTS_FP8_E4M3 = range(2)
SLOT_FORMAT_CODES = {"input": H2O_SLOTS_INPUT, "e4m3": H2O_SLOTS_FP8_E4M3}
H2O_MAX_SLOTS = 8192

H2O_NOALLOC_SCRATCH_BYTES = 8 << 20

EXPORTS = ("h2o_reset", "h2o_workspace_bytes", "h2o_prefill", "h2o_decode_step",
           "h2o_prefill_ragged", "h2o_decode_step_ragged", "h2o_decode_step_noalloc",
           "h2o_status_str", "h2o_last_error")


class CacheDesc(ctypes.Structure):
    """h2o_cache_desc."""
    _fields_ = [("batch", c_int32), ("heads", c_int32), ("head_dim", c_int32),
                ("k_heavy", c_int32), ("k_local", c_int32), ("dtype", c_int32),
                ("k_slots", c_void_p), ("v_slots", c_void_p),
                ("slot_pos", c_void_p), ("acc_score", c_void_p),
                ("policy", c_int32), ("policy_param", c_int32),
                ("slot_format", c_int32), ("k_scale", c_float), ("v_scale", c_float)]


class DecodeAux(ctypes.Structure):
    """h2o_decode_aux."""
    _fields_ = [("victim_slot", c_void_p), ("evicted_pos", c_void_p),
                ("evicted_acc", c_void_p)]


class H2OError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {h2o_status_str(status)}: {h2o_last_error()}")


_lib = None


def library() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m kv_cache_eviction_03_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        lib.h2o_reset.argtypes = [P(CacheDesc), c_void_p]
        lib.h2o_reset.restype = c_int32
        lib.h2o_workspace_bytes.argtypes = [P(CacheDesc), c_int32]
        lib.h2o_workspace_bytes.restype = c_size_t
        lib.h2o_prefill.argtypes = [P(CacheDesc), c_void_p, c_void_p, c_void_p, c_int32,
                                    c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        lib.h2o_prefill.restype = c_int32
        lib.h2o_decode_step.argtypes = [P(CacheDesc), c_int64, c_void_p, c_void_p, c_void_p,
                                        c_void_p, P(DecodeAux), c_void_p, c_size_t, c_void_p]
        lib.h2o_decode_step.restype = c_int32
        lib.h2o_prefill_ragged.argtypes = [P(CacheDesc), c_void_p, c_void_p, c_void_p, c_int32,
                                           c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                           c_void_p]
        lib.h2o_prefill_ragged.restype = c_int32
        lib.h2o_decode_step_ragged.argtypes = [P(CacheDesc), c_void_p, c_void_p, c_void_p,
                                               c_void_p, c_void_p, P(DecodeAux), c_void_p,
                                               c_size_t, c_void_p]
        lib.h2o_decode_step_ragged.restype = c_int32
        lib.h2o_decode_step_noalloc.argtypes = [P(CacheDesc), c_int64, c_void_p, c_void_p,
                                                c_void_p, c_void_p, P(DecodeAux), c_void_p]
        lib.h2o_decode_step_noalloc.restype = c_int32
        lib.h2o_status_str.argtypes = [c_int32]
        lib.h2o_status_str.restype = c_char_p
        lib.h2o_last_error.argtypes = []
        lib.h2o_last_error.restype = c_char_p
        _lib = lib
    return _lib


def h2o_reset(desc: CacheDesc, stream: int) -> int:
    return library().h2o_reset(ctypes.byref(desc), stream)


def h2o_workspace_bytes(desc: CacheDesc, max_prompt: int) -> int:
    return library().h2o_workspace_bytes(ctypes.byref(desc), max_prompt)


def h2o_prefill(desc: CacheDesc, q: int, k: int, v: int, T: int, out: int, colsum_out: int,
                workspace: int, workspace_bytes: int, stream: int) -> int:
    return library().h2o_prefill(ctypes.byref(desc), q, k, v, T, out, colsum_out or None,
                                 workspace or None, workspace_bytes, stream)


def h2o_decode_step(desc: CacheDesc, t: int, q: int, k_new: int, v_new: int, out: int,
                    aux: DecodeAux | None, workspace: int, workspace_bytes: int,
                    stream: int) -> int:
    return library().h2o_decode_step(ctypes.byref(desc), t, q, k_new, v_new, out,
                                     ctypes.byref(aux) if aux is not None else None,
                                     workspace or None, workspace_bytes, stream)


def h2o_prefill_ragged(desc: CacheDesc, q: int, k: int, v: int, T_max: int, lens: int, out: int,
                       colsum_out: int, workspace: int, workspace_bytes: int, stream: int) -> int:
    return library().h2o_prefill_ragged(ctypes.byref(desc), q, k, v, T_max, lens or None, out,
                                        colsum_out or None, workspace or None, workspace_bytes,
                                        stream)


def h2o_decode_step_ragged(desc: CacheDesc, t: int, q: int, k_new: int, v_new: int, out: int,
                           aux: DecodeAux | None, workspace: int, workspace_bytes: int,
                           stream: int) -> int:
    return library().h2o_decode_step_ragged(ctypes.byref(desc), t or None, q, k_new, v_new, out,
                                            ctypes.byref(aux) if aux is not None else None,
                                            workspace or None, workspace_bytes, stream)


def h2o_decode_step_noalloc(desc: CacheDesc, t: int, q: int, k_new: int, v_new: int, out: int,
                            aux: DecodeAux | None, stream: int) -> int:
    return library().h2o_decode_step_noalloc(ctypes.byref(desc), t, q, k_new, v_new, out,
                                             ctypes.byref(aux) if aux is not None else None,
                                             stream)


def h2o_status_str(status: int) -> str:
    return library().h2o_status_str(status).decode()


def h2o_last_error() -> str:
    return library().h2o_last_error().decode()


def check(status: int, where: str) -> None:
    if status != H2O_OK:
        raise H2OError(status, where)
