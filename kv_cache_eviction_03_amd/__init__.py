"""H2O (Heavy-Hitter Oracle) KV-cache eviction hot path for AMD MI355X (gfx950).

The compute lives in libh2o.so (hand-written HIP kernels behind a C ABI, see
include/h2o.h). This package is its Python binding: `_abi` mirrors the C
functions one to one; `H2OCache` owns one layer's device buffers and calls
them on torch's current stream; `H2OStack` steps one cache per layer of a model
together and records runs of model steps as HIP graphs.
"""
from ._abi import (EXPORTS, H2O_BF16, H2O_ERR_HIP, H2O_ERR_INVALID, H2O_ERR_UNSUPPORTED,
                   H2O_ERR_WORKSPACE, H2O_F16, H2O_F32, H2O_MAX_SLOTS, H2O_NOALLOC_SCRATCH_BYTES,
                   H2O_OK, H2O_SLOTS_FP8_E4M3, H2O_SLOTS_INPUT, LIB_PATH,
                   CacheDesc, DecodeAux, H2OError, h2o_decode_step, h2o_decode_step_noalloc,
                   h2o_decode_step_ragged,
                   h2o_last_error, h2o_prefill, h2o_prefill_ragged, h2o_reset, h2o_status_str,
                   h2o_workspace_bytes, library)
from .cache import H2OCache
from .stack import H2OStack

__all__ = ["EXPORTS", "H2O_BF16", "H2O_ERR_HIP", "H2O_ERR_INVALID", "H2O_ERR_UNSUPPORTED",
           "H2O_ERR_WORKSPACE", "H2O_F16", "H2O_F32", "H2O_MAX_SLOTS",
           "H2O_NOALLOC_SCRATCH_BYTES", "H2O_OK",
           "H2O_SLOTS_FP8_E4M3", "H2O_SLOTS_INPUT", "LIB_PATH",
           "CacheDesc", "DecodeAux", "H2OError", "H2OCache", "H2OStack", "h2o_decode_step",
           "h2o_decode_step_noalloc",
           "h2o_decode_step_ragged", "h2o_last_error", "h2o_prefill", "h2o_prefill_ragged",
           "h2o_reset", "h2o_status_str", "h2o_workspace_bytes", "library"]
