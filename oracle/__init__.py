"""CPU oracle for the H2O hot path. Test infrastructure only; see h2o_oracle."""
from .h2o_oracle import (E4M3_MAX, FREE, POLICIES, SLOT_FORMATS, ParityError, UnitCache,
                         adopt_prefill_kept,
                         causal_softmax, column_sums, decode, e4m3_decode, e4m3_encode,
                         e4m3_round, policy_seed_scores, prefill, quantize_row, run_unit,
                         seed_positions)

__all__ = ["E4M3_MAX", "FREE", "POLICIES", "SLOT_FORMATS", "ParityError", "UnitCache",
           "adopt_prefill_kept",
           "causal_softmax", "column_sums", "decode", "e4m3_decode", "e4m3_encode",
           "e4m3_round", "policy_seed_scores", "prefill", "quantize_row", "run_unit",
           "seed_positions"]
