"""CPU oracle for the H2O hot path. Test infrastructure only; see h2o_oracle."""
from .h2o_oracle import (FREE, POLICIES, ParityError, UnitCache, causal_softmax, column_sums,
                         decode, policy_seed_scores, prefill, run_unit, seed_positions)

__all__ = ["FREE", "POLICIES", "ParityError", "UnitCache", "causal_softmax", "column_sums",
           "decode", "policy_seed_scores", "prefill", "run_unit", "seed_positions"]
