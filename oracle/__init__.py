"""CPU oracle (test infrastructure only; see lce_oracle)."""
from .lce_oracle import (IGNORE_INDEX, Result, bf16_to_f64, cross_entropy, ring_fold,  # noqa: F401
                         token_rows, weight_rows)
