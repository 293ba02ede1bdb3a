"""fp64 CPU oracle for exact attention -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library or its binding.
"""
from .attention import (attention_bwd, attention_fwd, attention_probs,
                        visible_mask, visible_pairs)

__all__ = ["attention_fwd", "attention_bwd", "attention_probs",
           "visible_mask", "visible_pairs"]
