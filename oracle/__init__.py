"""CPU float64 oracle for scaled-dot-product attention forward.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are its only callers. It shares no code with the GPU library.
"""
from .attention import (MASK_BOOL, MASK_CAUSAL, MASK_NONE, head_probabilities,
                        probabilities, sdpa, visible_keys)

__all__ = ["sdpa", "probabilities", "head_probabilities", "visible_keys",
           "MASK_NONE", "MASK_CAUSAL", "MASK_BOOL"]
