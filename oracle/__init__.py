"""fp64 CPU oracles for the attention path and the fused linear cross-entropy.

TEST INFRASTRUCTURE: only tests/, the package smoke check and the benchmark's
CPU-baseline leg may import this.  It shares no code with the HIP library.
"""
from .attention import (attention_backward, attention_backward_rows, attention_forward,
                        attention_rows, visible_mask, visible_pairs)
from .cross_entropy import lce_backward, lce_forward, lce_rows

__all__ = ["attention_forward", "attention_backward", "attention_rows", "attention_backward_rows",
           "visible_mask", "visible_pairs", "lce_forward", "lce_backward", "lce_rows"]
