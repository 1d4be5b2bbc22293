"""fp64 CPU oracle for the attention path.

TEST INFRASTRUCTURE: only tests/, the package smoke check and the benchmark's
CPU-baseline leg may import this.  It shares no code with the HIP library.
"""
from .attention import (attention_backward, attention_backward_rows, attention_forward,
                        attention_rows, visible_mask, visible_pairs)

__all__ = ["attention_forward", "attention_backward", "attention_rows", "attention_backward_rows",
           "visible_mask", "visible_pairs"]
