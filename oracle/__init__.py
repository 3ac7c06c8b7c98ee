"""Float64 CPU oracle for relative-position-bias attention (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this
package; the product path never imports it.
"""
from .relbias_oracle import (MODE_NONE, MODE_TABLE, MODE_RPROJ, attention,
                             attention_backward, bias_matrix, decode, prefill, prefill_backward,
                             temperature, visible_mask)

__all__ = ["MODE_NONE", "MODE_TABLE", "MODE_RPROJ", "attention", "attention_backward",
           "bias_matrix", "decode", "prefill", "prefill_backward", "temperature", "visible_mask"]
