"""CPU fp64 oracle for fused linear cross-entropy -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  The GPU library never uses it.
"""
from .flce_oracle import (IGNORE_INDEX, backward, forward, forward_backward, grad_logits,
                          log_sum_exp_rows, logits, reduced_loss, rows_forward_dH)

__all__ = ["IGNORE_INDEX", "backward", "forward", "forward_backward", "grad_logits",
           "log_sum_exp_rows", "logits", "reduced_loss", "rows_forward_dH"]
