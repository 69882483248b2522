"""Float64 CPU oracle for the fused linear cross-entropy head.

Test infrastructure only: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product library.
"""
from .flce_oracle import (flce_reference, flce_bruteforce, flce_rows, flce_dw_rows,  # noqa: F401
                          validity,
                          count_valid, scale_factor, loss_only, distill_reference,
                          distill_bruteforce)
