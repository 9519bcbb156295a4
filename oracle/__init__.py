"""Float64 CPU oracle for the fused CE + TVD loss.

TEST INFRASTRUCTURE: only the tests, the package smoke check and the benchmark's
CPU-baseline leg may import it.  It shares no code with the HIP path.
"""
from .ce_tvd import (backward, decode, forward, linear_forward_backward, logsumexp_rows, probs_rows,  # noqa: F401
                     reduce_mean)
