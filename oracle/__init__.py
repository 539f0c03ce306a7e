"""Plain CPU fp64 oracle for the FlashAttention backward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never calls it, and it never calls the
product path.

Everything here follows the CANN ops-transformer "FlashAttnGrad" article
(page "CANN ops-transformer FlashAttnGrad 算子详解", section 一 "算子功能与数学原理":
the forward formulas S = scale*QK^T, P = exp(S - softmax_lse), Y = PV and the
backward formulas dV, dP, sfmg, dS, dQ, dK), written as the plain definitions
in float64 with NumPy.
"""

from .attention import (  # noqa: F401
    MASK_NONE, MASK_CAUSAL, MASK_WINDOW,
    resolve_scale, mask_bounds, allowed_matrix,
    bf16_round, f16_round, split_heads, merge_heads,
    head_forward, head_backward,
    forward, store, sfmg, backward, backward_rows,
)
